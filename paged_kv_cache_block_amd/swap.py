"""Layer-by-layer swap-in that gates each layer's attention on its own event.

Pensieve page (流水线KV缓存恢复): the worker does not wait for all of a
batch's swapped-out K/V to return before computing; it starts the transfer of
every layer at once and launches a layer's attention as soon as that layer's
K/V are on the GPU, tracked with GPU events.  (实现细节与优化): copies in the
two directions slow each other down, so swap-outs wait until the swap-ins in
flight are done.

Here the swap-ins of all layers are enqueued in layer order on one copy
stream (default priority), each followed by an event; the compute stream
waits on event l right before layer l's attention.  Swap-outs go on a second
copy stream by default: on MI355X, 128 MB each way took 2.8-3.6 ms
concurrently and 4.7 ms one direction after the other (bench.py --swap), the
opposite of the page's observation on its platform.  ``ordered_out=True`` puts them
behind the swap-ins on the first stream instead, the page's policy.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import torch

from . import binding


@dataclass
class LayerSwap:
    """One layer's pools and the blocks to move (int32 CPU [n][2] pairs)."""
    dev_k: torch.Tensor
    dev_v: torch.Tensor
    host_k: torch.Tensor
    host_v: torch.Tensor
    pairs: torch.Tensor


class LayerSwapPipeline:
    def __init__(self, copy_stream: Optional[torch.cuda.Stream] = None, ordered_out: bool = False):
        self.copy_stream = copy_stream if copy_stream is not None else torch.cuda.Stream()
        self.out_stream = self.copy_stream if ordered_out else torch.cuda.Stream()
        self.events: List[torch.cuda.Event] = []

    def start_swap_in(self, layers: List[LayerSwap]) -> List[torch.cuda.Event]:
        """Enqueue every layer's swap-in; returns one event per layer."""
        # The copy stream must not start before the compute stream's earlier
        # work that produced or freed these blocks.
        self.copy_stream.wait_stream(torch.cuda.current_stream())
        self.events = []
        for ls in layers:
            if ls.pairs.numel():
                binding.pa_swap_blocks(ls.dev_k, ls.dev_v, ls.host_k, ls.host_v, ls.pairs,
                                       binding.PA_SWAP_IN, stream=self.copy_stream)
            ev = torch.cuda.Event()
            ev.record(self.copy_stream)
            self.events.append(ev)
        return self.events

    def wait_layer(self, layer: int, stream: Optional[torch.cuda.Stream] = None) -> None:
        """Make `stream` (default: the current stream) wait for layer's swap-in."""
        (stream if stream is not None else torch.cuda.current_stream()).wait_event(self.events[layer])

    def swap_out(self, layers: List[LayerSwap]) -> torch.cuda.Event:
        """Enqueue swap-outs on the out stream; the blocks are read once the
        compute stream's work so far is done.  Returns the completion event."""
        self.out_stream.wait_stream(torch.cuda.current_stream())
        for ls in layers:
            if ls.pairs.numel():
                binding.pa_swap_blocks(ls.dev_k, ls.dev_v, ls.host_k, ls.host_v, ls.pairs,
                                       binding.PA_SWAP_OUT, stream=self.out_stream)
        ev = torch.cuda.Event()
        ev.record(self.out_stream)
        return ev
