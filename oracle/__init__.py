"""CPU oracle for paged KV-cache attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library does not import it and
shares no code with it.
"""
from .pa_oracle import (DTYPES, attention, attention_seq, combine_partials,  # noqa: F401
                        copy_blocks, gather_context, partial_state, swap_blocks, to_f64,
                        write_kv)
