"""Summaries of rocprofv3 results for the library's kernels.

    python -m paged_kv_cache_block_amd.profiling trace <results.db>
        per-kernel calls and durations (kernel-trace run), as a Markdown table
    python -m paged_kv_cache_block_amd.profiling pmc <results.db> [name-filter]
        per-kernel mean of each collected counter (--pmc run)
    python -m paged_kv_cache_block_amd.profiling traffic --kernel K --config C \\
            --fetch <db> --write <db> --copy-fetch <db> --copy-write <db>
        HBM bytes per launch of kernel K: FETCH_SIZE and WRITE_SIZE (KiB per
        dispatch) scaled by what the same counters read for pa_copy_blocks
        copying a known byte count (bench.py --copy-calibration).  Prints a
        one-line traffic record for a profiles/*.md file.

    python -m paged_kv_cache_block_amd.profiling mfma --kernel K --config C <db>
        MFMA-busy fraction of kernel K from one --pmc run of
        SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE: the busy cycles summed
        over the chip's SIMDs, over SIMDs x the launch's cycles per XCD.
        Prints a one-line mfma record for a profiles/*.md file.

``traffic_record_for`` / ``counter_record_for`` let bench.py pick a record
back up; a record only applies while the kernel's sources hash to the value
stored in it.
"""
from __future__ import annotations

import argparse
import collections
import glob
import hashlib
import json
import os
import re
import sqlite3

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
KERNEL_SOURCES = {
    # The planner's order of work items shapes the attention kernels' traffic.
    "decode_mfma_kernel": ["csrc/pa_decode.hip", "csrc/pa_plan.hip"],
    "tile_attn_kernel": ["csrc/pa_tile.hip", "csrc/pa_plan.hip"],
    "row_attn_kernel": ["csrc/pa_rows.hip"],
    "combine_kernel": ["csrc/pa_rows.hip"],
    "write_kv_kernel": ["csrc/pa_kv.hip"],
    "copy_blocks_kernel": ["csrc/pa_kv.hip"],
}
# build.py holds the compile flags (per source, too).
COMMON_SOURCES = ["csrc/pa_device.h", "csrc/pa_internal.h", "build.py"]
COPY_CAL_BYTES = 2 * 4096 * 40 * 16 * 128 * 2      # bench.py --copy-calibration, each way


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel] + COMMON_SOURCES:
        with open(os.path.join(PKG, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _short(name: str) -> str:
    n = re.sub(r"pa::\(anonymous namespace\)::", "", name)
    n = re.sub(r"\(pa::AttnArgs.*|\(HIP_vector_type.*|\(int const\*.*|\(pa::.*|\(uint4.*", "", n)
    return n[:72]


def trace_table(db: str) -> str:
    con = sqlite3.connect(db)
    rows = con.execute(
        "select name, count(*), sum(duration), avg(duration), min(duration), max(duration), "
        "max(grid_x), max(grid_y), max(grid_z), max(workgroup_x), max(vgpr_count), "
        "max(accum_vgpr_count), max(lds_size) from kernels group by name "
        "order by sum(duration) desc").fetchall()
    out = ["| kernel | calls | total us | avg us | min us | max us | grid (x,y,z) | wg | vgpr | agpr | lds B |",
           "|---|---|---|---|---|---|---|---|---|---|---|"]
    for n, c, tot, avg, mn, mx, gx, gy, gz, wx, vg, ag, lds in rows:
        out.append(f"| `{_short(n)}` | {c} | {tot / 1e3:.1f} | {avg / 1e3:.2f} | {mn / 1e3:.2f} | "
                   f"{mx / 1e3:.2f} | {gx},{gy},{gz} | {wx} | {vg} | {ag} | {lds} |")
    return "\n".join(out)


def pmc_means(db: str, name_filter: str = "") -> dict:
    """{kernel: {counter: mean over dispatches of the per-dispatch sum}}"""
    con = sqlite3.connect(db)
    rows = con.execute(
        "select name, dispatch_id, counter_name, sum(counter_value) from pmc_events "
        "group by dispatch_id, counter_name").fetchall()
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for name, _, cname, val in rows:
        n = _short(name)
        if name_filter and name_filter not in n:
            continue
        agg[n][cname].append(val)
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in agg.items()}


def _one(db: str, kernel: str, counter: str) -> float:
    vals = [cs[counter] for k, cs in pmc_means(db, kernel).items() if counter in cs]
    if not vals:
        raise SystemExit(f"no {counter} for {kernel} in {db}")
    return vals[0]


def traffic_record(kernel: str, config: int, fetch_db: str, write_db: str, copy_fetch_db: str,
                   copy_write_db: str) -> dict:
    fscale = COPY_CAL_BYTES / (_one(copy_fetch_db, "copy_blocks_kernel", "FETCH_SIZE") * 1024)
    wscale = COPY_CAL_BYTES / (_one(copy_write_db, "copy_blocks_kernel", "WRITE_SIZE") * 1024)
    fetch = _one(fetch_db, kernel, "FETCH_SIZE") * 1024 * fscale
    write = _one(write_db, kernel, "WRITE_SIZE") * 1024 * wscale
    return {"kernel": kernel, "config": config, "source_sha256": kernel_source_hash(kernel),
            "fetch_bytes": int(fetch), "write_bytes": int(write),
            "fetch_scale": round(fscale, 4), "write_scale": round(wscale, 4)}


# MI355X: 256 compute units of 4 SIMDs, in 8 XCDs.
NUM_SIMDS = 1024
NUM_XCDS = 8


def mfma_record(kernel: str, config: int, db: str) -> dict:
    busy = _one(db, kernel, "SQ_VALU_MFMA_BUSY_CYCLES")
    gui = _one(db, kernel, "GRBM_GUI_ACTIVE")
    cycles = gui / NUM_XCDS
    return {"kernel": kernel, "config": config, "source_sha256": kernel_source_hash(kernel),
            "mfma_busy_frac": round(busy / (NUM_SIMDS * cycles), 4),
            "mfma_busy_cycles": int(busy), "launch_cycles_per_xcd": int(cycles)}


def counter_record_for(tag: str, kernel: str, config: int):
    """The stored ``tag`` record for (kernel, config) if the kernel is
    unchanged since it was taken."""
    want = kernel_source_hash(kernel)
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as f:
            for line in f:
                if line.startswith(tag + ":"):
                    rec = json.loads(line.split(":", 1)[1])
                    if rec.get("kernel") == kernel and rec.get("config") == config \
                            and rec.get("source_sha256") == want:
                        return rec
    return None


def traffic_record_for(kernel: str, config: int):
    """The stored traffic record for (kernel, config) if the kernel is unchanged since."""
    return counter_record_for("traffic-record", kernel, config)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    p = sub.add_parser("pmc")
    p.add_argument("db")
    p.add_argument("filter", nargs="?", default="")
    r = sub.add_parser("traffic")
    r.add_argument("--kernel", required=True)
    r.add_argument("--config", type=int, required=True)
    for k in ("fetch", "write", "copy-fetch", "copy-write"):
        r.add_argument("--" + k, required=True)
    m = sub.add_parser("mfma")
    m.add_argument("--kernel", required=True)
    m.add_argument("--config", type=int, required=True)
    m.add_argument("db")
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        print(trace_table(a.db))
    elif a.cmd == "pmc":
        for k, cs in pmc_means(a.db, a.filter).items():
            print(k)
            for c, v in sorted(cs.items()):
                print(f"    {c:34s} {v:.6g}")
    elif a.cmd == "mfma":
        print("mfma-record: " + json.dumps(mfma_record(a.kernel, a.config, a.db)))
    else:
        rec = traffic_record(a.kernel, a.config, a.fetch, a.write, a.copy_fetch, a.copy_write)
        print("traffic-record: " + json.dumps(rec))
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
