"""Summaries of rocprofv3 result databases (SQLite, the tool's default output).

    python -m block_diffusion_vlm_amd.rocprof_summary trace <results.db>
        per-kernel dispatch count and average / min / max duration (us)
    python -m block_diffusion_vlm_amd.rocprof_summary pmc <results.db> <COUNTER>
        per-kernel dispatch count and average counter value per dispatch
    python -m block_diffusion_vlm_amd.rocprof_summary traffic <fetch.db> <write.db> <out.json> [bf16|fp8]
        HBM bytes of one bd_lmhead_conf (bf16, default) or bd_lmhead_conf_fp8
        call (the streaming kernel plus its merge kernel), from FETCH_SIZE and
        WRITE_SIZE (KiB per dispatch), each scaled by the ratio of known bytes
        to the counter value of a plain 256 MiB device copy recorded in the
        same run.
"""
from __future__ import annotations

import collections
import hashlib
import json
import re
import sqlite3
import sys
from pathlib import Path

COPY_BYTES = 256 * 2 ** 20


def _short(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "")
    return re.sub(r"\(.*", "", name).strip()


def kernel_rows(db: str):
    con = sqlite3.connect(db)
    return con.execute("select id, name, start, end, grid_x, grid_y, grid_z from kernels "
                       "order by start").fetchall()


def trace(db: str) -> str:
    """Per kernel: calls, average, median, min and max duration, share of the
    total.  The median is the figure to compare with event timings when some
    dispatches of a kernel return at once (the skipped steps of the block
    loop)."""
    agg = collections.OrderedDict()
    for _, n, s, e, *_ in kernel_rows(db):
        agg.setdefault(_short(n), []).append((e - s) / 1000.0)
    tot = sum(sum(v) for v in agg.values())
    out = [f"{'kernel':58s} {'calls':>6s} {'avg_us':>8s} {'med_us':>8s} {'min_us':>8s} "
           f"{'max_us':>8s} {'time%':>6s}"]
    for k, v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        med = sorted(v)[len(v) // 2]
        out.append(f"{k[:58]:58s} {len(v):6d} {sum(v) / len(v):8.2f} {med:8.2f} {min(v):8.2f} "
                   f"{max(v):8.2f} {100 * sum(v) / tot:6.2f}")
    return "\n".join(out)


def pmc_per_dispatch(db: str, counter: str):
    """[(kernel short name, grid, counter value)] for every dispatch."""
    con = sqlite3.connect(db)
    rows = con.execute(
        "select kernel_name, grid_size_x, grid_size_y, grid_size_z, value "
        "from counters_collection where counter_name = ? order by dispatch_id",
        (counter,)).fetchall()
    return [(_short(n), (gx, gy, gz), float(v)) for n, gx, gy, gz, v in rows]


def pmc(db: str, counter: str) -> str:
    agg = collections.OrderedDict()
    for n, grid, v in pmc_per_dispatch(db, counter):
        agg.setdefault((n, grid), []).append(v)
    out = [f"{'kernel':64s} {'grid':>18s} {'calls':>6s} {'avg ' + counter:>16s}"]
    for (n, grid), v in agg.items():
        out.append(f"{n[:64]:64s} {str(grid):>18s} {len(v):6d} {sum(v) / len(v):16.1f}")
    return "\n".join(out)


def _avg(rows, pred):
    vals = [v for n, g, v in rows if pred(n, g)]
    return (sum(vals) / len(vals)) if vals else None


# Streaming kernel of each LM-head flavour and the sources its hash covers.
LMHEAD_KINDS = {
    "bf16": ("void bd::lmhead_bf16_kernel", ("k_lmhead.hip", "lmhead_common.h")),
    "fp8": ("void bd::lmhead_fp8_kernel", ("k_lmhead_fp8.hip", "lmhead_common.h")),
}


def source_sha(names) -> str:
    csrc = Path(__file__).resolve().parent / "csrc"
    h = hashlib.sha256()
    for n in names:
        h.update((csrc / n).read_bytes())
    return h.hexdigest()[:16]


def traffic(fetch_db: str, write_db: str, out_json: str, kind: str = "bf16") -> dict:
    prefix, sources = LMHEAD_KINDS[kind]
    res = {}
    for kind, db, cname in (("fetch", fetch_db, "FETCH_SIZE"), ("write", write_db, "WRITE_SIZE")):
        rows = pmc_per_dispatch(db, cname)
        # the calibration copy: the benchmark's 256 MiB device-to-device copies,
        # picked out among the copy dispatches by a counter value above a
        # quarter of 256 MiB (the small state-restore copies move a few bytes;
        # FETCH_SIZE reads about half the true bytes for this copy, which is
        # exactly what the scale corrects)
        kib = COPY_BYTES / 1024.0
        vals = [v for n, g, v in rows if "copy" in n.lower() and 0.25 * kib <= v <= 1.5 * kib]
        copy = sum(vals) / len(vals) if vals else None
        lm = _avg(rows, lambda n, g: n.startswith(prefix))
        merge = _avg(rows, lambda n, g: "lmhead_combine" in n)
        if copy is None or lm is None:
            raise SystemExit(f"{cname}: calibration copy or LM-head dispatches not found")
        scale = COPY_BYTES / (copy * 1024.0)        # counter is in KiB
        res[kind] = {"counter": cname, "copy_kib": copy, "scale": scale, "lmhead_kib": lm,
                     "merge_kib": merge or 0.0,
                     "bytes_per_call": (lm + (merge or 0.0)) * 1024.0 * scale}
    res["hbm_bytes_per_call"] = res["fetch"]["bytes_per_call"] + res["write"]["bytes_per_call"]
    res["kernel_source_sha"] = source_sha(sources)
    Path(out_json).write_text(json.dumps(res, indent=1) + "\n")
    return res


def main(argv):
    if len(argv) >= 2 and argv[0] == "trace":
        print(trace(argv[1]))
    elif len(argv) >= 3 and argv[0] == "pmc":
        print(pmc(argv[1], argv[2]))
    elif len(argv) >= 4 and argv[0] == "traffic":
        kind = argv[4] if len(argv) >= 5 else "bf16"
        print(json.dumps(traffic(argv[1], argv[2], argv[3], kind), indent=1))
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
