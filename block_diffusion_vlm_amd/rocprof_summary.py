"""Summaries of rocprofv3 result databases (SQLite, the tool's default output).

    python -m block_diffusion_vlm_amd.rocprof_summary trace <results.db> [--by-grid]
        per-kernel dispatch count and average / median / min / max duration
        (us); with --by-grid, one line per kernel and grid size (a kernel
        launched at several shapes, such as the block attention of the
        linear and the fused speculation steps, then gets a line per shape)
    python -m block_diffusion_vlm_amd.rocprof_summary pmc <results.db> <COUNTER>
        per-kernel dispatch count and average counter value per dispatch
    python -m block_diffusion_vlm_amd.rocprof_summary traffic <fetch.db> <write.db> <out.json> [bf16|fp8|attn]
        HBM bytes of one bd_lmhead_conf (bf16, default), bd_lmhead_conf_fp8
        or bd_block_attn (attn) call (the main kernel plus its merge kernel),
        from FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by the
        ratio of known bytes to the counter value of a plain 256 MiB device
        copy recorded in the same run.
    python -m block_diffusion_vlm_amd.rocprof_summary mfma <pmc.db> [<trace.db>]
        per library kernel: the average of every collected counter per
        dispatch; the MFMA pipes' busy fraction (SQ_VALU_MFMA_BUSY_CYCLES over
        SIMDs x median duration x 2.4 GHz, durations from the kernel trace of
        the same command when given) and the profiler's MfmaUtil (busy cycles
        over GRBM_GUI_ACTIVE per instance x SIMDs); the bf16 MFMA flops
        executed (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512); instructions per MFMA;
        the kernel's registers and LDS.
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
SIMD_NUM = 256 * 4          # MI355X: 256 CUs x 4 SIMDs


def _short(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "")
    return re.sub(r"\(.*", "", name).strip()


def kernel_rows(db: str):
    con = sqlite3.connect(db)
    return con.execute("select id, name, start, end, grid_x, grid_y, grid_z from kernels "
                       "order by start").fetchall()


def trace(db: str, by_grid: bool = False) -> str:
    """Per kernel (and grid size, with by_grid): calls, average, median, min
    and max duration, share of the total.  The median is the figure to
    compare with event timings when some dispatches of a kernel return at
    once (the skipped steps of the block loop)."""
    agg = collections.OrderedDict()
    for _, n, s, e, gx, gy, gz in kernel_rows(db):
        key = (_short(n), (gx, gy, gz) if by_grid else None)
        agg.setdefault(key, []).append((e - s) / 1000.0)
    tot = sum(sum(v) for v in agg.values())
    gcol = f" {'grid':>20s}" if by_grid else ""
    out = [f"{'kernel':58s}{gcol} {'calls':>6s} {'avg_us':>8s} {'med_us':>8s} {'min_us':>8s} "
           f"{'max_us':>8s} {'time%':>6s}"]
    for (k, grid), v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        med = sorted(v)[len(v) // 2]
        g = f" {str(grid):>20s}" if by_grid else ""
        out.append(f"{k[:58]:58s}{g} {len(v):6d} {sum(v) / len(v):8.2f} {med:8.2f} "
                   f"{min(v):8.2f} {max(v):8.2f} {100 * sum(v) / tot:6.2f}")
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


# Main kernel of each measured call, the name fragment of its merge kernel,
# and the sources the recorded hash covers.
LMHEAD_KINDS = {
    "bf16": ("void bd::lmhead_bf16_kernel", ("k_lmhead.hip", "lmhead_common.h"), "lmhead_combine"),
    "fp8": ("void bd::lmhead_fp8_kernel", ("k_lmhead_fp8.hip", "lmhead_common.h"),
            "lmhead_combine"),
    "attn": ("void bd::block_attn_split_kernel<false, false>",
             ("k_block_attn.hip", "attn_common.h"), "block_attn_combine"),
}


def source_sha(names) -> str:
    csrc = Path(__file__).resolve().parent / "csrc"
    h = hashlib.sha256()
    for n in names:
        h.update((csrc / n).read_bytes())
    return h.hexdigest()[:16]


def traffic(fetch_db: str, write_db: str, out_json: str, kind: str = "bf16") -> dict:
    prefix, sources, merge_name = LMHEAD_KINDS[kind]
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
        merge = _avg(rows, lambda n, g: merge_name in n)
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


def pmc_table(db: str):
    """{dispatch id: (kernel short name, {counter: value}, info)} of a --pmc
    run; the database view sums each counter over its hardware instances, and
    `info` holds the dispatch's duration in that run (us) and the kernel's
    register and LDS use."""
    con = sqlite3.connect(db)
    rows = con.execute("select dispatch_id, kernel_name, counter_name, value, duration, "
                       "vgpr_count, accum_vgpr_count, sgpr_count, lds_block_size "
                       "from counters_collection").fetchall()
    out = {}
    for did, n, c, v, dur, vg, ag, sg, lds in rows:
        _, cs, _ = out.setdefault(did, (_short(n), {}, {"us": dur / 1000.0, "vgpr": vg,
                                                         "agpr": ag, "sgpr": sg, "lds": lds}))
        cs[c] = cs.get(c, 0.0) + float(v)
    return out


def counter_instances(db: str, counter: str):
    """Hardware instances summed into one dispatch's value of `counter`."""
    con = sqlite3.connect(db)
    try:
        r = con.execute("select count(*) from rocpd_pmc_event E join rocpd_info_pmc I "
                        "on I.id = E.pmc_id and I.guid = E.guid where I.name = ? "
                        "group by E.event_id limit 1", (counter,)).fetchone()
    except sqlite3.Error:
        return None
    return r[0] if r else None


def mfma(pmc_db: str, trace_db: str | None = None, clock_ghz: float = 2.4) -> str:
    """Per library kernel: average counters per dispatch; the MFMA busy
    fraction over the SIMDs at the nominal clock (busy cycles / (SIMDs x
    duration x clock), durations from the trace when given, else from the
    counter run); the profiler's MfmaUtil (busy cycles / (GRBM_GUI_ACTIVE x
    SIMDs), with GRBM_GUI_ACTIVE taken per instance); executed bf16 MFMA
    flops; instructions per MFMA; registers."""
    agg = collections.OrderedDict()
    info = {}
    for _, (n, cs, inf) in sorted(pmc_table(pmc_db).items()):
        agg.setdefault(n, []).append(cs)
        info.setdefault(n, []).append(inf)
    grbm_inst = counter_instances(pmc_db, "GRBM_GUI_ACTIVE") or 1
    dur = {}
    if trace_db:
        for _, n, st, en, *_ in kernel_rows(trace_db):
            dur.setdefault(_short(n), []).append((en - st) / 1000.0)
    lines = [f"GRBM_GUI_ACTIVE instances summed per dispatch: {grbm_inst}"]
    for n, disp in agg.items():
        if not n.startswith("void bd::") and not n.startswith("bd::"):
            continue
        names = sorted({c for d in disp for c in d})
        avg = {c: sum(d.get(c, 0.0) for d in disp) / len(disp) for c in names}
        i0 = info[n][0]
        pmc_us = sorted(x["us"] for x in info[n])[len(info[n]) // 2]
        lines.append(f"{n}  ({len(disp)} dispatches; VGPR {i0['vgpr']}, AGPR {i0['agpr']}, "
                     f"SGPR {i0['sgpr']}, LDS {i0['lds']} B)")
        for c in names:
            lines.append(f"    {c:34s} {avg[c]:18.1f}")
        d = sorted(dur[n])[len(dur[n]) // 2] if n in dur else pmc_us
        lines.append(f"    {'median duration (us), ' + ('trace' if n in dur else 'pmc run'):34s} "
                     f"{d:18.2f}")
        busy, act = avg.get("SQ_VALU_MFMA_BUSY_CYCLES"), avg.get("GRBM_GUI_ACTIVE")
        if busy is not None:
            frac = busy / (SIMD_NUM * d * 1e-6 * clock_ghz * 1e9)
            label = f"MFMA busy % at {clock_ghz:.1f} GHz"
            lines.append(f"    {label:34s} {100.0 * frac:18.2f}")
            if act:
                lines.append(f"    {'MfmaUtil % (per GRBM instance)':34s} "
                             f"{100.0 * busy / (act / grbm_inst * SIMD_NUM):18.2f}")
        mops = avg.get("SQ_INSTS_VALU_MFMA_MOPS_BF16")
        if mops:
            lines.append(f"    {'bf16 MFMA GFLOP executed':34s} {mops * 512 / 1e9:18.3f}")
        if avg.get("SQ_INSTS_MFMA"):
            for c in ("SQ_INSTS_VALU", "SQ_INSTS_LDS"):
                if c in avg:
                    lines.append(f"    {c + ' per MFMA':34s} {avg[c] / avg['SQ_INSTS_MFMA']:18.3f}")
    return "\n".join(lines)


def main(argv):
    if len(argv) >= 2 and argv[0] == "trace":
        print(trace(argv[1], by_grid="--by-grid" in argv[2:]))
    elif len(argv) >= 3 and argv[0] == "pmc":
        print(pmc(argv[1], argv[2]))
    elif len(argv) >= 2 and argv[0] == "mfma":
        print(mfma(argv[1], argv[2] if len(argv) >= 3 else None))
    elif len(argv) >= 4 and argv[0] == "traffic":
        kind = argv[4] if len(argv) >= 5 else "bf16"
        print(json.dumps(traffic(argv[1], argv[2], argv[3], kind), indent=1))
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
