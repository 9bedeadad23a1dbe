"""Summaries of rocprofv3 output (its SQLite results database) as short text.

    python -m token_activation_perturbation_amd.profiling trace <results.db> <title> <command>
    python -m token_activation_perturbation_amd.profiling pmc <fetch.db> <write.db> <kernel> <copy_bytes>
    python -m token_activation_perturbation_amd.profiling counters <results.db> <title> <command>

`trace` prints a markdown table of per-kernel calls and durations from a
`--kernel-trace --stats` run.  `pmc` turns two counter runs (FETCH_SIZE,
then WRITE_SIZE, in KiB per dispatch) into HBM bytes per launch of `kernel`,
scaled by what the same counters read for the largest plain copy kernel in
the run (whose true traffic is copy_bytes read + copy_bytes written).
`counters` turns one SQ counter run into per-kernel unit utilisation on the
MI355X (1024 SIMDs in 8 XCDs, GRBM_GUI_ACTIVE counted per XCD):
  * VALU issue = issue slots / (2 x quad-cycles x 1024): a SIMD issues up to
    two single-pass VALU instructions per quad-cycle (128 lanes per CU per
    clock, the fp32 vector peak), and the slots weight every issued VALU
    instruction by its rate class as the ALU cost model does: 1 for a
    single-pass instruction, 2 for a 64-bit integer or conversion
    instruction (SQ_INSTS_VALU_INT64, SQ_INSTS_VALU_CVT: half rate), 4 for
    a transcendental (SQ_INSTS_VALU_TRANS_F32: quarter rate); quad-cycles
    = the kernel's GPU-busy clock (GRBM_GUI_ACTIVE averaged over the XCDs)
    / 4.  It is a fraction of the issue capacity, at most 1;
  * MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / 1024 / GPU-busy cycles;
  * VALU and MFMA instructions per wave, and the transcendental, 64-bit
    integer and conversion instructions per wave.
"""
from __future__ import annotations

import json
import re
import sqlite3
import sys


def short_name(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    depth, out = 0, []
    for ch in name:  # drop the argument list, keep template arguments
        if ch == "(" and depth == 0:
            break
        depth += ch == "<"
        depth -= ch == ">"
        out.append(ch)
    s = "".join(out)
    return s if len(s) < 90 else s[:87] + "..."


def trace_rows(db: str):
    con = sqlite3.connect(db)
    return list(con.execute(
        "select name, total_calls, total_duration, average, percentage from top_kernels"))


def trace_markdown(db: str, title: str, command: str) -> str:
    lines = [f"# {title}", "", "Command (repository root, on an MI355X):", "", "```", command,
             "```", "", "| kernel | calls | total us | avg us | % |", "|---|---|---|---|---|"]
    for name, calls, tot, avg, pct in trace_rows(db):
        lines.append(f"| `{short_name(name)}` | {calls} | {tot:.1f} | {avg:.2f} | {pct:.1f} |")
    return "\n".join(lines) + "\n"


def _pmc_per_dispatch(db: str, counter: str):
    """{kernel name: [value per dispatch]} for one counter."""
    con = sqlite3.connect(db)
    cols = [r[1] for r in con.execute("pragma table_info(counters_collection)")]
    name_col = "kernel_name" if "kernel_name" in cols else "name"
    value_col = "value" if "value" in cols else "counter_value"
    cname_col = "counter_name" if "counter_name" in cols else "counter"
    out = {}
    q = (f"select {name_col}, dispatch_id, sum({value_col}) from counters_collection "
         f"where {cname_col} = ? group by dispatch_id")
    for name, _did, val in con.execute(q, (counter,)):
        out.setdefault(name, []).append(float(val))
    return out


def pmc_traffic(fetch_db: str, write_db: str, kernel: str, copy_bytes: int) -> dict:
    fetch = _pmc_per_dispatch(fetch_db, "FETCH_SIZE")
    write = _pmc_per_dispatch(write_db, "WRITE_SIZE")

    def pick(d, pattern):
        keys = [k for k in d if re.search(pattern, k)]
        if not keys:
            raise KeyError(pattern)
        return keys[0]

    def largest_copy(d):
        # the copy dispatch with the most traffic is the calibration copy
        vals = [v for k, vs in d.items() if re.search(r"copy|Copy", k) for v in vs]
        if not vals:
            raise KeyError("no copy kernel in the counter run")
        return max(vals)

    copy_f = largest_copy(fetch)
    copy_w = largest_copy(write)
    f_scale = copy_bytes / (copy_f * 1024.0)
    w_scale = copy_bytes / (copy_w * 1024.0)
    kf = pick(fetch, re.escape(kernel))
    kw = pick(write, re.escape(kernel))
    fetch_kib = sum(fetch[kf]) / len(fetch[kf])
    write_kib = sum(write[kw]) / len(write[kw])
    return {"kernel": kernel, "fetch_kib_per_dispatch": fetch_kib,
            "write_kib_per_dispatch": write_kib, "copy_fetch_kib": copy_f,
            "copy_write_kib": copy_w, "fetch_scale": f_scale, "write_scale": w_scale,
            "bytes_per_launch": fetch_kib * 1024.0 * f_scale + write_kib * 1024.0 * w_scale}


N_SIMD = 1024
N_XCD = 8


def counter_table(db: str, title: str, command: str) -> str:
    con = sqlite3.connect(db)
    rows = con.execute("select kernel_name, dispatch_id, counter_name, value "
                       "from counters_collection").fetchall()
    acc, disp = {}, {}
    for name, did, cname, val in rows:
        if "dust" not in name:
            continue
        k = short_name(name)
        acc.setdefault(k, {}).setdefault(cname, 0.0)
        acc[k][cname] += float(val)
        disp.setdefault(k, set()).add(did)
    lines = [f"# {title}", "", "Command (repository root, on an MI355X):", "", "```", command,
             "```", "",
             "VALU issue = (SQ_INSTS_VALU + 3 SQ_INSTS_VALU_TRANS_F32 + SQ_INSTS_VALU_INT64 + "
             "SQ_INSTS_VALU_CVT) / (2 x GRBM_GUI_ACTIVE / 8 / 4 x 1024): issue slots weighted by "
             "rate class (single-pass 1, 64-bit integer and conversion 2, transcendental 4) over "
             "the SIMDs' capacity of two single-pass instructions per quad-cycle; at most 1.  "
             "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / 1024 / (GRBM_GUI_ACTIVE / 8).", "",
             "| kernel | dispatches | VALU issue | MFMA busy | VALU insts / wave | "
             "MFMA insts / wave | transcendental / wave | 64-bit int / wave | conversion / wave |",
             "|---|---|---|---|---|---|---|---|---|"]
    for k, c in acc.items():
        n = len(disp[k])
        gui = c.get("GRBM_GUI_ACTIVE", 0.0) / n / N_XCD
        waves = c.get("SQ_WAVES", 0.0) / n
        slots = (c.get("SQ_INSTS_VALU", 0.0) + 3 * c.get("SQ_INSTS_VALU_TRANS_F32", 0.0)
                 + c.get("SQ_INSTS_VALU_INT64", 0.0) + c.get("SQ_INSTS_VALU_CVT", 0.0)) / n
        valu = slots / (2.0 * gui / 4.0 * N_SIMD) if gui else float("nan")
        mfma = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / n / N_SIMD / gui if gui else float("nan")
        per = lambda name: c.get(name, 0.0) / n / waves if waves else float("nan")  # noqa: E731
        lines.append(f"| `{k}` | {n} | {valu:.2f} | {mfma:.2f} | {per('SQ_INSTS_VALU'):.0f} | "
                     f"{per('SQ_INSTS_MFMA'):.0f} | {per('SQ_INSTS_VALU_TRANS_F32'):.0f} | "
                     f"{per('SQ_INSTS_VALU_INT64'):.0f} | {per('SQ_INSTS_VALU_CVT'):.0f} |")
    return "\n".join(lines) + "\n"


if __name__ == "__main__":
    if len(sys.argv) >= 5 and sys.argv[1] == "trace":
        print(trace_markdown(sys.argv[2], sys.argv[3], sys.argv[4]), end="")
    elif len(sys.argv) >= 5 and sys.argv[1] == "counters":
        print(counter_table(sys.argv[2], sys.argv[3], sys.argv[4]), end="")
    elif len(sys.argv) >= 6 and sys.argv[1] == "pmc":
        print(json.dumps(pmc_traffic(sys.argv[2], sys.argv[3], sys.argv[4], int(sys.argv[5])),
                         indent=1))
    else:
        sys.exit(__doc__)
