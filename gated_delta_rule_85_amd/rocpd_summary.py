"""Summaries of rocprofv3 result databases (rocpd SQLite) for this library.

    python -m gated_delta_rule_85_amd.rocpd_summary trace RUN_results.db
        per-kernel dispatch count and duration (from --kernel-trace --stats)

    python -m gated_delta_rule_85_amd.rocpd_summary mfma RUN_results.db [SIMDS] [XCDS]
        per-kernel matrix-core counters from one --pmc run of SQ_VALU_MFMA_BUSY_CYCLES,
        SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_INSTS_VALU_MFMA_MOPS_F32 and GRBM_GUI_ACTIVE:
        matrix-core FLOPs (MOPS x 512), and utilisation = busy cycles summed over
        the SIMDs / (active cycles of one XCD x SIMDS); GRBM_GUI_ACTIVE arrives
        summed over the XCDS accelerator dies (default 1024 SIMDs, 8 XCDs)

    python -m gated_delta_rule_85_amd.rocpd_summary pmc FETCH.db WRITE.db [COPY_BYTES]
        mean FETCH_SIZE / WRITE_SIZE per dispatch (KiB) from two --pmc runs,
        and bytes per dispatch after calibration against the plain device copy
        of COPY_BYTES bytes found in the same runs (the largest copy dispatch;
        its counters divided by its known size give the factor that turns a
        counter into bytes)
"""
from __future__ import annotations

import collections
import sqlite3
import sys

PREFIX = "_ZN3gdr12_GLOBAL__N_1"


def _short(name: str, width: int = 70) -> str:
    return name.replace(PREFIX, "")[:width]


def trace(db: str) -> str:
    con = sqlite3.connect(db)
    rows = con.execute(
        "select name, count(*), avg(duration), sum(duration), min(duration), max(duration) "
        "from kernels group by name order by sum(duration) desc").fetchall()
    total = sum(r[3] for r in rows) or 1
    out = ["| kernel | calls | avg us | min us | max us | total us | % |",
           "|---|---:|---:|---:|---:|---:|---:|"]
    for n, c, avg, tot, mn, mx in rows:
        out.append(f"| `{_short(n)}` | {c} | {avg / 1e3:.2f} | {mn / 1e3:.2f} | {mx / 1e3:.2f} | "
                   f"{tot / 1e3:.1f} | {100 * tot / total:.1f} |")
    return "\n".join(out)


def _pmc(db: str):
    con = sqlite3.connect(db)
    agg = collections.defaultdict(list)
    for name, counter, value in con.execute(
            "select kernel_name, counter_name, value from counters_collection"):
        agg[(name, counter)].append(value)
    return {k: sum(v) / len(v) for k, v in agg.items()}, {k: len(v) for k, v in agg.items()}


def _max_copy(db: str, counter: str):
    """The counter of the largest plain device copy in the run: the calibration
    copy (other, smaller copies may run too)."""
    con = sqlite3.connect(db)
    vals = [v for (v,) in con.execute(
        "select value from counters_collection where counter_name = ? and kernel_name like "
        "'%copyBuffer%'", (counter,))]
    return max(vals) if vals else None


def pmc(fetch_db: str, write_db: str, copy_bytes: int = 1 << 28) -> str:
    f, fn = _pmc(fetch_db)
    w, _ = _pmc(write_db)
    fr = wr = None
    cf, cw = _max_copy(fetch_db, "FETCH_SIZE"), _max_copy(write_db, "WRITE_SIZE")
    if cf and cw:
        fr = cf * 1024 / copy_bytes
        wr = cw * 1024 / copy_bytes
    lines = [f"calibration (plain device copy of {copy_bytes} bytes): "
             f"FETCH_SIZE reads {fr:.4f} x bytes, WRITE_SIZE reads {wr:.4f} x bytes"
             if fr else "calibration: no copy kernel found"]
    lines.append("kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read bytes | write bytes | "
                 "total bytes (calibrated, per dispatch)")
    for (name, counter), val in sorted(f.items(), key=lambda kv: -kv[1]):
        if counter != "FETCH_SIZE":
            continue
        wv = w.get((name, "WRITE_SIZE"), float("nan"))
        rb = val * 1024 / fr if fr else float("nan")
        wb = wv * 1024 / wr if wr else float("nan")
        lines.append(f"{_short(name)} | {fn[(name, counter)]} | {val:.1f} | {wv:.1f} | "
                     f"{rb:.0f} | {wb:.0f} | {rb + wb:.0f}")
    return "\n".join(lines)


def mfma(db: str, simds: int = 1024, xcds: int = 8) -> str:
    con = sqlite3.connect(db)
    agg = collections.defaultdict(list)
    dur = collections.defaultdict(dict)
    for name, counter, value, d, did in con.execute(
            "select kernel_name, counter_name, value, duration, dispatch_id "
            "from counters_collection"):
        agg[(name, counter)].append(value)
        dur[name][did] = d
    out = ["| kernel | dispatches | avg us | GRBM_GUI_ACTIVE / XCD | MFMA busy cycles | "
           "bf16 GFLOP | fp32 GFLOP | matrix TFLOP/s | MFMA util % |",
           "|---|---:|---:|---:|---:|---:|---:|---:|---:|"]
    mean = lambda n, c: sum(agg[(n, c)]) / len(agg[(n, c)]) if agg.get((n, c)) else 0.0
    names = sorted({n for n, _ in agg}, key=lambda n: -mean(n, "SQ_VALU_MFMA_BUSY_CYCLES"))
    for n in names:
        busy = mean(n, "SQ_VALU_MFMA_BUSY_CYCLES")
        if busy == 0:
            continue
        act = mean(n, "GRBM_GUI_ACTIVE") / xcds
        fb = mean(n, "SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512
        ff = mean(n, "SQ_INSTS_VALU_MFMA_MOPS_F32") * 512
        us = sum(dur[n].values()) / len(dur[n]) / 1e3
        out.append(f"| `{_short(n)}` | {len(dur[n])} | {us:.1f} | {act:.0f} | {busy:.0f} | "
                   f"{fb / 1e9:.3f} | {ff / 1e9:.3f} | {(fb + ff) / (us * 1e-6) / 1e12:.1f} | "
                   f"{100 * busy / (act * simds):.2f} |")
    return "\n".join(out)


def main(argv):
    if len(argv) >= 2 and argv[0] == "trace":
        print(trace(argv[1]))
    elif len(argv) >= 2 and argv[0] == "mfma":
        print(mfma(argv[1], *(int(x) for x in argv[2:4])))
    elif len(argv) >= 3 and argv[0] == "pmc":
        print(pmc(argv[1], argv[2], int(argv[3]) if len(argv) > 3 else 1 << 28))
    else:
        print(__doc__)
        return 2
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))
