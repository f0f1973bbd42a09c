"""Summaries of rocprofv3 runs of the benchmark (kernel statistics and HBM counters).

Usage, after the three rocprofv3 runs (``--kernel-trace --stats``, ``--pmc FETCH_SIZE``,
``--pmc WRITE_SIZE``, each with ``-f csv -d DIR``) of the same bench.py command, plus for
matrix-core kernels a fourth (``--pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE
SQ_INSTS_VALU_MFMA_MOPS_I8 SQ_INSTS_VALU_MFMA_MOPS_BF16``, passed as ``--mfma DIR``) and a
fifth with the instruction-issue counters (``ISSUE_COUNTERS``, passed as ``--issue DIR``)::

    python -m int4_group_quantized_g128_amd.profiling \\
        --stats DIR_STATS --fetch DIR_FETCH --write DIR_WRITE \\
        --role 'gate_up=k_gemm<\\(q4::Act\\)0, 1, false, 1, 1, 4, 2>' \\
        --workload "..." --commands "..." --out profiles/NAME

Each ``--role NAME=REGEX`` names one kernel instantiation (a regular expression searched
in the demangled kernel name).  The summary ``NAME.md`` keeps every library kernel's
average duration and, per role, the FETCH_SIZE / WRITE_SIZE counters per dispatch scaled
by what the same counters read for a plain device copy of known size (the bench's
``--copy-calibration`` copy of 512 MiB, ``__amd_rocclr_copyBuffer``), plus a hash of the
GEMM kernel sources the counters were taken with.  ``NAME.txt`` repeats the derived
figures as ``key=value`` lines; bench.py reports them as the roofline traffic only while
the hash still matches the sources.
"""
import argparse
import collections
import csv
import glob
import hashlib
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
KERNEL_SOURCES = ("csrc/common.h", "csrc/internal.h", "csrc/gemm.hip", "csrc/gemm_prefill.hip")
COPY_BYTES = 512 * 1024 * 1024
COPY_KERNEL = "__amd_rocclr_copyBuffer"
SIMD_NUM = 256 * 4                     # MI355X: 256 CUs x 4 SIMDs
XCD_NUM = 8                            # GRBM_GUI_ACTIVE comes summed over the 8 XCDs
MOPS_UNIT = 512                        # one SQ_INSTS_VALU_MFMA_MOPS_* count = 512 operations
PEAK = {"i8": 5.0e15, "bf16": 2.5e15}  # dense MFMA operations / s
# one --pmc run (7 SQ counters and one GRBM counter: within one pass's limits)
ISSUE_COUNTERS = ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_WAVE_CYCLES",
                  "SQ_WAIT_ANY", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE")


def source_hash():
    """Hash of the GEMM kernel sources (counters are stale once these change)."""
    h = hashlib.sha1()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_kv(path):
    """The key=value figures of a summary (empty dict when the file is missing)."""
    out = {}
    if not os.path.exists(path):
        return out
    with open(path) as f:
        for line in f:
            if "=" in line:
                k, v = line.rstrip("\n").split("=", 1)
                out[k] = v
    return out


def _csv(d, suffix):
    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    rows = []
    for fn in files:
        with open(fn) as f:
            rows += list(csv.DictReader(f))
    return rows


def kernel_stats(d):
    """kernel name -> (calls, average ns)"""
    return {r["Name"]: (int(r["Calls"]), float(r["AverageNs"])) for r in _csv(d, "kernel_stats.csv")}


def counter_values(d, counter):
    """kernel name -> per-dispatch counter values (KiB for the *_SIZE counters)."""
    agg = collections.defaultdict(list)
    for r in _csv(d, "counter_collection.csv"):
        if r.get("Counter_Name") == counter:
            agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return agg


def _match(names, rx):
    hits = [n for n in names if re.search(rx, n)]
    if len(hits) != 1:
        raise SystemExit(f"role regex {rx!r} matches {len(hits)} kernels: {hits}")
    return hits[0]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--stats", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--role", action="append", default=[], help="NAME=REGEX")
    ap.add_argument("--workload", required=True)
    ap.add_argument("--commands", default="")
    ap.add_argument("--mfma", default=None, help="pmc run with the MFMA busy / ops counters")
    ap.add_argument("--issue", default=None, help="pmc run with the instruction-issue counters (ISSUE_COUNTERS)")
    ap.add_argument("--live", action="append", default=[],
                    help="NAME=MS: the same kernel's average from bench.py's HIP events in the stats run")
    ap.add_argument("--out", required=True)
    a = ap.parse_args()

    stats = kernel_stats(a.stats)
    fetch = counter_values(a.fetch, "FETCH_SIZE")
    write = counter_values(a.write, "WRITE_SIZE")
    kib = COPY_BYTES / 1024.0
    cf = max(fetch.get(COPY_KERNEL, [0.0]))
    cw = max(write.get(COPY_KERNEL, [0.0]))
    if not (cf and cw):
        raise SystemExit("the counter runs hold no copy-calibration dispatch")
    f_scale, w_scale = kib / cf, kib / cw
    sh = source_hash()
    lines = [f"# rocprofv3 summary: {a.workload}", "",
             f"GEMM kernel source hash `{sh}` (csrc/common.h, internal.h, gemm.hip, gemm_prefill.hip).", "",
             "Commands (on an MI355X; $R is the repository root):", "", "```", a.commands.strip(), "```", "",
             "## Kernel statistics (--kernel-trace --stats)", "",
             "| kernel | calls | average µs |", "|---|---|---|"]
    for name, (calls, avg) in sorted(stats.items(), key=lambda kv: -kv[1][0] * kv[1][1]):
        if "q4::" in name:
            lines.append(f"| `{name.split('(q4::GemmArgs)')[0][:120]}` | {calls} | {avg / 1e3:.2f} |")
    lines += ["", "## HBM counters per dispatch (--pmc FETCH_SIZE; --pmc WRITE_SIZE)", "",
              f"Calibration: the {COPY_BYTES}-byte device copy reads FETCH_SIZE {cf:.0f} KiB and WRITE_SIZE "
              f"{cw:.0f} KiB, so one counted KiB stands for {f_scale:.4f} KiB read and {w_scale:.4f} KiB written.",
              "", "| role | kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read bytes | written bytes | "
              "average µs (trace) |", "|---|---|---|---|---|---|---|---|"]
    kv = {"source_hash": sh, "fetch_scale": f"{f_scale:.6f}", "write_scale": f"{w_scale:.6f}"}
    for role in a.role:
        rname, rx = role.split("=", 1)
        kn = _match(set(fetch) | set(write) | set(stats), rx)
        fv, wv = fetch.get(kn, []), write.get(kn, [])
        fm = sum(fv) / max(len(fv), 1)
        wm = sum(wv) / max(len(wv), 1)
        rb, wb = fm * 1024 * f_scale, wm * 1024 * w_scale
        avg = stats.get(kn, (0, 0.0))[1] / 1e3
        lines.append(f"| {rname} | `{kn.split('(q4::GemmArgs)')[0]}` | {len(fv)} | {fm:.0f} | {wm:.0f} | "
                     f"{rb:.4g} | {wb:.4g} | {avg:.2f} |")
        kv[f"kernel[{rname}]"] = kn
        kv[f"read_bytes[{rname}]"] = f"{rb:.0f}"
        kv[f"write_bytes[{rname}]"] = f"{wb:.0f}"
        kv[f"traffic_bytes[{rname}]"] = f"{rb + wb:.0f}"
        kv[f"avg_us[{rname}]"] = f"{avg:.3f}"
    live = dict(x.split("=", 1) for x in a.live)
    if live:
        lines += ["", "## Kernel averages: rocprofv3 trace vs the bench's HIP events (same run)", "",
                  "| role | trace average µs | HIP-event average µs | ratio |", "|---|---|---|---|"]
        for rname, ms in live.items():
            tr = float(kv.get(f"avg_us[{rname}]", "nan"))
            ev = float(ms) * 1e3
            lines.append(f"| {rname} | {tr:.2f} | {ev:.2f} | {tr / ev:.4f} |")
            kv[f"live_avg_us[{rname}]"] = f"{ev:.3f}"
    if a.mfma:
        busy = counter_values(a.mfma, "SQ_VALU_MFMA_BUSY_CYCLES")
        gui = counter_values(a.mfma, "GRBM_GUI_ACTIVE")
        mops = {"i8": counter_values(a.mfma, "SQ_INSTS_VALU_MFMA_MOPS_I8"),
                "bf16": counter_values(a.mfma, "SQ_INSTS_VALU_MFMA_MOPS_BF16")}
        lines += ["", "## Matrix-core counters per dispatch (--pmc SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE "
                  "SQ_INSTS_VALU_MFMA_MOPS_I8 SQ_INSTS_VALU_MFMA_MOPS_BF16)", "",
                  f"MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x {SIMD_NUM} SIMDs), "
                  f"rocprofv3's MfmaUtil (its per-XCD maximum taken as the reported sum over the {XCD_NUM} XCDs / "
                  f"{XCD_NUM}); operations = MOPS x {MOPS_UNIT}; the rate divides them by the trace average.", "",
                  "| role | dispatches | MFMA busy % | INT8 ops / dispatch | bf16 ops / dispatch | rate | "
                  "of the dense peak |", "|---|---|---|---|---|---|---|"]
        for role in a.role:
            rname, rx = role.split("=", 1)
            kn = _match(set(busy) | set(stats), rx)
            bv, gv = busy.get(kn, []), gui.get(kn, [])
            if not bv or not gv:
                continue
            pct = 100.0 * (sum(bv) / len(bv)) / ((sum(gv) / len(gv)) / XCD_NUM * SIMD_NUM)
            ops = {t: (sum(v.get(kn, [0.0])) / max(len(v.get(kn, [])), 1)) * MOPS_UNIT for t, v in mops.items()}
            kind = "i8" if ops["i8"] >= ops["bf16"] else "bf16"
            avg_s = stats.get(kn, (0, 0.0))[1] * 1e-9
            rate = ops[kind] / avg_s if avg_s else 0.0
            lines.append(f"| {rname} | {len(bv)} | {pct:.1f} | {ops['i8']:.4g} | {ops['bf16']:.4g} | "
                         f"{rate / 1e12:.1f} T{'OP' if kind == 'i8' else 'FLOP'}/s | {rate / PEAK[kind]:.3f} |")
            kv[f"mfma_busy_pct[{rname}]"] = f"{pct:.2f}"
            kv[f"mfma_ops[{rname}]"] = f"{ops[kind]:.0f}"
            kv[f"mfma_frac_counter[{rname}]"] = f"{rate / PEAK[kind]:.4f}"
    if a.issue:
        cv = {c: counter_values(a.issue, c) for c in ISSUE_COUNTERS}
        lines += ["", f"## Instruction issue per dispatch (--pmc {' '.join(ISSUE_COUNTERS)})", "",
                  "VALU issue = SQ_INSTS_VALU x 4 cycles (a wave64 VALU instruction occupies its 16-lane SIMD "
                  f"4 cycles) / (GRBM_GUI_ACTIVE per XCD x {SIMD_NUM} SIMDs); waiting = SQ_WAIT_ANY / "
                  "SQ_WAVE_CYCLES (wave cycles spent waiting on anything: barriers, memory and LDS counters, "
                  "dependencies); LDS conflicts = SQ_LDS_BANK_CONFLICT cycles per SQ_INSTS_LDS instruction.", "",
                  "| role | dispatches | VALU instructions per MFMA | VALU issue % | waiting % of wave cycles | "
                  "LDS conflict cycles per LDS instruction |", "|---|---|---|---|---|---|"]
        for role in a.role:
            rname, rx = role.split("=", 1)
            kn = _match(set(cv["SQ_INSTS_VALU"]) | set(stats), rx)
            m = {c: (sum(v[kn]) / len(v[kn]) if v.get(kn) else 0.0) for c, v in cv.items()}
            if not m["GRBM_GUI_ACTIVE"] or not m["SQ_INSTS_MFMA"] or not m["SQ_WAVE_CYCLES"]:
                continue
            valu_pct = 100.0 * m["SQ_INSTS_VALU"] * 4 / (m["GRBM_GUI_ACTIVE"] / XCD_NUM * SIMD_NUM)
            wait_pct = 100.0 * m["SQ_WAIT_ANY"] / m["SQ_WAVE_CYCLES"]
            per_mfma = m["SQ_INSTS_VALU"] / m["SQ_INSTS_MFMA"]
            conf = m["SQ_LDS_BANK_CONFLICT"] / m["SQ_INSTS_LDS"] if m["SQ_INSTS_LDS"] else 0.0
            lines.append(f"| {rname} | {len(cv['SQ_INSTS_VALU'].get(kn, []))} | {per_mfma:.2f} | {valu_pct:.1f} | "
                         f"{wait_pct:.1f} | {conf:.2f} |")
            kv[f"valu_per_mfma[{rname}]"] = f"{per_mfma:.3f}"
            kv[f"valu_issue_pct[{rname}]"] = f"{valu_pct:.2f}"
            kv[f"wait_pct[{rname}]"] = f"{wait_pct:.2f}"
            kv[f"lds_conflict_per_inst[{rname}]"] = f"{conf:.3f}"
    os.makedirs(os.path.dirname(os.path.abspath(a.out)), exist_ok=True)
    with open(a.out + ".md", "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(a.out + ".txt", "w") as f:
        for k, v in kv.items():
            f.write(f"{k}={v}\n")
    print("\n".join(lines))


if __name__ == "__main__":
    main()
