"""Summaries of rocprofv3 output for the sigattn kernels.

    python -m padding_aware_sigmoid_amd.profiling stats    TRACE_DIR  [-o OUT.md]
    python -m padding_aware_sigmoid_amd.profiling counters PMC_DIR... [-o OUT.md]
    python -m padding_aware_sigmoid_amd.profiling traffic  --fetch DIR --write DIR --workload NAME
                                                           --copy-bytes N [-o OUT.json]

`stats` tabulates a `--kernel-trace --stats` run: per kernel and grid size
(one workload's launches), calls, mean, the warm median (every dispatch but
the first, cold one), min and max; then rocprofv3's own per-kernel stats. `counters` tabulates `--pmc` runs: each counter's mean per
dispatch, per kernel. `traffic` turns a FETCH_SIZE run and a WRITE_SIZE run
into HBM bytes per launch. Each counter is scaled by the factor that makes it
read the known size of a plain device copy recorded in the same run
(`bench.py --copy-bytes N`). The JSON carries a hash of the kernel sources, so
a reader can tell when the kernels have changed since the counters were taken.
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import pathlib
import re
import sys

ROOT = pathlib.Path(__file__).resolve().parent.parent
KERNEL_SOURCES = ["padding_aware_sigmoid_amd/csrc/common.hpp", "padding_aware_sigmoid_amd/csrc/fwd.hip",
                  "padding_aware_sigmoid_amd/csrc/bwd_kernels.hpp", "padding_aware_sigmoid_amd/csrc/bwd.hip",
                  "padding_aware_sigmoid_amd/csrc/bwd_softmax_dk128.hip", "padding_aware_sigmoid_amd/csrc/softmax.hip",
                  "padding_aware_sigmoid_amd/csrc/fp8.hip", "padding_aware_sigmoid_amd/build.py"]
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update((ROOT / p).read_bytes())
    return h.hexdigest()[:16]


def short_name(kernel: str) -> str | None:
    """The bench name of a sigattn kernel from its demangled or mangled name,
    else None. Sigmoid bf16: fwd, dq, dk, dv, dkdv; softmax: the same with an
    sm_ prefix, plus sm_rowstats; fp32 kernels carry a _fp32 suffix; the FP8
    path's kernels are fp8_fwd and fp8_quantize. The dK/dV kernel with queries
    and keys exchanged (its last template argument true) computes dQ."""
    m = re.search(r"sigattn::(\w+?)_kernel<([^>]*)>", kernel)
    if m is not None:
        base, args = m.group(1), [a.strip() for a in m.group(2).split(",")]
        ints = [int(a) for a in args if a.isdigit()]
        float_arg = "float" in args
        swapped = "true" in args
    else:  # e.g. _ZN7sigattn16dkdv_bf16_kernelILi128ELi1ELi0EEEv...
        m = re.search(r"_ZN7sigattn\d+(\w+?)_kernelI(.*?)EEv", kernel)
        if m is None:
            return None
        base = m.group(1)
        ints = [int(x) for x in re.findall(r"Li(\d+)E", m.group(2))]
        float_arg = m.group(2).startswith("f")
        swapped = "Lb1E" in m.group(2)
    sm = base.startswith("sm_")
    core = base[3:] if sm else base
    if core == "rowstats":
        return "sm_rowstats" + ("_fp32" if float_arg else "")
    if core in ("fwd_fp8", "quantize_fp8"):
        return "fp8_" + core.split("_")[0]
    mk = re.fullmatch(r"(fwd|dq|dkdv)_(bf16|fp32)", core)
    if mk is None:
        return None
    kind, dtype = mk.groups()
    if dtype == "bf16" and kind == "dq" and len(ints) > 1:
        sm = sm or ints[1] == 1
    if dtype == "bf16" and kind == "dkdv" and len(ints) > 1:
        kind = "dq" if swapped else {0: "dkdv", 1: "dk", 2: "dv"}[ints[1]]
        sm = sm or (len(ints) > 2 and ints[2] == 1)
    return ("sm_" if sm else "") + kind + ("" if dtype == "bf16" else "_fp32")


def _csv(path: pathlib.Path, suffix: str) -> list[dict]:
    files = sorted(path.rglob(f"*{suffix}")) if path.is_dir() else [path]
    if not files:
        raise FileNotFoundError(f"no *{suffix} under {path}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def stats_table(trace_dir: pathlib.Path) -> str:
    rows = _csv(trace_dir, "kernel_stats.csv")
    out = ["| kernel | calls | avg ms | min ms | max ms | share of GPU time |", "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        name = short_name(r["Name"]) or r["Name"][:48]
        out.append(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e6:.4f} | {float(r['MinNs']) / 1e6:.4f} | "
                   f"{float(r['MaxNs']) / 1e6:.4f} | {float(r['Percentage']):.2f}% |")
    return "\n".join(out)


def _grid(r: dict) -> int:
    for key in ("Grid_Size_X", "Grid_Size", "Grid_SizeX"):
        if key in r and r[key] not in ("", None):
            return int(r[key])
    return 0


def trace_groups(trace_dir: pathlib.Path) -> dict:
    """Per-dispatch durations (ns, in start order) from a --kernel-trace run,
    keyed by (kernel name, grid size): one workload's launches of a kernel
    share a grid size, so the same kernel run on two workloads falls into two
    groups."""
    groups: dict = {}
    for r in sorted(_csv(trace_dir, "kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"])):
        name = short_name(r["Kernel_Name"]) or r["Kernel_Name"][:48]
        dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        groups.setdefault((name, _grid(r)), []).append(dur)
    return groups


def trace_table(trace_dir: pathlib.Path) -> str:
    """Calls, mean, warm median (every dispatch but the group's first, which
    is cold), min and max per (kernel, grid size)."""
    out = ["| kernel | grid (work-items) | calls | avg ms | warm median ms | min ms | max ms |",
           "|---|---:|---:|---:|---:|---:|---:|"]
    rows = []
    for (name, grid), d in trace_groups(trace_dir).items():
        warm = sorted(d[1:]) if len(d) > 1 else list(d)
        med = warm[len(warm) // 2] if len(warm) % 2 else 0.5 * (warm[len(warm) // 2 - 1] + warm[len(warm) // 2])
        rows.append((sum(d), f"| {name} | {grid} | {len(d)} | {sum(d) / len(d) / 1e6:.4f} | {med / 1e6:.4f} | "
                             f"{min(d) / 1e6:.4f} | {max(d) / 1e6:.4f} |"))
    out += [r for _, r in sorted(rows, key=lambda x: -x[0])]
    return "\n".join(out)


def counter_means(pmc_dirs: list[pathlib.Path]) -> dict:
    """{kernel: {counter: mean per dispatch}} over the sigattn kernels (and the copy kernel)."""
    acc: dict = {}
    for d in pmc_dirs:
        for r in _csv(d, "counter_collection.csv"):
            name = short_name(r["Kernel_Name"]) or (COPY_KERNEL if COPY_KERNEL in r["Kernel_Name"] else None)
            if name is None:
                continue
            acc.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: {c: sum(v) / len(v) for c, v in cs.items()} for k, cs in acc.items()}


# Ratios read off the SQ counters. SQ_WAVE_CYCLES, SQ_WAIT_ANY and
# SQ_ACTIVE_INST_VALU count wave-cycles in units of 4 clocks;
# SQ_VALU_MFMA_BUSY_CYCLES counts SIMD clocks. With one wave per SIMD (every
# bf16 kernel at D = 128, the head size these counters are taken at),
# 4 * SQ_WAVE_CYCLES is the SIMD clocks the waves were resident, so the
# MFMA-busy fraction needs no assumption about the clock. At two waves per
# SIMD (D = 64) it would read half the true fraction.
DERIVED = (
    ("VALU instr / MFMA", ("SQ_INSTS_VALU", "SQ_INSTS_MFMA"), lambda a, b: a / b),
    ("transcendental instr / MFMA", ("SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_MFMA"), lambda a, b: a / b),
    ("LDS instr / MFMA", ("SQ_INSTS_LDS", "SQ_INSTS_MFMA"), lambda a, b: a / b),
    ("MFMA busy / SIMD clocks", ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_WAVE_CYCLES"), lambda a, b: a / (4 * b)),
    ("VALU active / wave cycles", ("SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES"), lambda a, b: a / b),
    ("waiting / wave cycles", ("SQ_WAIT_ANY", "SQ_WAVE_CYCLES"), lambda a, b: a / b),
    ("LDS bank conflicts / LDS active", ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE"), lambda a, b: a / b),
)


def counters_table(pmc_dirs: list[pathlib.Path]) -> str:
    means = counter_means(pmc_dirs)
    names = sorted({c for cs in means.values() for c in cs})
    out = ["| kernel | " + " | ".join(names) + " |", "|---|" + "---:|" * len(names)]
    for k, cs in means.items():
        if k == COPY_KERNEL:
            continue
        out.append(f"| {k} | " + " | ".join(f"{cs[c]:.4g}" if c in cs else "" for c in names) + " |")
    rows = [(label, f) for label, need, f in DERIVED if all(n in names for n in need)]
    if rows:
        kernels = [k for k in means if k != COPY_KERNEL]
        out += ["", "| ratio | " + " | ".join(kernels) + " |", "|---|" + "---:|" * len(kernels)]
        for label, need, f in DERIVED:
            if not all(n in names for n in need):
                continue
            vals = []
            for k in kernels:
                a, b = (means[k].get(n) for n in need)
                vals.append("" if a is None or not b else f"{f(a, b):.3f}")
            out.append(f"| {label} | " + " | ".join(vals) + " |")
    return "\n".join(out)


def _copy_factor(rows: list[dict], counter: str, copy_bytes: int) -> float:
    """Known bytes / counted bytes for the calibration copy: the copy-kernel
    dispatches with the largest grid in the run (the inputs' own small copies
    have far smaller grids)."""
    copies = [r for r in rows if COPY_KERNEL in r["Kernel_Name"] and r["Counter_Name"] == counter]
    if not copies:
        raise ValueError(f"no {COPY_KERNEL} dispatch in the {counter} run")
    g = max(int(r["Grid_Size"]) for r in copies)
    vals = [float(r["Counter_Value"]) * 1024 for r in copies if int(r["Grid_Size"]) == g]
    return copy_bytes / (sum(vals) / len(vals))


def traffic(fetch_dir: pathlib.Path, write_dir: pathlib.Path, workload: str, copy_bytes: int) -> dict:
    frows = _csv(fetch_dir, "counter_collection.csv")
    wrows = _csv(write_dir, "counter_collection.csv")
    f_fac = _copy_factor(frows, "FETCH_SIZE", copy_bytes)
    w_fac = _copy_factor(wrows, "WRITE_SIZE", copy_bytes)
    means = counter_means([fetch_dir, write_dir])
    kernels = {}
    for k, cs in means.items():
        if k == COPY_KERNEL or "FETCH_SIZE" not in cs or "WRITE_SIZE" not in cs:
            continue
        fb, wb = cs["FETCH_SIZE"] * 1024 * f_fac, cs["WRITE_SIZE"] * 1024 * w_fac
        kernels[k] = {"fetch_kib_raw": round(cs["FETCH_SIZE"], 2), "write_kib_raw": round(cs["WRITE_SIZE"], 2),
                      "fetch_bytes": round(fb), "write_bytes": round(wb), "hbm_bytes_per_launch": round(fb + wb)}
    return {"kernel_source_hash": kernel_source_hash(), "workload": workload, "copy_bytes": copy_bytes,
            "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4), "kernels": kernels}


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("stats")
    a.add_argument("trace_dir", type=pathlib.Path)
    a.add_argument("-o", type=pathlib.Path)
    c = sub.add_parser("counters")
    c.add_argument("pmc_dirs", type=pathlib.Path, nargs="+")
    c.add_argument("-o", type=pathlib.Path)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", type=pathlib.Path, required=True)
    t.add_argument("--write", type=pathlib.Path, required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("-o", type=pathlib.Path)
    args = ap.parse_args(argv)
    if args.cmd == "stats":
        try:
            text = trace_table(args.trace_dir) + "\n\n" + stats_table(args.trace_dir)
        except FileNotFoundError:
            text = stats_table(args.trace_dir)
    elif args.cmd == "counters":
        text = counters_table(args.pmc_dirs)
    else:
        text = json.dumps(traffic(args.fetch, args.write, args.workload, args.copy_bytes), indent=1)
    if args.o:
        args.o.write_text(text + "\n")
    else:
        sys.stdout.write(text + "\n")


if __name__ == "__main__":
    main()
