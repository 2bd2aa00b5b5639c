"""Benchmark: padding-aware sigmoid attention fwd + bwd on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload nopad16k] [--no-cpu-baseline]

Definitions:
* A step is one pass of the whole hot path over one batch of resident
  synthetic input: sigattn_fwd, then the backward (sigattn_bwd_dkdv, one
  fused dK/dV kernel, then sigattn_bwd_dq), one kernel per call, all on
  torch's current stream. This is exactly the work of sigattn_fwd +
  sigattn_bwd.
* `value` is whole-step throughput in TFLOP/s. FLOPs are counted the pages'
  way (valid tokens only; backward = 2.5x forward) and divided by host wall
  time over exactly K steps, with a device synchronisation on both sides.
* Each kernel is also timed with HIP events recorded on the stream it runs
  on. Those times feed the per-kernel figures and the roofline of the
  dominant kernel.
* The line also carries the 25%-padding workload at the same shape per
  sample. The pages report both no padding and 25% padding.
* `varlen`: the cell-batch workload (71% padded tokens) timed fwd+bwd in the
  padded layout and in the packed layout on the same valid rows.
* `fp8`: the FP8 forward on the main workload: quantisation of Q, K and V
  (per-tile E4M3), then the forward on FP8 MFMA, each timed with HIP events;
  its TFLOP/s against the FP8 dense peak and against the bf16 forward.
* `softmax`: padding-aware softmax attention fwd+bwd on the main workload,
  with the same FLOP count, timed per call (forward: one kernel; backward:
  row statistics, fused dK/dV, dQ) with HIP events on the launch stream.

One GPU only. --gpus above 1 exits with a message.
"""

from __future__ import annotations

import argparse
import json
import os
import pathlib
import sys
import time

ROOT = pathlib.Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 MFMA, published
TRAFFIC_FILE = ROOT / "profiles" / "hbm_traffic.json"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="nopad16k")
    ap.add_argument("--pad-workload", default="pad25_16k", help="secondary workload reported in the same line ('' to skip)")
    ap.add_argument("--varlen-workload", default="cellbatch8k",
                    help="workload timed in the padded and the packed layout ('none' skips)")
    ap.add_argument("--fp8-workload", default="nopad16k",
                    help="workload of the FP8 forward sub-object ('' to skip)")
    ap.add_argument("--softmax-workload", default="nopad16k",
                    help="workload of the softmax fwd+bwd sub-object ('' to skip)")
    ap.add_argument("--configs", default="tiny,nopad16k,pad25_16k,cellbatch8k,nopad8k_d64,stress8k@1,stress8k@4,stress8k@16",
                    help="workloads (name or name@qk_scale) whose per-pass TFLOP/s the line reports under 'configs' "
                         "('' to skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after the timed steps, copy a buffer of this many bytes twice (a plain device copy of "
                         "known size that calibrates the rocprofv3 HBM byte counters); 0 skips it")
    return ap.parse_args()


def run_gpu(name, steps, warmup, seed=0, qk_scale=None):
    import torch

    import padding_aware_sigmoid_amd as sa
    import workloads
    from padding_aware_sigmoid_amd import accounting

    inp = workloads.make_inputs(name, seed=seed, qk_scale=qk_scale)
    w = inp["workload"]
    dev = torch.device("cuda:0")
    q, k, v, do = (inp[x].to(dev) for x in ("q", "k", "v", "do"))
    nq = torch.as_tensor(inp["seqlens_q"]).to(dev)
    nk = torch.as_tensor(inp["seqlens_k"]).to(dev)
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    stream = torch.cuda.current_stream(dev)

    # The kernels of one step, in launch order, with each kernel's algorithmic
    # contraction FLOPs per valid score pair: fwd 4D (QK^T, PV); dK/dV 8D (S,
    # dP, dV, dK, fused); dQ 6D (S, dP, dQ).
    a, b = w.alpha, w.bias
    launches = [("fwd", 4, lambda: sa.sigattn_fwd(q, k, v, nq, nk, a, b, out=o)),
                ("dkdv", 8, lambda: sa.sigattn_bwd_dkdv(q, k, v, do, nq, nk, a, b, dk=dk, dv=dv)),
                ("dq", 6, lambda: sa.sigattn_bwd_dq(q, k, v, do, nq, nk, a, b, dq=dq))]
    nl = len(launches)

    def step(ev=None):
        for i, (_, _, fn) in enumerate(launches):
            if ev is not None:
                ev[i].record(stream)
            fn()
        if ev is not None:
            ev[nl].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nl + 1)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    fl = accounting.attention_flops(w.Z, w.L, w.H, w.D, inp["seqlens_q"], inp["seqlens_k"])
    pairs = float((inp["seqlens_q"].astype("int64") * inp["seqlens_k"].astype("int64")).sum()) * w.H
    kern = {}
    for i, (name, per_pair, _) in enumerate(launches):
        ms = sum(e[i].elapsed_time(e[i + 1]) for e in events) / steps
        kern[name] = {"ms": ms, "flop": per_pair * w.D * pairs}
    for kv in kern.values():
        kv["tflops"] = kv["flop"] / (kv["ms"] * 1e-3) / 1e12
        kv["frac_peak"] = kv["tflops"] / PEAK_BF16_TFLOPS
    t_fwd = kern["fwd"]["ms"]
    t_bwd = sum(kv["ms"] for name, kv in kern.items() if name != "fwd")
    ms_step = elapsed / steps * 1e3
    res = {
        "workload": w,
        "qk_scale": inp["qk_scale"],
        "lengths": inp["seqlens_q"].tolist(),
        "ms_per_step": ms_step,
        "fwd_ms": t_fwd,
        "bwd_ms": t_bwd,
        "tflops_valid": fl["total_valid"] / (ms_step * 1e-3) / 1e12,
        "tflops_padded": fl["total_padded"] / (ms_step * 1e-3) / 1e12,
        "fwd_tflops_valid": fl["fwd_valid"] / (t_fwd * 1e-3) / 1e12,
        "bwd_tflops_valid": fl["bwd_valid"] / (t_bwd * 1e-3) / 1e12,
        "fwd_tflops_padded": fl["fwd_padded"] / (t_fwd * 1e-3) / 1e12,
        "bwd_tflops_padded": fl["bwd_padded"] / (t_bwd * 1e-3) / 1e12,
        "kernels": kern,
        "flops": fl,
    }
    del q, k, v, do, o, dq, dk, dv
    torch.cuda.empty_cache()
    return res


def run_layouts(name, steps, warmup, seed=0):
    """fwd+bwd of one workload in the padded layout and in the packed (varlen)
    layout, on the same valid rows, each timed with HIP events on the launch
    stream over `steps` steps. Returns ms per step for both."""
    import numpy as np
    import torch

    import padding_aware_sigmoid_amd as sa
    import workloads
    from padding_aware_sigmoid_amd import accounting

    inp = workloads.make_inputs(name, seed=seed)
    w = inp["workload"]
    dev = torch.device("cuda:0")
    q, k, v, do = (inp[x].to(dev) for x in ("q", "k", "v", "do"))
    n = inp["seqlens_q"]
    nq = torch.as_tensor(n).to(dev)
    nk = torch.as_tensor(inp["seqlens_k"]).to(dev)
    pack = lambda t: torch.cat([t[z, : int(n[z])] for z in range(w.Z)], 0).contiguous()  # noqa: E731
    qp, kp, vp, dop = (pack(t) for t in (q, k, v, do))
    cu = torch.as_tensor(np.concatenate([[0], np.cumsum(n)]).astype(np.int32)).to(dev)
    a, b = w.alpha, w.bias
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    op, dqp, dkp, dvp = (torch.empty_like(qp) for _ in range(4))
    stream = torch.cuda.current_stream(dev)

    def padded():
        sa.sigattn_fwd(q, k, v, nq, nk, a, b, out=o)
        sa.sigattn_bwd(q, k, v, do, nq, nk, a, b, dq=dq, dk=dk, dv=dv)

    def packed():
        sa.sigattn_fwd_varlen(qp, kp, vp, cu, cu, w.L, a, b, out=op)
        sa.sigattn_bwd_varlen(qp, kp, vp, dop, cu, cu, w.L, a, b, dq=dqp, dk=dkp, dv=dvp)

    res = {}
    for label, fn in (("padded", padded), ("packed", packed)):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res[label] = e0.elapsed_time(e1) / steps
    fl = accounting.attention_flops(w.Z, w.L, w.H, w.D, inp["seqlens_q"], inp["seqlens_k"])
    out = {"workload": w.name, "Z": w.Z, "H": w.H, "L": w.L, "D": w.D, "lengths": n.tolist(),
           "valid_token_fraction": round(float(n.sum()) / (w.Z * w.L), 4)}
    for label, ms in res.items():
        out[f"{label}_ms"] = round(ms, 4)
        out[f"{label}_tflops_valid"] = round(fl["total_valid"] / (ms * 1e-3) / 1e12, 2)
    out["packed_speedup"] = round(res["padded"] / res["packed"], 3)
    del q, k, v, do, qp, kp, vp, dop, o, dq, dk, dv, op, dqp, dkp, dvp
    torch.cuda.empty_cache()
    return out


def run_fp8(name, steps, warmup, seed=0):
    """FP8 forward on one workload: quantisation of Q, K, V and the forward,
    each timed per call with HIP events on the launch stream."""
    import torch

    import padding_aware_sigmoid_amd as sa
    import workloads
    from padding_aware_sigmoid_amd import accounting

    inp = workloads.make_inputs(name, seed=seed)
    w = inp["workload"]
    dev = torch.device("cuda:0")
    q, k, v = (inp[x].to(dev) for x in ("q", "k", "v"))
    nq = torch.as_tensor(inp["seqlens_q"]).to(dev)
    nk = torch.as_tensor(inp["seqlens_k"]).to(dev)
    q8, sq = sa.sigattn_quantize_fp8(q, nq)
    k8, sk = sa.sigattn_quantize_fp8(k, nk)
    v8, sv = sa.sigattn_quantize_fp8(v, nk)
    o8 = torch.empty_like(q)
    o = torch.empty_like(q)
    stream = torch.cuda.current_stream(dev)
    calls = [
        lambda: (sa.sigattn_quantize_fp8(q, nq, out=q8, scales=sq), sa.sigattn_quantize_fp8(k, nk, out=k8, scales=sk),
                 sa.sigattn_quantize_fp8(v, nk, out=v8, scales=sv)),
        lambda: sa.sigattn_fwd_fp8(q8, k8, v8, sq, sk, sv, nq, nk, w.alpha, w.bias, out=o8),
        lambda: sa.sigattn_fwd(q, k, v, nq, nk, w.alpha, w.bias, out=o),
    ]
    for _ in range(warmup):
        for fn in calls:
            fn()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for e in ev:
        for i, fn in enumerate(calls):
            e[i].record(stream)
            fn()
        e[3].record(stream)
    torch.cuda.synchronize()
    t = [sum(e[i].elapsed_time(e[i + 1]) for e in ev) / steps for i in range(3)]
    fl = accounting.attention_flops(w.Z, w.L, w.H, w.D, inp["seqlens_q"], inp["seqlens_k"])
    tf = fl["fwd_valid"] / (t[1] * 1e-3) / 1e12
    diff = float((o8.float() - o.float()).abs().max() / o.float().abs().max())
    out = {"workload": w.name, "Z": w.Z, "H": w.H, "L": w.L, "D": w.D, "format": "OCP E4M3, per-tile E8M0 scales",
           "quantize_qkv_ms": round(t[0], 4), "fwd_ms": round(t[1], 4), "fwd_tflops_valid": round(tf, 2),
           "frac_of_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4), "bf16_fwd_ms": round(t[2], 4),
           "speedup_vs_bf16_fwd": round(t[2] / t[1], 3), "max_rel_diff_vs_bf16_fwd": round(diff, 4)}
    del q, k, v, q8, k8, v8, o8, o
    torch.cuda.empty_cache()
    return out


def run_softmax(name, steps, warmup, seed=0):
    """Softmax attention fwd + bwd (padded layout) on one workload: ms per
    forward call and per backward call, from HIP events on the launch stream,
    and TFLOP/s counted as for sigmoid attention (valid tokens, bwd = 2.5x fwd)."""
    import torch

    import padding_aware_sigmoid_amd as sa
    import workloads
    from padding_aware_sigmoid_amd import accounting

    inp = workloads.make_inputs(name, seed=seed)
    w = inp["workload"]
    dev = torch.device("cuda:0")
    q, k, v, do = (inp[x].to(dev) for x in ("q", "k", "v", "do"))
    nq = torch.as_tensor(inp["seqlens_q"]).to(dev)
    nk = torch.as_tensor(inp["seqlens_k"]).to(dev)
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=dev)
    ws = torch.empty(w.Z * w.L * w.H * 8, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    calls = [lambda: sa.sigattn_softmax_fwd(q, k, v, nq, nk, w.alpha, out=o, lse=lse),
             lambda: sa.sigattn_softmax_bwd(q, k, v, o, do, lse, nq, nk, w.alpha, dq=dq, dk=dk, dv=dv, workspace=ws)]
    for _ in range(warmup):
        for fn in calls:
            fn()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in ev:
        for i, fn in enumerate(calls):
            e[i].record(stream)
            fn()
        e[2].record(stream)
    torch.cuda.synchronize()
    t_fwd = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    t_bwd = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    fl = accounting.attention_flops(w.Z, w.L, w.H, w.D, inp["seqlens_q"], inp["seqlens_k"])
    out = {"workload": w.name, "Z": w.Z, "H": w.H, "L": w.L, "D": w.D, "alpha": w.alpha,
           "ms_per_step": round(t_fwd + t_bwd, 4), "fwd_ms": round(t_fwd, 4), "bwd_ms": round(t_bwd, 4),
           "tflops_valid": round(fl["total_valid"] / ((t_fwd + t_bwd) * 1e-3) / 1e12, 2),
           "fwd_tflops_valid": round(fl["fwd_valid"] / (t_fwd * 1e-3) / 1e12, 2),
           "bwd_tflops_valid": round(fl["bwd_valid"] / (t_bwd * 1e-3) / 1e12, 2)}
    del q, k, v, do, o, dq, dk, dv, lse, ws
    torch.cuda.empty_cache()
    return out


def host_description():
    """Who ran the CPU baseline: core counts, CPU model, BLAS threads."""
    info = {"nproc": os.cpu_count()}
    try:
        info["cores_usable"] = len(os.sched_getaffinity(0))
    except AttributeError:
        info["cores_usable"] = os.cpu_count()
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                info["cpu_model"] = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info

        pools = threadpool_info()
        info["blas"] = [{"api": i.get("internal_api"), "threads": i.get("num_threads")} for i in pools]
        info["blas_threads"] = max([i.get("num_threads", 1) for i in pools] or [1])
    except Exception:  # noqa: BLE001
        info["blas_threads"] = None
    return info


# The CPU baseline's samples: (config key, workload, qk_scale, sample z,
# heads). One whole (z, h) head each, at the sample's true length, fwd + bwd:
# the oracle's cost depends on n_q * n_k * D only, so one head stands for the
# others of its sample, and its TFLOP/s for the config. To bound the run (the
# oracle is slow), the 25%-padding config takes its shortest sample and the
# cell-batch and stress configs their median one; the score scale of the
# stress config does not change the oracle's work, so s = 1 stands for all.
CPU_SAMPLES = (("tiny", "tiny", None, None, None), ("nopad16k", "nopad16k", None, 0, 1),
               ("pad25_16k", "pad25_16k", None, "shortest", 1), ("cellbatch8k", "cellbatch8k", None, "median", 1),
               ("stress8k", "stress8k", 1.0, "median", 1))


def cpu_baseline(main_name):
    """The oracle, as it stands, fwd + bwd on one whole head of every config
    (tiny: the whole batch), in float64 (the oracle) and in float32 (its
    timing mode), on the host cores. value: float64 on the main workload."""
    import numpy as np

    import oracle
    import workloads

    per = {}
    for key, name, scale, zsel, heads in CPU_SAMPLES:
        w = workloads.WORKLOADS[name]
        n_all = workloads.lengths(w, 0)
        if zsel is None:  # the whole batch
            Zs, Hs, n = w.Z, w.H, n_all
            q, k, v, do = workloads.make_tensors(w.Z, w.L, w.H, w.D, w.dtype, seed=0)
        else:
            order = np.argsort(n_all, kind="stable")
            z = int(order[len(n_all) // 2] if zsel == "median" else (order[0] if zsel == "shortest" else zsel))
            Zs, Hs, n = 1, heads, n_all[z:z + 1]
            q, k, v, do = workloads.make_tensors(1, w.L, heads, w.D, w.dtype, seed=0, qk_scale=scale or 1.0)
        Q, K, V, DO = (t.float().numpy() for t in (q, k, v, do))
        flop = 3.5 * 4.0 * w.D * float(np.sum(n.astype(np.int64) ** 2)) * Hs
        rec = {"workload": name, "sample": "batch" if zsel is None else f"z={z}", "Z": Zs, "H": Hs, "D": w.D,
               "lengths": n.tolist()}
        for dt in oracle.sigmoid_attention.TIMING_DTYPES:
            t0 = time.perf_counter()
            oracle.forward(Q, K, V, n, n, w.alpha, w.bias, dtype=dt)
            oracle.backward(Q, K, V, DO, n, n, w.alpha, w.bias, dtype=dt)
            dt_s = time.perf_counter() - t0
            rec[np.dtype(dt).name] = {"seconds": round(dt_s, 3), "tflops": flop / dt_s / 1e12}
        per[key] = rec
    host = host_description()
    main = per[main_name]
    return {"value": main["float64"]["tflops"], "unit": "TFLOP/s", "cores": host.get("blas_threads") or host["nproc"],
            "kind": "oracle",
            "sample": f"one whole (z,h) head of {main_name} (n={main['lengths'][0]}, D={main['D']}), fwd+bwd, the "
                      f"oracle in NumPy float64, {main['float64']['seconds']:.1f} s; FLOPs counted as for the GPU "
                      f"(3.5 x 4*D*n^2 per head). Every config in float64 and float32 under 'configs'.",
            "host": host, "configs": per}


def config_record(res):
    """Per-pass TFLOP/s of one workload's run, on valid and on padded FLOPs."""
    w, fl = res["workload"], res["flops"]
    tf = lambda f, ms: round(f / (ms * 1e-3) / 1e12, 2)  # noqa: E731
    return {"workload": w.name, "Z": w.Z, "H": w.H, "L": w.L, "D": w.D, "dtype": w.dtype,
            "qk_scale": res["qk_scale"], "lengths": res["lengths"],
            "fwd_ms": round(res["fwd_ms"], 4), "bwd_ms": round(res["bwd_ms"], 4),
            "ms_per_step": round(res["ms_per_step"], 4),
            "fwd_tflops_valid": tf(fl["fwd_valid"], res["fwd_ms"]),
            "bwd_tflops_valid": tf(fl["bwd_valid"], res["bwd_ms"]),
            "tflops_valid": tf(fl["total_valid"], res["ms_per_step"]),
            "fwd_tflops_padded": tf(fl["fwd_padded"], res["fwd_ms"]),
            "bwd_tflops_padded": tf(fl["bwd_padded"], res["bwd_ms"]),
            "tflops_padded": tf(fl["total_padded"], res["ms_per_step"]),
            "frac_of_bf16_peak_valid": round(fl["total_valid"] / (res["ms_per_step"] * 1e-3) / 1e12
                                             / PEAK_BF16_TFLOPS, 4),
            "kernels_ms": {k: round(v["ms"], 4) for k, v in res["kernels"].items()}}


def traffic_for(kernel_name: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, when it was taken
    on the current kernel sources. Otherwise null."""
    if not TRAFFIC_FILE.exists():
        return None
    try:
        rec = json.loads(TRAFFIC_FILE.read_text())
    except Exception:  # noqa: BLE001
        return None
    from padding_aware_sigmoid_amd.profiling import kernel_source_hash

    if rec.get("kernel_source_hash") != kernel_source_hash() or rec.get("workload") != workload:
        return None
    k = rec.get("kernels", {}).get(kernel_name)
    return None if k is None else k.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this path shards with no "
              "communication, one (z, h) slice per GPU).", file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(1)
    import padding_aware_sigmoid_amd as sa
    import workloads

    sa.load()
    main_res = run_gpu(args.workload, args.steps, args.warmup)
    pad_res = run_gpu(args.pad_workload, args.steps, args.warmup) if args.pad_workload not in ('', 'none') else None
    # every config: forward, backward and fwd+bwd TFLOP/s, valid and padded FLOPs
    configs = {}
    if args.configs not in ("", "none"):
        for key in args.configs.split(","):
            name, _, scale = key.partition("@")
            if name == args.workload and not scale:
                res = main_res
            elif pad_res is not None and name == args.pad_workload and not scale:
                res = pad_res
            else:
                res = run_gpu(name, args.steps, args.warmup, qk_scale=float(scale) if scale else None)
            configs[key] = config_record(res)
    w = main_res["workload"]
    dom_name = max(main_res["kernels"], key=lambda k: main_res["kernels"][k]["ms"])
    dom = main_res["kernels"][dom_name]
    roofline = {"bound": "mfma", "kernel": f"{dom_name}_bf16<D={w.D}>", "achieved": round(dom["tflops"], 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(dom["tflops"] / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic_for(dom_name, args.workload),
                "launch_ms": round(dom["ms"], 4), "flop_per_launch": dom["flop"]}
    line = {
        "metric": "sigmoid-attn fwd+bwd TFLOPS, L=16K D=128 bf16 (valid-token FLOPs, bwd=2.5x fwd)",
        "value": round(main_res["tflops_valid"], 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "Z": w.Z, "H": w.H, "L": w.L, "D": w.D, "alpha": w.alpha,
                   "bias": round(w.bias, 6), "lengths": main_res["lengths"], "parallelism": "none (1 GPU)"},
        "frac_of_bf16_peak": round(main_res["tflops_valid"] / PEAK_BF16_TFLOPS, 4),
        "fwd_tflops": round(main_res["fwd_tflops_valid"], 2),
        "bwd_tflops": round(main_res["bwd_tflops_valid"], 2),
        "kernels": {k: {"ms": round(v["ms"], 4), "tflops": round(v["tflops"], 2), "frac_peak": round(v["frac_peak"], 4)}
                    for k, v in main_res["kernels"].items()},
        "roofline": roofline,
    }
    if pad_res is not None:
        pw = pad_res["workload"]
        line["pad25"] = {
            "workload": pw.name, "Z": pw.Z, "H": pw.H, "L": pw.L, "D": pw.D, "lengths": pad_res["lengths"],
            "ms_per_step": round(pad_res["ms_per_step"], 4),
            "tflops_valid": round(pad_res["tflops_valid"], 2), "tflops_padded": round(pad_res["tflops_padded"], 2),
            "fwd_tflops_valid": round(pad_res["fwd_tflops_valid"], 2),
            "bwd_tflops_valid": round(pad_res["bwd_tflops_valid"], 2),
            "tflops_loss_vs_nopad": round(1.0 - pad_res["tflops_valid"] / main_res["tflops_valid"], 4),
        }
    if args.varlen_workload not in ("", "none"):
        line["varlen"] = run_layouts(args.varlen_workload, args.steps, args.warmup)
        # the same shape with no padding, when the config sweep timed it: how
        # close the cell batch comes to its kernels' rate on full tiles
        vw = workloads.WORKLOADS[args.varlen_workload]
        for key, rec in configs.items():
            cw = workloads.WORKLOADS[key.partition("@")[0]]
            if (cw.length_model == "full" and (cw.Z, cw.H, cw.L, cw.D) == (vw.Z, vw.H, vw.L, vw.D)
                    and rec.get("tflops_valid")):
                line["varlen"]["nopad_same_shape"] = {
                    "workload": key, "tflops_valid": rec["tflops_valid"],
                    "padded_frac_of_nopad": round(line["varlen"]["padded_tflops_valid"] / rec["tflops_valid"], 4),
                    "packed_frac_of_nopad": round(line["varlen"]["packed_tflops_valid"] / rec["tflops_valid"], 4)}
    if args.fp8_workload not in ("", "none"):
        line["fp8"] = run_fp8(args.fp8_workload, args.steps, args.warmup)
    if args.softmax_workload not in ("", "none"):
        sm = run_softmax(args.softmax_workload, args.steps, args.warmup)
        if args.softmax_workload == args.workload:
            sm["sigmoid_speedup"] = round(sm["ms_per_step"] / main_res["ms_per_step"], 3)
        line["softmax"] = sm
    if args.copy_bytes > 0:
        src = torch.ones(args.copy_bytes, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        line["copy_bytes"] = args.copy_bytes
    if configs:
        line["configs"] = configs
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.workload)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
