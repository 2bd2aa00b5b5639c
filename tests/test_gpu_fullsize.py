"""Parity at the full workload sizes, in the launch configuration the bench times.

At these sizes the oracle computes sampled rows one by one. This is exact:
* an O or dQ row depends only on its own query row;
* a dK or dV row depends only on its own key row.
The sampled rows always include rows 0 and 1, tile edges, n-1, n (the first
padded row) and L-1, plus random rows. Every sampled padded row must be
exactly 0. The skip decisions (tile counters) are compared in full with the
oracle's tile plan.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import device_inputs, note, rel_err

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2


def _sample_rows(n, L, rng):
    fixed = [0, 1, 63, 64, 127, 128, 255, 256, n - 1, n, n + 1, L - 1]
    extra = rng.integers(0, max(1, n), 4).tolist() if n > 0 else []
    return np.array(sorted({r for r in fixed + extra if 0 <= r < L}), dtype=np.int64)


def _run_full(name, qk_scale=None, heads_per_sample=2, seed=0):
    import padding_aware_sigmoid_amd as sa

    inp = workloads.make_inputs(name, seed=seed, qk_scale=qk_scale)
    w = inp["workload"]
    nq, nk = inp["seqlens_q"], inp["seqlens_k"]
    note(f"full-size {name} scale={inp['qk_scale']} Z={w.Z} L={w.L} H={w.H} D={w.D} n={nq.tolist()}")
    dq_, dk_, dv_, ddo, dnq, dnk = device_inputs(inp["q"], inp["k"], inp["v"], inp["do"], nq, nk)
    tcs = {}
    for kname, kern, axis in (("fwd", sa.KERNEL_FWD, 0), ("dq", sa.KERNEL_DQ, 0), ("dkdv", sa.KERNEL_DKDV, 1)):
        bq, bk = sa.sigattn_tile_config(kern, w.D, torch.bfloat16)
        tcs[kname] = (bq, bk, torch.full((w.Z * w.H * -(-w.L // (bq if axis == 0 else bk)),), -1,
                                          dtype=torch.int32, device="cuda"))
    o = sa.sigattn_fwd(dq_, dk_, dv_, dnq, dnk, w.alpha, w.bias, tile_counts=tcs["fwd"][2])
    gq, gk, gv = sa.sigattn_bwd(dq_, dk_, dv_, ddo, dnq, dnk, w.alpha, w.bias, tile_counts_dq=tcs["dq"][2],
                                tile_counts_dkdv=tcs["dkdv"][2])
    torch.cuda.synchronize()
    # skip decisions, in full
    for kname, (bq, bk, t) in tcs.items():
        by_q, by_k = oracle.tile_plan(nq, nk, w.L, bq, bk)
        want = by_k if kname == "dkdv" else by_q
        got = t.cpu().numpy().reshape(w.Z, w.H, -1)
        assert all(np.array_equal(got[:, h], want) for h in range(w.H)), f"{name}: {kname} skip plan differs"
    outs = {"O": o, "dQ": gq, "dK": gk, "dV": gv}
    assert all(bool(torch.isfinite(t).all()) for t in outs.values()), f"{name}: non-finite output"
    Q, K, V, DO = (t.float().numpy() for t in (inp["q"], inp["k"], inp["v"], inp["do"]))
    rng = np.random.default_rng(1234)
    got = {k: [] for k in outs}
    ref = {k: [] for k in outs}
    for z in range(w.Z):
        heads = sorted({0, w.H - 1, int(rng.integers(0, w.H))})[:max(1, heads_per_sample)]
        qrows = _sample_rows(int(nq[z]), w.L, rng)
        krows = _sample_rows(int(nk[z]), w.L, rng)
        for h in heads:
            o_ref = oracle.forward_rows(Q, K, V, nq, nk, w.alpha, w.bias, z, h, qrows)
            dq_ref, dk_ref, dv_ref = oracle.backward_rows(Q, K, V, DO, nq, nk, w.alpha, w.bias, z, h, qrows, krows)
            for key, rows, r in (("O", qrows, o_ref), ("dQ", qrows, dq_ref), ("dK", krows, dk_ref),
                                 ("dV", krows, dv_ref)):
                g = outs[key][z, torch.as_tensor(rows, device="cuda"), h].float().cpu().numpy().astype(np.float64)
                pad = rows >= (nq[z] if key in ("O", "dQ") else nk[z])
                assert np.all(g[pad] == 0.0), f"{name}: {key} padded sampled row not exactly 0 (z={z})"
                got[key].append(g)
                ref[key].append(r)
    errs = {k: rel_err(np.concatenate(got[k]), np.concatenate(ref[k])) for k in outs}
    for k, e in errs.items():
        assert e <= BF16_TOL, f"{name} scale={inp['qk_scale']}: {k} sampled rel err {e:.3e} > {BF16_TOL}"
    del dq_, dk_, dv_, ddo, o, gq, gk, gv
    torch.cuda.empty_cache()
    return errs


def test_nopad16k():
    _run_full("nopad16k", heads_per_sample=3)


def test_pad25_16k():
    _run_full("pad25_16k")


def test_cellbatch8k():
    _run_full("cellbatch8k")


@pytest.mark.parametrize("scale", [1.0, 4.0, 16.0])
def test_stress8k(scale):
    _run_full("stress8k", qk_scale=scale)
