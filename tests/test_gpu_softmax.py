"""Padding-aware softmax attention on the GPU against the CPU oracle
(oracle.softmax_attention).

* O, LSE, dQ, dK and dV at sizes that span several tiles with a ragged tail,
  bf16 (2e-2 relative to the largest reference value) and fp32 (1e-5), D = 64
  and 128, lengths that include 0 keys and 0 queries.
* LSE: bf16 sums the row's P after rounding it to bf16 (so that O is a convex
  combination of V rows), which moves the row sum by at most 2^-8 relative
  (bf16's unit roundoff) and LSE by at most 2^-8 absolute: 4e-3. fp32: 1e-5.
* fp32 gradients: dS = P (dP - D) subtracts numbers of the size of dP, and the
  sums over rows cancel on top, so fp32 rounding is relative to the sums of
  the terms' absolute values, not to the result (on these inputs those sums
  reach a few hundred times max|dK|). The bound is 2^-22 (4 fp32 unit
  roundoffs) of that absolute-term scale, and never tighter than 1e-5 of
  max|ref|.
* Padded rows of every output are exactly 0, and padded input rows (NaN here)
  are never read.
* The packed layout against the padded one, bit for bit.
* At the 16K bench size, sampled rows against the oracle's row functions.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import assert_padding_zero, device_inputs, f64, host, note, rel_err

pytestmark = pytest.mark.gpu

SM = oracle.softmax_attention
TOL = {"bf16": 2e-2, "fp32": 1e-5}
LSE_TOL = {"bf16": 4e-3, "fp32": 1e-5}

CASES = [
    # (label, dtype, Z, L, H, D, nq, nk)
    ("bf16-d64", "bf16", 3, 300, 2, 64, [300, 131, 7], [250, 131, 40]),
    ("bf16-d128", "bf16", 3, 333, 2, 128, [333, 0, 200], [100, 5, 333]),
    ("bf16-d128-nokeys", "bf16", 2, 260, 1, 128, [260, 90], [0, 260]),
    ("fp32-d64", "fp32", 2, 200, 2, 64, [200, 77], [150, 200]),
    ("fp32-d128", "fp32", 2, 130, 1, 128, [65, 130], [130, 1]),
    # both sides of the fused dK/dV kernel's 128-row passes and 256-row tiles
    ("bf16-d128-passes", "bf16", 6, 400, 1, 128, [1, 127, 128, 129, 256, 385], [385, 256, 129, 128, 127, 1]),
    ("bf16-d64-passes", "bf16", 6, 400, 1, 64, [1, 127, 128, 129, 256, 385], [385, 256, 129, 128, 127, 1]),
]


def _packed(t, n):
    return torch.cat([t[z, : int(n[z])] for z in range(t.shape[0])], 0).contiguous()


def _cu(n):
    return np.concatenate([[0], np.cumsum(np.asarray(n, np.int64))]).astype(np.int32)


def _abs_term_scales(Q, K, V, DO, nq, nk, alpha):
    """Per gradient, the largest sum of its terms' absolute values: dQ from
    alpha |dS| |K|, dK from alpha |dS|^T |Q|, dV from P^T |dO|, with
    |dS| <= P (|dP| + |D|). P comes from the oracle's own (O, LSE)."""
    out = {"dQ": 0.0, "dK": 0.0, "dV": 0.0}
    for z in range(Q.shape[0]):
        a, b = int(nq[z]), int(nk[z])
        if a == 0 or b == 0:
            continue
        for h in range(Q.shape[2]):
            q, k, v, do = Q[z, :a, h], K[z, :b, h], V[z, :b, h], DO[z, :a, h]
            o, lse = SM.head_forward(q, k, v, alpha)
            p = np.exp(alpha * (q @ k.T) - lse[:, None])
            ads = p * (np.abs(do @ v.T) + np.abs((do * o).sum(1))[:, None])
            out["dQ"] = max(out["dQ"], float((alpha * ads @ np.abs(k)).max()))
            out["dK"] = max(out["dK"], float((alpha * ads.T @ np.abs(q)).max()))
            out["dV"] = max(out["dV"], float((p.T @ np.abs(do)).max()))
    return out


def _lse_err(got, ref, dtype):
    d = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    if dtype == "fp32":
        return d / max(1.0, float(np.max(np.abs(ref))))
    return d


@pytest.mark.parametrize("label,dtype,Z,L,H,D,nq,nk", CASES)
def test_softmax_matches_oracle(label, dtype, Z, L, H, D, nq, nk):
    import padding_aware_sigmoid_amd as sa

    note(f"softmax {label} nq={nq} nk={nk}")
    q, k, v, do = workloads.make_tensors(Z, L, H, D, dtype, seed=31)
    dq_, dk_, dv_, ddo, dnq, dnk = device_inputs(q, k, v, do, nq, nk)
    alpha = 1.0 / np.sqrt(D)
    o, lse = sa.sigattn_softmax_fwd(dq_, dk_, dv_, dnq, dnk, alpha)
    g = sa.sigattn_softmax_bwd(dq_, dk_, dv_, o, ddo, lse, dnq, dnk, alpha)
    torch.cuda.synchronize()
    Q, K, V, DO = (f64(t) for t in (q, k, v, do))
    o_ref, lse_ref = SM.forward(Q, K, V, nq, nk, alpha)
    refs = (o_ref,) + SM.backward(Q, K, V, DO, nq, nk, alpha)
    scales = _abs_term_scales(Q, K, V, DO, nq, nk, alpha) if dtype == "fp32" else {}
    for name, got, ref in zip(("O", "dQ", "dK", "dV"), (o,) + tuple(g), refs):
        e = rel_err(host(got), ref)
        tol = TOL[dtype]
        if name in scales and np.abs(ref).max() > 0:
            tol = max(tol, 2.0**-22 * scales[name] / float(np.abs(ref).max()))
        assert e <= tol, f"{label}: {name} rel err {e:.3e} > {tol:.3e}"
    lse_h = host(lse)  # [Z, L, H]; the oracle's is [Z, H, L]
    e = _lse_err(lse_h, lse_ref.transpose(0, 2, 1), dtype)
    assert e <= LSE_TOL[dtype], f"{label}: LSE err {e:.3e}"
    for name, t, n in (("O", o, nq), ("LSE", lse, nq), ("dQ", g[0], nq), ("dK", g[1], nk), ("dV", g[2], nk)):
        assert_padding_zero(name, host(t), n)
    for z in range(Z):  # a sample with no key has O = 0 and LSE = 0 on every row
        if nk[z] == 0:
            assert np.all(host(o)[z] == 0.0) and np.all(lse_h[z] == 0.0)


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 128), ("fp32", 128)])
def test_softmax_padding_is_never_read(dtype, D):
    import padding_aware_sigmoid_amd as sa

    note(f"softmax NaN padding {dtype} D={D}")
    Z, L, H = 2, 300, 2
    nq, nk = [300, 140], [170, 300]
    q, k, v, do = workloads.make_tensors(Z, L, H, D, dtype, seed=32)
    dq_, dk_, dv_, ddo, dnq, dnk = device_inputs(q, k, v, do, nq, nk)
    outs = []
    for poison in (False, True):
        tq, tk, tv, tdo = (t.clone() for t in (dq_, dk_, dv_, ddo))
        if poison:
            for z in range(Z):
                tq[z, nq[z]:] = float("nan")
                tdo[z, nq[z]:] = float("nan")
                tk[z, nk[z]:] = float("nan")
                tv[z, nk[z]:] = float("nan")
        o, lse = sa.sigattn_softmax_fwd(tq, tk, tv, dnq, dnk)
        if poison:
            for z in range(Z):  # O's padded rows are outputs: poison what the backward reads
                o[z, nq[z]:] = float("nan")
        g = sa.sigattn_softmax_bwd(tq, tk, tv, o, tdo, lse, dnq, dnk)
        torch.cuda.synchronize()
        if poison:
            for z in range(Z):
                o[z, nq[z]:] = 0.0
        outs.append((o, lse) + tuple(g))
    for name, a, b in zip(("O", "LSE", "dQ", "dK", "dV"), outs[0], outs[1]):
        assert torch.equal(a, b), f"softmax {dtype} D={D}: {name} changed when padding held NaN"


@pytest.mark.parametrize("label,dtype,Z,L,H,D,nq,nk", CASES)
def test_softmax_packed_matches_padded(label, dtype, Z, L, H, D, nq, nk):
    import padding_aware_sigmoid_amd as sa

    note(f"softmax packed {label}")
    q, k, v, do = workloads.make_tensors(Z, L, H, D, dtype, seed=33)
    dq_, dk_, dv_, ddo, dnq, dnk = device_inputs(q, k, v, do, nq, nk)
    o, lse = sa.sigattn_softmax_fwd(dq_, dk_, dv_, dnq, dnk)
    g = sa.sigattn_softmax_bwd(dq_, dk_, dv_, o, ddo, lse, dnq, dnk)
    qp, dop = _packed(dq_, nq), _packed(ddo, nq)
    kp, vp = _packed(dk_, nk), _packed(dv_, nk)
    cq = torch.as_tensor(_cu(nq)).to(dq_.device)
    ck = torch.as_tensor(_cu(nk)).to(dq_.device)
    o_p, lse_p = sa.sigattn_softmax_fwd(qp, kp, vp, cq, ck, max_len=L)
    g_p = sa.sigattn_softmax_bwd(qp, kp, vp, o_p, dop, lse_p, cq, ck, max_len=L)
    torch.cuda.synchronize()
    for name, a, b, n in (("O", o_p, o, nq), ("LSE", lse_p, lse, nq), ("dQ", g_p[0], g[0], nq),
                          ("dK", g_p[1], g[1], nk), ("dV", g_p[2], g[2], nk)):
        assert torch.equal(a, _packed(b, n)), f"{label}: packed {name} differs from padded {name}"


def test_softmax_autograd_matches_entry_points():
    import padding_aware_sigmoid_amd as sa

    note("softmax autograd")
    Z, L, H, D = 2, 150, 2, 64
    n = [150, 61]
    q, k, v, do = workloads.make_tensors(Z, L, H, D, "bf16", seed=34)
    dq_, dk_, dv_, ddo, dn, _ = device_inputs(q, k, v, do, n, n)
    leaves = [t.clone().requires_grad_(True) for t in (dq_, dk_, dv_)]
    o = sa.softmax_attention(*leaves, dn, dn)
    o.backward(ddo)
    o2, lse2 = sa.sigattn_softmax_fwd(dq_, dk_, dv_, dn, dn)
    g2 = sa.sigattn_softmax_bwd(dq_, dk_, dv_, o2, ddo, lse2, dn, dn)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o2)
    for leaf, g in zip(leaves, g2):
        assert torch.equal(leaf.grad, g)


def _sample_rows(n, L, rng):
    fixed = [0, 1, 63, 64, 127, 128, 255, 256, n - 1, n, n + 1, L - 1]
    extra = rng.integers(0, max(1, n), 4).tolist() if n > 0 else []
    return np.array(sorted({r for r in fixed + extra if 0 <= r < L}), dtype=np.int64)


@pytest.mark.parametrize("name", ["nopad16k", "pad25_16k"])
def test_softmax_fullsize_sampled(name):
    """The bench's sizes: sampled rows against the oracle's exact row functions."""
    import padding_aware_sigmoid_amd as sa

    inp = workloads.make_inputs(name, seed=35)
    w = inp["workload"]
    nq, nk = inp["seqlens_q"], inp["seqlens_k"]
    note(f"softmax full-size {name} Z={w.Z} L={w.L} H={w.H} D={w.D}")
    dq_, dk_, dv_, ddo, dnq, dnk = device_inputs(inp["q"], inp["k"], inp["v"], inp["do"], nq, nk)
    o, lse = sa.sigattn_softmax_fwd(dq_, dk_, dv_, dnq, dnk, w.alpha)
    gq, gk, gv = sa.sigattn_softmax_bwd(dq_, dk_, dv_, o, ddo, lse, dnq, dnk, w.alpha)
    torch.cuda.synchronize()
    outs = {"O": o, "dQ": gq, "dK": gk, "dV": gv}
    assert all(bool(torch.isfinite(t).all()) for t in outs.values()), f"{name}: non-finite output"
    Q, K, V, DO = (t.float().numpy() for t in (inp["q"], inp["k"], inp["v"], inp["do"]))
    rng = np.random.default_rng(4321)
    got = {k: [] for k in outs}
    ref = {k: [] for k in outs}
    lse_d = 0.0
    for z in range(w.Z):
        qrows = _sample_rows(int(nq[z]), w.L, rng)
        krows = _sample_rows(int(nk[z]), w.L, rng)
        for h in sorted({0, w.H - 1}):
            o_ref, lse_ref = SM.forward_rows(Q, K, V, nq, nk, w.alpha, z, h, qrows)
            dq_ref, dk_ref, dv_ref = SM.backward_rows(Q, K, V, DO, nq, nk, w.alpha, z, h, qrows, krows)
            lse_g = lse[z, torch.as_tensor(qrows, device="cuda"), h].cpu().numpy().astype(np.float64)
            lse_d = max(lse_d, float(np.max(np.abs(lse_g - lse_ref))))
            for key, rows, r in (("O", qrows, o_ref), ("dQ", qrows, dq_ref), ("dK", krows, dk_ref),
                                 ("dV", krows, dv_ref)):
                g = outs[key][z, torch.as_tensor(rows, device="cuda"), h].float().cpu().numpy().astype(np.float64)
                pad = rows >= (nq[z] if key in ("O", "dQ") else nk[z])
                assert np.all(g[pad] == 0.0), f"{name}: {key} padded sampled row not exactly 0 (z={z})"
                got[key].append(g)
                ref[key].append(r)
    for key in outs:
        e = rel_err(np.concatenate(got[key]), np.concatenate(ref[key]))
        assert e <= TOL["bf16"], f"{name}: softmax {key} sampled rel err {e:.3e}"
    assert lse_d <= LSE_TOL["bf16"], f"{name}: softmax LSE err {lse_d:.3e}"
    del dq_, dk_, dv_, ddo, o, gq, gk, gv
    torch.cuda.empty_cache()


@pytest.mark.parametrize("D", [64, 128])
def test_softmax_scores_that_keep_growing(D):
    """Scores rise along the keys, by about 7.7 per 32-key block (11 in log2
    units), so a block's maximum usually lies far above the forward's running
    reference: such blocks force its lazy rescale while the previous block's
    P still waits for its P V MFMAs, and that P must be rescaled with O and
    the row sum. One sample is cut at n_k = 200 so the masked tail takes part.
    O and LSE are held to the usual bounds. The gradients are held to 2^-7 of
    the sum of their terms' absolute values (4 bf16 unit roundoffs, the bf16
    counterpart of the fp32 bound above): with keys this close to one common
    direction, dS K cancels almost completely (the rows of dS sum to 0), so a
    bound relative to the result would measure that cancellation, not the
    kernels. The backward recomputes P from LSE and has no running maximum."""
    import padding_aware_sigmoid_amd as sa

    Z, L, H = 2, 256, 1
    nq, nk = [256, 256], [256, 200]
    note(f"softmax growing scores D={D}")
    g = torch.Generator().manual_seed(71)
    q = torch.full((Z, L, H, D), 0.5)
    # key j: components t_j + 0.1 N(0, 1), t_j = 0.24 j / D, so q.k_j is about 0.12 j
    t = 0.24 * torch.arange(L, dtype=torch.float32) / D
    k = t[None, :, None, None] + 0.1 * torch.randn(Z, L, H, D, generator=g)
    v = torch.randn(Z, L, H, D, generator=g)
    do = torch.randn(Z, L, H, D, generator=g)
    q, k, v, do = (x.to(torch.bfloat16) for x in (q, k, v, do))
    dq_, dk_, dv_, ddo, dnq, dnk = device_inputs(q, k, v, do, nq, nk)
    alpha = 2.0
    Q, K, V, DO = (f64(x) for x in (q, k, v, do))
    # the blocks whose maximum rises past the rescale threshold (8 in log2 units)
    blk = (alpha * (Q[0, 0, 0] @ K[0, :, 0].T) * np.log2(np.e)).reshape(-1, 32).max(axis=1)
    rises = int(np.sum(np.diff(np.maximum.accumulate(blk)) > 8.0))
    assert rises >= 4, f"only {rises} blocks rise past the rescale threshold"
    o, lse = sa.sigattn_softmax_fwd(dq_, dk_, dv_, dnq, dnk, alpha)
    gq, gk, gv = sa.sigattn_softmax_bwd(dq_, dk_, dv_, o, ddo, lse, dnq, dnk, alpha)
    torch.cuda.synchronize()
    ro, rlse = SM.forward(Q, K, V, nq, nk, alpha)
    rq, rk, rv = SM.backward(Q, K, V, DO, nq, nk, alpha)
    e = rel_err(host(o), ro)
    assert e <= TOL["bf16"], f"O: rel err {e:.3e}"
    e = _lse_err(lse.cpu().numpy().astype(np.float64), rlse.transpose(0, 2, 1), "bf16")
    assert e <= LSE_TOL["bf16"], f"LSE err {e:.3e}"
    scales = _abs_term_scales(Q, K, V, DO, nq, nk, alpha)
    for name, got, ref in (("dQ", gq, rq), ("dK", gk, rk), ("dV", gv, rv)):
        d = float(np.max(np.abs(host(got) - ref)))
        assert d <= 2.0**-7 * scales[name], f"{name}: max abs err {d:.3e} > {2.0**-7 * scales[name]:.3e}"
