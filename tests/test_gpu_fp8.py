"""The FP8 path on the GPU against the FP8 oracle (oracle.fp8_attention).

* Quantisation: E4M3 codes and E8M0 tile scale bytes bit for bit (both sides
  decide each code from the same exact value, x * 2^-E with x in bf16), in
  the padded and the packed layout, D = 64 and 128, ragged lengths, empty
  samples.
* Forward: O against the oracle's quantised forward on the same codes,
  max|GPU - oracle| / max|oracle| <= 2e-2. The two sides differ only where
  fp32 and fp64 scores put a P on opposite sides of an E4M3 rounding boundary
  (one code step, rare), and in the bf16 rounding of O (2^-8 relative).
* Distance to exact attention. The FP8 oracle encodes this library's own
  quantisation design (the pages fix no FP8 scheme), so the GPU output is
  also held, element by element, to a bound derived from the format against
  the unquantised sigmoid attention of the same (dequantised) Q, K and V:
    |O - O_exact| <= (2^-4 + 2^-12) sum_j P_j |V_j|      E4M3 relative step of P
                   + 2^-16 max_j P_j sum_j |V_j|         subnormal tail of P's tile
                   + 2^-8 |O_exact| + 2^-20 max|O_exact|  bf16 rounding of O, fp32 sums
  P_j from the sigmoid oracle. The E4M3 half-step is 2^-4 relative for
  normal codes; below the smallest normal (2^-6 after the tile's scale 2^e,
  e <= log2 max P - 7) the half-step is 2^-10 * 2^e <= 2^-17 max P, doubled
  in case fp32 and fp64 put the tile's maximum on opposite sides of a power
  of two. 2^-12 covers the fp32 scores and weights, 2^-8 the bf16 output.
  Every FP8 test case and the full-size rows are held to it.
* Padded rows of O are exactly 0; padded input rows (NaN here) are never
  read; the packed layout equals the padded one bit for bit.
* At the 16K bench size, sampled rows against the oracle's row function.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import device_inputs, f64, host, note, rel_err

pytestmark = pytest.mark.gpu

F8 = oracle.fp8_attention
TOL = 2e-2

CASES = [
    # (label, Z, L, H, D, nq, nk)
    ("d64", 3, 300, 2, 64, [300, 131, 7], [250, 131, 40]),
    ("d128", 3, 333, 2, 128, [333, 0, 200], [100, 5, 333]),
    ("d128-tail", 2, 260, 1, 128, [260, 90], [1, 260]),
]


def _packed(t, n):
    return torch.cat([t[z, : int(n[z])] for z in range(t.shape[0])], 0).contiguous()


def _cu(n):
    return np.concatenate([[0], np.cumsum(np.asarray(n, np.int64))]).astype(np.int32)


@pytest.mark.parametrize("label,Z,L,H,D,nq,nk", CASES)
def test_quantize_bit_exact(label, Z, L, H, D, nq, nk):
    import padding_aware_sigmoid_amd as sa

    note(f"fp8 quantize {label} n={nq}")
    q, k, v, do = workloads.make_tensors(Z, L, H, D, "bf16", seed=41)
    x = q * torch.exp(torch.linspace(-8, 8, H)).to(torch.bfloat16)[None, None, :, None]  # spread the tile ranges
    dx, _, _, _, dn, _ = device_inputs(x, k, v, do, nq, nk)
    codes, sc = sa.sigattn_quantize_fp8(dx, dn)
    torch.cuda.synchronize()
    c_ref, s_ref = F8.quantize(f64(x), nq)
    assert np.array_equal(sc.cpu().numpy(), s_ref), f"{label}: scale bytes differ"
    got = codes.cpu().numpy()
    bad = np.argwhere(got != c_ref)
    assert bad.size == 0, f"{label}: {len(bad)} codes differ, first at {bad[0].tolist()}"
    # packed: the same codes for the valid rows, the same scale bytes
    xp = _packed(dx, nq)
    cp, sp = sa.sigattn_quantize_fp8(xp, torch.as_tensor(_cu(nq)).to(dx.device), max_len=L)
    torch.cuda.synchronize()
    assert torch.equal(cp, _packed(codes, nq)), f"{label}: packed codes differ"
    assert torch.equal(sp, sc), f"{label}: packed scale bytes differ"


def _quantized(dq_, dk_, dv_, dnq, dnk):
    import padding_aware_sigmoid_amd as sa

    q8, sq = sa.sigattn_quantize_fp8(dq_, dnq)
    k8, sk = sa.sigattn_quantize_fp8(dk_, dnk)
    v8, sv = sa.sigattn_quantize_fp8(dv_, dnk)
    return q8, k8, v8, sq, sk, sv


@pytest.mark.parametrize("bias_mode", ["constant", "neg_log_nk"])
@pytest.mark.parametrize("label,Z,L,H,D,nq,nk", CASES)
def test_fp8_forward_matches_oracle(label, Z, L, H, D, nq, nk, bias_mode):
    import padding_aware_sigmoid_amd as sa

    note(f"fp8 forward {label} {bias_mode} nq={nq} nk={nk}")
    q, k, v, do = workloads.make_tensors(Z, L, H, D, "bf16", seed=42)
    dq_, dk_, dv_, _, dnq, dnk = device_inputs(q, k, v, do, nq, nk)
    alpha = 1.0 / np.sqrt(D)
    bias = -np.log(L) if bias_mode == "constant" else 0.0
    q8, k8, v8, sq, sk, sv = _quantized(dq_, dk_, dv_, dnq, dnk)
    o = sa.sigattn_fwd_fp8(q8, k8, v8, sq, sk, sv, dnq, dnk, alpha, bias, bias_mode=bias_mode)
    torch.cuda.synchronize()
    b = bias if bias_mode == "constant" else oracle.per_sample_bias(nk, bias)
    args = [t.cpu().numpy() for t in (q8, k8, v8, sq, sk, sv)]
    ref = F8.forward(*args, nq, nk, alpha, b)
    got = host(o)
    e = rel_err(got, ref)
    assert e <= TOL, f"{label} {bias_mode}: O rel err {e:.3e} > {TOL}"
    for z in range(Z):
        assert np.all(got[z, nq[z]:] == 0.0), f"{label}: padded rows of sample {z} not exactly 0"
    # distance to exact attention of the dequantised operands, element by element
    Qd, Kd, Vd = (F8.dequantize(c, sc) for c, sc in ((args[0], args[3]), (args[1], args[4]), (args[2], args[5])))
    exact = oracle.forward(Qd, Kd, Vd, nq, nk, alpha, b)
    spv = oracle.forward(Qd, Kd, np.abs(Vd), nq, nk, alpha, b)
    psum = oracle.forward(Qd, Kd, np.ones_like(Vd), nq, nk, alpha, b)
    sv_abs = np.zeros_like(Vd)
    for z in range(Z):
        sv_abs[z, :] = np.abs(Vd[z, : nk[z]]).sum(axis=0)[None]
    _assert_within_e4m3_bound(got, exact, spv, psum, sv_abs, f"{label} {bias_mode}")
    # for the record: the distance to the sigmoid forward on the bf16 inputs
    full = oracle.forward(f64(q), f64(k), f64(v), nq, nk, alpha, b)
    note(f"  vs oracle fp8 {e:.2e}; fp8 oracle vs bf16-input oracle {rel_err(ref, full):.2e}")


def test_fp8_padding_is_never_read():
    import padding_aware_sigmoid_amd as sa

    note("fp8 NaN padding")
    Z, L, H, D = 2, 300, 2, 128
    nq, nk = [300, 140], [170, 300]
    q, k, v, do = workloads.make_tensors(Z, L, H, D, "bf16", seed=43)
    dq_, dk_, dv_, _, dnq, dnk = device_inputs(q, k, v, do, nq, nk)
    outs = []
    for poison in (False, True):
        tq, tk, tv = (t.clone() for t in (dq_, dk_, dv_))
        if poison:
            for z in range(Z):
                tq[z, nq[z]:] = float("nan")
                tk[z, nk[z]:] = float("nan")
                tv[z, nk[z]:] = float("nan")
        q8, k8, v8, sq, sk, sv = _quantized(tq, tk, tv, dnq, dnk)
        if poison:  # the forward must not read padded code rows either
            for z in range(Z):
                q8[z, nq[z]:] = 0x7F
                k8[z, nk[z]:] = 0x7F
                v8[z, nk[z]:] = 0x7F
        o = sa.sigattn_fwd_fp8(q8, k8, v8, sq, sk, sv, dnq, dnk)
        torch.cuda.synchronize()
        outs.append(o)
    assert torch.equal(outs[0], outs[1]), "the FP8 forward changed when padding held NaN"


@pytest.mark.parametrize("label,Z,L,H,D,nq,nk", CASES)
def test_fp8_packed_matches_padded(label, Z, L, H, D, nq, nk):
    import padding_aware_sigmoid_amd as sa

    note(f"fp8 packed {label}")
    q, k, v, do = workloads.make_tensors(Z, L, H, D, "bf16", seed=44)
    dq_, dk_, dv_, _, dnq, dnk = device_inputs(q, k, v, do, nq, nk)
    q8, k8, v8, sq, sk, sv = _quantized(dq_, dk_, dv_, dnq, dnk)
    o = sa.sigattn_fwd_fp8(q8, k8, v8, sq, sk, sv, dnq, dnk)
    cq = torch.as_tensor(_cu(nq)).to(dq_.device)
    ck = torch.as_tensor(_cu(nk)).to(dq_.device)
    o_p = sa.sigattn_fwd_fp8(_packed(q8, nq), _packed(k8, nk), _packed(v8, nk), sq, sk, sv, cq, ck, max_len=L)
    torch.cuda.synchronize()
    assert torch.equal(o_p, _packed(o, nq)), f"{label}: packed O differs from padded O"


def _assert_within_e4m3_bound(got, exact, spv, pmax, sv_abs, what):
    """got, exact, spv (sum_j P_j |V_j|), pmax (an upper bound of max_j P_j,
    here sum_j P_j), sv_abs (sum_j |V_j|), all of one shape."""
    bound = (2.0**-4 + 2.0**-12) * spv + 2.0**-16 * pmax * sv_abs + 2.0**-8 * np.abs(exact) \
        + 2.0**-20 * float(np.max(np.abs(exact), initial=0.0))
    excess = np.abs(got - exact) - bound
    worst = np.unravel_index(int(np.argmax(excess)), excess.shape) if excess.size else None
    assert excess.size == 0 or excess[worst] <= 0.0, (
        f"{what}: FP8 output beyond the E4M3 bound of exact attention at {worst}: "
        f"|diff| {abs(got[worst] - exact[worst]):.3e} > bound {bound[worst]:.3e}")
    rel = float(np.max(np.abs(got - exact)) / max(np.max(np.abs(exact)), 1e-300))
    note(f"  {what}: max|FP8 - exact| / max|exact| = {rel:.2e}, worst bound use "
         f"{float(np.max(np.abs(got - exact) / np.maximum(bound, 1e-300))):.2f}")


def _sample_rows(n, L, rng):
    fixed = [0, 1, 63, 64, 127, 128, 255, 256, n - 1, n, n + 1, L - 1]
    extra = rng.integers(0, max(1, n), 4).tolist() if n > 0 else []
    return np.array(sorted({r for r in fixed + extra if 0 <= r < L}), dtype=np.int64)


@pytest.mark.parametrize("name", ["nopad16k", "pad25_16k"])
def test_fp8_fullsize_sampled(name):
    import padding_aware_sigmoid_amd as sa

    inp = workloads.make_inputs(name, seed=45)
    w = inp["workload"]
    nq, nk = inp["seqlens_q"], inp["seqlens_k"]
    note(f"fp8 full-size {name} Z={w.Z} L={w.L} H={w.H} D={w.D}")
    dq_, dk_, dv_, _, dnq, dnk = device_inputs(inp["q"], inp["k"], inp["v"], inp["do"], nq, nk)
    q8, k8, v8, sq, sk, sv = _quantized(dq_, dk_, dv_, dnq, dnk)
    o = sa.sigattn_fwd_fp8(q8, k8, v8, sq, sk, sv, dnq, dnk, w.alpha, w.bias)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()), f"{name}: non-finite output"
    args = [t.cpu().numpy() for t in (q8, k8, v8, sq, sk, sv)]
    del dq_, dk_, dv_
    rng = np.random.default_rng(5432)
    got, ref, exact, spv, psum, svs = [], [], [], [], [], []
    for z in range(w.Z):
        rows = _sample_rows(int(nq[z]), w.L, rng)
        # dequantised operands of sample z, for exact attention on the sampled rows
        Qz, Kz, Vz = (F8.dequantize(c[z:z + 1], sc[z:z + 1]) for c, sc in ((args[0], args[3]), (args[1], args[4]),
                                                                           (args[2], args[5])))
        nqz, nkz = np.array([nq[z]]), np.array([nk[z]])
        for h in sorted({0, w.H - 1}):
            r = F8.forward_rows(*args, nq, nk, w.alpha, w.bias, z, h, rows)
            g = o[z, torch.as_tensor(rows, device="cuda"), h].float().cpu().numpy().astype(np.float64)
            assert np.all(g[rows >= nq[z]] == 0.0), f"{name}: padded sampled row not 0 (z={z})"
            got.append(g)
            ref.append(r)
            exact.append(oracle.forward_rows(Qz, Kz, Vz, nqz, nkz, w.alpha, w.bias, 0, h, rows))
            spv.append(oracle.forward_rows(Qz, Kz, np.abs(Vz), nqz, nkz, w.alpha, w.bias, 0, h, rows))
            psum.append(oracle.forward_rows(Qz, Kz, np.ones_like(Vz), nqz, nkz, w.alpha, w.bias, 0, h, rows))
            svs.append(np.broadcast_to(np.abs(Vz[0, : nk[z], h]).sum(axis=0), (len(rows), w.D)))
    e = rel_err(np.concatenate(got), np.concatenate(ref))
    assert e <= TOL, f"{name}: fp8 sampled rel err {e:.3e}"
    _assert_within_e4m3_bound(*(np.concatenate(x) for x in (got, exact, spv, psum, svs)), name)
    del o, q8, k8, v8
    torch.cuda.empty_cache()
