"""Properties of the GPU path that must hold exactly.

* Skip decisions: the kernels' tile counters equal the oracle's tile plan.
* Padded rows of every output are exactly 0.
* Valid outputs are bitwise identical when the padding holds garbage, NaN or
  Inf, and when L grows.
* Two runs give bitwise identical results (no atomics).
* Empty inputs are no-ops. Invalid arguments give error codes, not faults.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import device_inputs, note

pytestmark = pytest.mark.gpu


def _fwd_bwd(q, k, v, do, nq, nk, alpha, bias, counters=False):
    import padding_aware_sigmoid_amd as sa

    Z, L, H, D = q.shape
    tc = {}
    if counters:
        for name, kern, axis in (("fwd", sa.KERNEL_FWD, 0), ("dq", sa.KERNEL_DQ, 0), ("dkdv", sa.KERNEL_DKDV, 1)):
            bq, bk = sa.sigattn_tile_config(kern, D, q.dtype)
            ntiles = -(-L // (bq if axis == 0 else bk))
            tc[name] = torch.full((Z * H * ntiles,), -7, dtype=torch.int32, device=q.device)
    o = sa.sigattn_fwd(q, k, v, nq, nk, alpha, bias, tile_counts=tc.get("fwd"))
    g = sa.sigattn_bwd(q, k, v, do, nq, nk, alpha, bias, tile_counts_dq=tc.get("dq"),
                       tile_counts_dkdv=tc.get("dkdv"))
    torch.cuda.synchronize()
    return o, g, tc


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 128), ("fp32", 64)])
def test_tile_counters_match_oracle_plan(dtype, D):
    import padding_aware_sigmoid_amd as sa

    Z, L, H = 5, 520, 2
    n_q = np.array([520, 0, 1, 129, 384])
    n_k = np.array([64, 520, 300, 0, 385])
    note(f"tile counters dtype={dtype} D={D}")
    q, k, v, do = workloads.make_tensors(Z, L, H, D, dtype, seed=3)
    args = device_inputs(q, k, v, do, n_q, n_k)
    _, _, tc = _fwd_bwd(*args, 1 / math.sqrt(D), -math.log(L), counters=True)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    for name, kern in (("fwd", sa.KERNEL_FWD), ("dq", sa.KERNEL_DQ), ("dkdv", sa.KERNEL_DKDV)):
        bq, bk = sa.sigattn_tile_config(kern, D, tdt)
        by_q, by_k = oracle.tile_plan(n_q, n_k, L, bq, bk)
        want = by_q if name != "dkdv" else by_k
        got = tc[name].cpu().numpy().reshape(Z, H, -1)
        for h in range(H):
            assert np.array_equal(got[:, h, :], want), f"{name}: skip decisions differ from the oracle plan"


@pytest.mark.parametrize("fill", ["garbage", "nan", "inf"])
def test_padding_contents_never_matter(fill):
    Z, L, H, D = 3, 300, 2, 128
    n = np.array([300, 77, 200])
    note(f"padding fill={fill}")
    q, k, v, do = workloads.make_tensors(Z, L, H, D, "bf16", seed=4)
    base = _fwd_bwd(*device_inputs(q, k, v, do, n, n), 1 / math.sqrt(D), -math.log(L))
    val = {"garbage": 1e4, "nan": float("nan"), "inf": float("inf")}[fill]
    q2, k2, v2, do2 = (t.clone() for t in (q, k, v, do))
    for z in range(Z):
        for t in (q2, k2, v2, do2):
            t[z, int(n[z]):] = val
    other = _fwd_bwd(*device_inputs(q2, k2, v2, do2, n, n), 1 / math.sqrt(D), -math.log(L))
    assert torch.equal(base[0], other[0]), "O changed with the padding contents"
    for a, b in zip(base[1], other[1]):
        assert torch.equal(a, b), "a gradient changed with the padding contents"


@pytest.mark.parametrize("bias_mode", ["constant", "neg_log_nk"])
@pytest.mark.parametrize("qk_scale", [1.0, 0.5])
def test_growing_L_is_bitwise_invariant(bias_mode, qk_scale):
    """Valid outputs do not change when L grows. At score scale 0.5 the
    forward's workgroups take the one-transcendental sigma, at 1 most of them
    the exact one (their first block has scores above its range)."""
    import padding_aware_sigmoid_amd as sa

    Z, L, H, D = 2, 256, 2, 64
    n = np.array([256, 100])
    note(f"growing L {bias_mode} scale={qk_scale}")
    q, k, v, do = workloads.make_tensors(Z, L, H, D, "bf16", seed=6, qk_scale=qk_scale)
    alpha, bias = 0.125, (-math.log(256) if bias_mode == "constant" else 0.0)

    def run(q, k, v, do):
        dq_, dk_, dv_, ddo, dn, _ = device_inputs(q, k, v, do, n, n)
        o = sa.sigattn_fwd(dq_, dk_, dv_, dn, dn, alpha, bias, bias_mode=bias_mode)
        g = sa.sigattn_bwd(dq_, dk_, dv_, ddo, dn, dn, alpha, bias, bias_mode=bias_mode)
        torch.cuda.synchronize()
        return o, g

    a = run(q, k, v, do)
    grow = lambda t: torch.cat([t, torch.randn(Z, 70, H, D).to(t.dtype)], dim=1)  # noqa: E731
    b = run(grow(q), grow(k), grow(v), grow(do))
    assert torch.equal(a[0], b[0][:, :L]) and torch.all(b[0][:, L:] == 0)
    for x, y in zip(a[1], b[1]):
        assert torch.equal(x, y[:, :L]) and torch.all(y[:, L:] == 0)


def test_bitwise_deterministic():
    Z, L, H, D = 2, 400, 2, 128
    n = np.array([400, 250])
    note("determinism")
    q, k, v, do = workloads.make_tensors(Z, L, H, D, "bf16", seed=7)
    args = device_inputs(q, k, v, do, n, n)
    a = _fwd_bwd(*args, 1 / math.sqrt(D), -math.log(L))
    b = _fwd_bwd(*args, 1 / math.sqrt(D), -math.log(L))
    assert torch.equal(a[0], b[0])
    for x, y in zip(a[1], b[1]):
        assert torch.equal(x, y)


def test_lengths_are_clamped():
    """Lengths below 0 act as 0, lengths above L act as L."""
    Z, L, H, D = 2, 128, 1, 64
    note("length clamping")
    q, k, v, do = workloads.make_tensors(Z, L, H, D, "bf16", seed=8)
    a = _fwd_bwd(*device_inputs(q, k, v, do, np.array([-5, 999]), np.array([L + 1, -1])), 0.125, -4.0)
    b = _fwd_bwd(*device_inputs(q, k, v, do, np.array([0, L]), np.array([L, 0])), 0.125, -4.0)
    assert torch.equal(a[0], b[0])
    for x, y in zip(a[1], b[1]):
        assert torch.equal(x, y)


def test_empty_and_errors():
    import padding_aware_sigmoid_amd as sa
    from padding_aware_sigmoid_amd import _lib

    lib = _lib.load()
    note("empty inputs and error codes")
    # An empty batch is a successful no-op.
    e = torch.empty(0, 16, 2, 64, dtype=torch.bfloat16, device="cuda")
    n0 = torch.empty(0, dtype=torch.int32, device="cuda")
    o = sa.sigattn_fwd(e, e, e, n0, n0)
    assert o.shape == e.shape
    g = sa.sigattn_bwd(e, e, e, e, n0, n0)
    assert all(t.shape == e.shape for t in g)
    # Error codes: bad D, bad dtype, NULL tensor, misaligned pointer.
    x = torch.zeros(1, 8, 1, 64, dtype=torch.bfloat16, device="cuda")
    n = torch.full((1,), 8, dtype=torch.int32, device="cuda")
    p = x.data_ptr()
    assert lib.sigattn_fwd(p, p, p, p, n.data_ptr(), n.data_ptr(), 1, 8, 1, 96, 1.0, 0.0, 0, None, None) == -1
    assert lib.sigattn_fwd(p, p, p, p, n.data_ptr(), n.data_ptr(), 1, 8, 1, 64, 1.0, 0.0, 7, None, None) == -2
    assert lib.sigattn_fwd(None, p, p, p, n.data_ptr(), n.data_ptr(), 1, 8, 1, 64, 1.0, 0.0, 0, None,
                           None) == -1
    assert lib.sigattn_fwd(p + 2, p, p, p, n.data_ptr(), n.data_ptr(), 1, 8, 1, 64, 1.0, 0.0, 0, None,
                           None) == -1
    assert lib.sigattn_fwd(p, p, p, p, n.data_ptr(), n.data_ptr(), 1, 8, 1, 64, float("nan"), 0.0, 0, None,
                           None) == -1
    torch.cuda.synchronize()
    # Outputs are fully written even where the caller left garbage in them.
    q, k, v, do = workloads.make_tensors(1, 96, 1, 64, "bf16", seed=9)
    dq_, dk_, dv_, ddo, dnq, dnk = device_inputs(q, k, v, do, [50], [30])
    out = torch.full_like(dq_, float("nan"))
    sa.sigattn_fwd(dq_, dk_, dv_, dnq, dnk, out=out)
    torch.cuda.synchronize()
    assert torch.all(torch.isfinite(out)) and torch.all(out[:, 50:] == 0)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("D", [64, 128])
def test_split_backward_entry_points_match(dtype, D):
    """sigattn_bwd_dkdv + sigattn_bwd_dq, and sigattn_bwd_dk + sigattn_bwd_dv,
    give exactly what sigattn_bwd gives, counters included."""
    import padding_aware_sigmoid_amd as sa

    Z, L, H = 2, 300, 2
    n = np.array([300, 123])
    note(f"split backward entry points {dtype} D={D}")
    q, k, v, do = workloads.make_tensors(Z, L, H, D, dtype, seed=10)
    dq_, dk_, dv_, ddo, dn, _ = device_inputs(q, k, v, do, n, n)
    _, bk = sa.sigattn_tile_config(sa.KERNEL_DKDV, D, dq_.dtype)
    ntk = Z * H * (-(-L // bk))
    c0, c1, c2 = (torch.full((ntk,), -7, dtype=torch.int32, device=dq_.device) for _ in range(3))
    a = sa.sigattn_bwd(dq_, dk_, dv_, ddo, dn, dn, tile_counts_dkdv=c0)
    gk, gv = sa.sigattn_bwd_dkdv(dq_, dk_, dv_, ddo, dn, dn)
    gq = sa.sigattn_bwd_dq(dq_, dk_, dv_, ddo, dn, dn)
    hk = sa.sigattn_bwd_dk(dq_, dk_, dv_, ddo, dn, dn, tile_counts_dkdv=c1)
    hv = sa.sigattn_bwd_dv(dq_, dk_, ddo, dn, dn, tile_counts_dkdv=c2)
    torch.cuda.synchronize()
    assert torch.equal(a[0], gq) and torch.equal(a[1], gk) and torch.equal(a[2], gv)
    assert torch.equal(a[1], hk) and torch.equal(a[2], hv)
    assert torch.equal(c0, c1) and torch.equal(c0, c2) and int(c0.min()) >= 0


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("bias_mode", ["constant", "neg_log_nk"])
def test_autograd_matches_entry_points_and_oracle(dtype, bias_mode):
    """sigmoid_attention (the autograd wrapper over the padded layout): its
    forward and its gradients equal sigattn_fwd / sigattn_bwd bit for bit,
    with the default alpha = 1/sqrt(D) and bias (-ln L for one bias; b_z =
    -ln n_k[z] per sample), and both match the oracle."""
    import padding_aware_sigmoid_amd as sa

    from gpu_util import host, rel_err

    Z, L, H, D = 3, 200, 2, 64
    n = np.array([200, 77, 0])
    note(f"padded autograd {dtype} {bias_mode}")
    q, k, v, do = workloads.make_tensors(Z, L, H, D, dtype, seed=31)
    dq_, dk_, dv_, ddo, dn, _ = device_inputs(q, k, v, do, n, n)
    leaves = [t.clone().requires_grad_(True) for t in (dq_, dk_, dv_)]
    o = sa.sigmoid_attention(*leaves, dn, dn, bias_mode=bias_mode)
    o.backward(ddo)
    # the wrapper's defaults: bias = -ln L for one bias, 0 (so b_z = -ln n_k[z]) per sample
    alpha, bias = 1 / math.sqrt(D), (-math.log(L) if bias_mode == "constant" else 0.0)
    o2 = sa.sigattn_fwd(dq_, dk_, dv_, dn, dn, alpha, bias, bias_mode=bias_mode)
    g2 = sa.sigattn_bwd(dq_, dk_, dv_, ddo, dn, dn, alpha, bias, bias_mode=bias_mode)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o2)
    for leaf, g in zip(leaves, g2):
        assert torch.equal(leaf.grad, g)
    Q, K, V, DO = (workloads.to_f64(t) for t in (q, k, v, do))
    if bias_mode == "constant":
        ref_o = oracle.forward(Q, K, V, n, n, alpha, bias)
        ref_g = oracle.backward(Q, K, V, DO, n, n, alpha, bias)
    else:
        b = oracle.per_sample_bias(n, bias)
        ref_o = oracle.forward(Q, K, V, n, n, alpha, b)
        ref_g = oracle.backward(Q, K, V, DO, n, n, alpha, b)
    tol = 2e-2 if dtype == "bf16" else 1e-5
    for name, got, ref in zip(("O", "dQ", "dK", "dV"), (o2, *g2), (ref_o, *ref_g)):
        g = host(got)
        err = rel_err(g, ref)
        assert err <= tol, f"{name}: {err:.3e} > {tol}"
        assert np.all(g[1, 77:] == 0.0) and np.all(g[2] == 0.0), f"{name}: padded rows not 0"
