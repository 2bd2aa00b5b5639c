"""Per-sample bias (b_z = bias - ln n_k[z]) and the packed (varlen) layout on the GPU.

* Both against the CPU oracle (per_sample_bias, forward_varlen,
  backward_varlen), bf16 (2e-2) and fp32 (1e-5), D = 64 and 128.
* The packed layout against the padded one, bit for bit: the kernels run the
  same arithmetic on the same rows, only the row addresses differ. The tile
  counters must agree too.
* The packed layout writes every row of every output and nothing else: the
  rows around a tensor that is a slice of a larger buffer stay untouched.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import assert_padding_zero, device_inputs, f64, host, note, rel_err

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
FP32_TOL = 1e-5


def _packed(t, n):
    return torch.cat([t[z, : int(n[z])] for z in range(t.shape[0])], 0).contiguous()


def _cu(n):
    return np.concatenate([[0], np.cumsum(np.asarray(n, np.int64))]).astype(np.int32)


CASES = [
    # (label, dtype, Z, L, H, D, nq, nk)
    ("bf16-d64", "bf16", 3, 300, 2, 64, [300, 131, 7], [250, 131, 40]),
    ("bf16-d128", "bf16", 3, 333, 2, 128, [333, 0, 200], [100, 5, 333]),
    ("fp32-d64", "fp32", 2, 200, 2, 64, [200, 77], [150, 200]),
    ("fp32-d128", "fp32", 2, 130, 1, 128, [65, 130], [130, 1]),
    # lengths on both sides of the fused dK/dV kernel's 128-row passes and
    # 256-row workgroup tiles (a second pass wholly in padding: 1, 127, 128)
    ("bf16-d128-passes", "bf16", 6, 400, 1, 128, [1, 127, 128, 129, 256, 385], [385, 256, 129, 128, 127, 1]),
    ("bf16-d64-passes", "bf16", 6, 400, 1, 64, [1, 127, 128, 129, 256, 385], [385, 256, 129, 128, 127, 1]),
]


@pytest.mark.parametrize("label,dtype,Z,L,H,D,nq,nk", CASES)
def test_per_sample_bias_matches_oracle(label, dtype, Z, L, H, D, nq, nk):
    import padding_aware_sigmoid_amd as sa

    note(f"per-sample bias {label} nq={nq} nk={nk}")
    q, k, v, do = workloads.make_tensors(Z, L, H, D, dtype, seed=21)
    dq_, dk_, dv_, ddo, dnq, dnk = device_inputs(q, k, v, do, nq, nk)
    alpha, bias = 1.0 / np.sqrt(D), 0.25
    o = sa.sigattn_fwd(dq_, dk_, dv_, dnq, dnk, alpha, bias, bias_mode="neg_log_nk")
    g = sa.sigattn_bwd(dq_, dk_, dv_, ddo, dnq, dnk, alpha, bias, bias_mode="neg_log_nk")
    torch.cuda.synchronize()
    Q, K, V, DO = (f64(t) for t in (q, k, v, do))
    bz = oracle.per_sample_bias(nk, bias)
    refs = (oracle.forward(Q, K, V, nq, nk, alpha, bz),) + oracle.backward(Q, K, V, DO, nq, nk, alpha, bz)
    tol = BF16_TOL if dtype == "bf16" else FP32_TOL
    for name, got, ref in zip(("O", "dQ", "dK", "dV"), (o,) + tuple(g), refs):
        e = rel_err(host(got), ref)
        assert e <= tol, f"{label}: {name} rel err {e:.3e} > {tol}"
    assert_padding_zero("O", host(o), nq)
    assert_padding_zero("dK", host(g[1]), nk)


@pytest.mark.parametrize("bias_mode", ["constant", "neg_log_nk"])
@pytest.mark.parametrize("label,dtype,Z,L,H,D,nq,nk", CASES)
def test_packed_matches_oracle_and_padded(label, dtype, Z, L, H, D, nq, nk, bias_mode):
    import padding_aware_sigmoid_amd as sa

    note(f"packed {label} bias_mode={bias_mode} nq={nq} nk={nk}")
    q, k, v, do = workloads.make_tensors(Z, L, H, D, dtype, seed=22)
    dq_, dk_, dv_, ddo, dnq, dnk = device_inputs(q, k, v, do, nq, nk)
    alpha, bias = 1.0 / np.sqrt(D), (-np.log(L) if bias_mode == "constant" else 0.0)
    cnt = {}
    for kern, axis in ((sa.KERNEL_FWD, 0), (sa.KERNEL_DQ, 0), (sa.KERNEL_DKDV, 1)):
        bq, bk = sa.sigattn_tile_config(kern, D, dq_.dtype)
        ntl = Z * H * -(-L // (bq if axis == 0 else bk))
        cnt[kern] = [torch.full((ntl,), -7, dtype=torch.int32, device=dq_.device) for _ in range(2)]
    # padded
    o_pad = sa.sigattn_fwd(dq_, dk_, dv_, dnq, dnk, alpha, bias, tile_counts=cnt[sa.KERNEL_FWD][0], bias_mode=bias_mode)
    g_pad = sa.sigattn_bwd(dq_, dk_, dv_, ddo, dnq, dnk, alpha, bias, tile_counts_dq=cnt[sa.KERNEL_DQ][0],
                           tile_counts_dkdv=cnt[sa.KERNEL_DKDV][0], bias_mode=bias_mode)
    # packed
    qp, dop = _packed(dq_, nq), _packed(ddo, nq)
    kp, vp = _packed(dk_, nk), _packed(dv_, nk)
    cq = torch.as_tensor(_cu(nq)).to(dq_.device)
    ck = torch.as_tensor(_cu(nk)).to(dq_.device)
    o_p = sa.sigattn_fwd_varlen(qp, kp, vp, cq, ck, L, alpha, bias, tile_counts=cnt[sa.KERNEL_FWD][1],
                                bias_mode=bias_mode)
    g_p = sa.sigattn_bwd_varlen(qp, kp, vp, dop, cq, ck, L, alpha, bias, tile_counts_dq=cnt[sa.KERNEL_DQ][1],
                                tile_counts_dkdv=cnt[sa.KERNEL_DKDV][1], bias_mode=bias_mode)
    torch.cuda.synchronize()
    # bit for bit against the padded layout on the valid rows
    for name, a, b, n in (("O", o_p, o_pad, nq), ("dQ", g_p[0], g_pad[0], nq), ("dK", g_p[1], g_pad[1], nk),
                          ("dV", g_p[2], g_pad[2], nk)):
        assert torch.equal(a, _packed(b, n)), f"{label}: packed {name} differs from padded {name}"
    for kern in cnt:
        assert torch.equal(cnt[kern][0], cnt[kern][1]), f"{label}: tile counters differ for kernel {kern}"
    # and against the oracle's packed definition
    Qp, Kp, Vp, DOp = (f64(t.cpu()) for t in (qp, kp, vp, dop))
    b = bias if bias_mode == "constant" else oracle.per_sample_bias(nk, bias)
    o_ref = oracle.forward_varlen(Qp, Kp, Vp, _cu(nq), _cu(nk), alpha, b)
    refs = (o_ref,) + oracle.backward_varlen(Qp, Kp, Vp, DOp, _cu(nq), _cu(nk), alpha, b)
    tol = BF16_TOL if dtype == "bf16" else FP32_TOL
    for name, got, ref in zip(("O", "dQ", "dK", "dV"), (o_p,) + tuple(g_p), refs):
        e = rel_err(host(got), ref)
        assert e <= tol, f"{label}: packed {name} rel err {e:.3e} > {tol}"


def test_packed_writes_only_its_rows():
    """Outputs that are views into a larger buffer: the rows before and after stay untouched."""
    import padding_aware_sigmoid_amd as sa

    note("packed writes only its rows")
    Z, L, H, D = 3, 200, 2, 128
    nq = nk = [130, 0, 70]
    q, k, v, do = workloads.make_tensors(Z, L, H, D, "bf16", seed=23)
    dq_, dk_, dv_, ddo, _, _ = device_inputs(q, k, v, do, nq, nk)
    qp, kp, vp, dop = (_packed(t, nq) for t in (dq_, dk_, dv_, ddo))
    T = qp.shape[0]
    cu = torch.as_tensor(_cu(nq)).to(dq_.device)
    bufs = [torch.full((T + 64, H, D), 7.0, dtype=torch.bfloat16, device=dq_.device) for _ in range(4)]
    views = [b[32 : 32 + T] for b in bufs]
    sa.sigattn_fwd_varlen(qp, kp, vp, cu, cu, L, out=views[0])
    sa.sigattn_bwd_varlen(qp, kp, vp, dop, cu, cu, L, dq=views[1], dk=views[2], dv=views[3])
    torch.cuda.synchronize()
    for b in bufs:
        assert torch.all(b[:32] == 7.0) and torch.all(b[32 + T :] == 7.0), "a packed kernel wrote outside its rows"
        assert torch.all(torch.isfinite(b[32 : 32 + T].float()))


def test_varlen_autograd_matches_entry_points():
    import padding_aware_sigmoid_amd as sa

    note("varlen autograd")
    Z, L, H, D = 2, 150, 2, 64
    n = [150, 61]
    q, k, v, do = workloads.make_tensors(Z, L, H, D, "bf16", seed=24)
    dq_, dk_, dv_, ddo, _, _ = device_inputs(q, k, v, do, n, n)
    qp, kp, vp, dop = (_packed(t, n) for t in (dq_, dk_, dv_, ddo))
    cu = torch.as_tensor(_cu(n)).to(dq_.device)
    leaves = [t.clone().requires_grad_(True) for t in (qp, kp, vp)]
    o = sa.sigmoid_attention_varlen(*leaves, cu, cu, L, bias_mode="neg_log_nk")
    o.backward(dop)
    o2 = sa.sigattn_fwd_varlen(qp, kp, vp, cu, cu, L, bias_mode="neg_log_nk")
    g2 = sa.sigattn_bwd_varlen(qp, kp, vp, dop, cu, cu, L, bias_mode="neg_log_nk")
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o2)
    for leaf, g in zip(leaves, g2):
        assert torch.equal(leaf.grad, g)


def test_packed_argument_errors():
    import padding_aware_sigmoid_amd as sa

    note("packed argument errors")
    x = torch.zeros(10, 2, 64, dtype=torch.bfloat16, device="cuda:0")
    cu = torch.tensor([0, 4, 10], dtype=torch.int32, device="cuda:0")
    with pytest.raises(ValueError):
        sa.sigattn_fwd_varlen(x.view(1, 10, 2, 64), x, x, cu, cu, 8)
    with pytest.raises(ValueError):
        sa.sigattn_fwd_varlen(x, x, x, cu, cu[:2], 8)
    with pytest.raises(ValueError):
        sa.sigattn_fwd(x.view(1, 10, 2, 64), x.view(1, 10, 2, 64), x.view(1, 10, 2, 64), [10], [10],
                       bias_mode="neg_log_n")
