"""sigattn_softmax_bwd_noalloc, the entry point that allocates nothing, against
sigattn_softmax_bwd with a caller's workspace: the same kernels on the same
inputs, so dQ, dK and dV must match bit for bit. Two calls in a row, the
second with a smaller input (the fixed buffer keeps the first call's
contents; the second must not depend on them), then a packed-layout call, and
the size limit. Calls go straight through the C ABI."""

import ctypes

import numpy as np
import pytest
import torch

import workloads
from gpu_util import device_inputs, note

pytestmark = pytest.mark.gpu


def _noalloc(lib, q, k, v, o, do, lse, sq, sk, layout, Z, L, H, D, alpha, dtype):
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(k)
    stream = torch.cuda.current_stream().cuda_stream
    rc = lib.sigattn_softmax_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                         lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), sq.data_ptr(),
                                         sk.data_ptr(), layout, Z, L, H, D, alpha, dtype, stream)
    assert rc == 0, lib.sigattn_last_error()
    return dq, dk, dv


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_noalloc_equals_workspace_entry_point(dtype):
    import padding_aware_sigmoid_amd as sa
    from padding_aware_sigmoid_amd import _lib

    lib = _lib.load()
    code = sa.BF16 if dtype == "bf16" else sa.FP32
    # a larger call, then a smaller one that reuses the same device buffer
    for Z, L, H, D, nq, nk in ((3, 700, 4, 128, [700, 333, 65], [512, 700, 1]),
                               (2, 200, 2, 64, [200, 77], [150, 9])):
        note(f"noalloc {dtype} Z={Z} L={L} H={H} D={D} nq={nq} nk={nk}")
        q, k, v, do = workloads.make_tensors(Z, L, H, D, dtype, seed=91 + D)
        dq_, dk_, dv_, ddo, dnq, dnk = device_inputs(q, k, v, do, nq, nk)
        alpha = 1.0 / np.sqrt(D)
        o, lse = sa.sigattn_softmax_fwd(dq_, dk_, dv_, dnq, dnk, alpha)
        ref = sa.sigattn_softmax_bwd(dq_, dk_, dv_, o, ddo, lse, dnq, dnk, alpha)
        got = _noalloc(lib, dq_, dk_, dv_, o, ddo, lse, dnq, dnk, sa.LAYOUT_PADDED, Z, L, H, D, alpha, code)
        torch.cuda.synchronize()
        for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
            assert torch.equal(a, b), f"{name} differs from sigattn_softmax_bwd"
    # packed layout, through the Python wrapper (marshalling only)
    Z, L, H, D, n = 3, 300, 2, 64, [300, 0, 129]
    q, k, v, do = workloads.make_tensors(Z, L, H, D, dtype, seed=97)
    dq_, dk_, dv_, ddo, dn, _ = device_inputs(q, k, v, do, n, n)
    pk = lambda t: torch.cat([t[z, : n[z]] for z in range(Z)], 0).contiguous()  # noqa: E731
    cu = torch.as_tensor(np.concatenate([[0], np.cumsum(n)]).astype(np.int32)).cuda()
    qp, kp, vp, dop = (pk(t) for t in (dq_, dk_, dv_, ddo))
    o, lse = sa.sigattn_softmax_fwd(qp, kp, vp, cu, cu, max_len=L)
    ref = sa.sigattn_softmax_bwd(qp, kp, vp, o, dop, lse, cu, cu, max_len=L)
    got = sa.sigattn_softmax_bwd_noalloc(qp, kp, vp, o, dop, lse, cu, cu, max_len=L)
    torch.cuda.synchronize()
    for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.equal(a, b), f"packed {name} differs from sigattn_softmax_bwd"


def test_noalloc_rejects_sizes_beyond_its_buffer():
    import padding_aware_sigmoid_amd as sa
    from padding_aware_sigmoid_amd import _lib

    lib = _lib.load()
    f = ctypes.c_void_p(256)
    # Z * L * H one row past the fixed buffer: rejected before any launch
    Z, L, H = 1, sa.NOALLOC_ROWS + 1, 1
    rc = lib.sigattn_softmax_bwd_noalloc(f, f, f, f, f, f, f, f, f, f, f, sa.LAYOUT_PADDED, Z, L, H, 64, 0.125,
                                         sa.BF16, None)
    assert rc == -1 and b"SIGATTN_NOALLOC_ROWS" in lib.sigattn_last_error()
