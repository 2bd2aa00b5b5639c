"""The tile loops run exactly the live tiles, for every remainder of the loop
unrolling.

The bf16 kernels unroll their tile loops over a ring of three LDS slots (the
FP8 forward over two), with the first and last tiles written apart from the
loop. These cases give every kernel tile counts of each residue modulo 3 and
2, in the padded and the packed layout, at both head sizes, for sigmoid and
softmax attention and the FP8 forward:
  lengths 1, 65, 129, 193, 257, 520 -> 1, 2, 3, 4, 5, 9 tiles of 64 rows
  (the forward's and dQ's key tiles and the dK/dV kernel's query tiles).
* Outputs against the oracle at the bf16 bound (2e-2 of max|ref|; the FP8
  forward within the derived elementwise bound of tests/fp8_bound.py),
  padded rows exactly 0.
* The tile counters, which the kernels write from the iterations they ran,
  equal the oracle's tile plan (sigmoid; softmax and FP8 keep no counters).
"""

import numpy as np
import pytest
import torch

import fp8_bound
import oracle
import workloads
from gpu_util import device_inputs, f64, host, note, rel_err

pytestmark = pytest.mark.gpu

TOL = 2e-2
L = 520
LENS = [1, 65, 129, 193, 257, 520]
NQ = LENS
NK = LENS[::-1]


def _packed(t, n):
    return torch.cat([t[z, : int(n[z])] for z in range(t.shape[0])], 0).contiguous()


def _cu(n):
    return torch.as_tensor(np.concatenate([[0], np.cumsum(np.asarray(n, np.int64))]).astype(np.int32))


def _counters(sa, Z, H, D):
    out = {}
    for name, kern, axis in (("fwd", sa.KERNEL_FWD, 0), ("dq", sa.KERNEL_DQ, 0), ("dkdv", sa.KERNEL_DKDV, 1)):
        bq, bk = sa.sigattn_tile_config(kern, D, torch.bfloat16)
        out[name] = (bq, bk, torch.full((Z * H * -(-L // (bq if axis == 0 else bk)),), -7, dtype=torch.int32,
                                        device="cuda"))
    return out


@pytest.mark.parametrize("layout", ["padded", "packed"])
@pytest.mark.parametrize("D", [64, 128])
def test_sigmoid_every_remainder(D, layout):
    import padding_aware_sigmoid_amd as sa

    Z, H = len(NQ), 2
    note(f"tile loops sigmoid D={D} {layout} nq={NQ} nk={NK}")
    q, k, v, do = workloads.make_tensors(Z, L, H, D, "bf16", seed=61)
    dq_, dk_, dv_, ddo, dnq, dnk = device_inputs(q, k, v, do, NQ, NK)
    alpha, bias = 1.0 / np.sqrt(D), -np.log(L)
    tc = _counters(sa, Z, H, D)
    if layout == "padded":
        o = sa.sigattn_fwd(dq_, dk_, dv_, dnq, dnk, alpha, bias, tile_counts=tc["fwd"][2])
        g = sa.sigattn_bwd(dq_, dk_, dv_, ddo, dnq, dnk, alpha, bias, tile_counts_dq=tc["dq"][2],
                           tile_counts_dkdv=tc["dkdv"][2])
    else:
        cq, ck = _cu(NQ).cuda(), _cu(NK).cuda()
        o = sa.sigattn_fwd_varlen(_packed(dq_, NQ), _packed(dk_, NK), _packed(dv_, NK), cq, ck, L, alpha, bias,
                                  tile_counts=tc["fwd"][2])
        g = sa.sigattn_bwd_varlen(_packed(dq_, NQ), _packed(dk_, NK), _packed(dv_, NK), _packed(ddo, NQ), cq, ck, L,
                                  alpha, bias, tile_counts_dq=tc["dq"][2], tile_counts_dkdv=tc["dkdv"][2])
    torch.cuda.synchronize()
    for name, (bq, bk, t) in tc.items():
        by_q, by_k = oracle.tile_plan(NQ, NK, L, bq, bk)
        want = by_k if name == "dkdv" else by_q
        got = t.cpu().numpy().reshape(Z, H, -1)
        for h in range(H):
            assert np.array_equal(got[:, h], want), f"{name}: executed tiles differ from the plan:\n{got[:, h]}\n{want}"
    Q, K, V, DO = (f64(t) for t in (q, k, v, do))
    refs = (oracle.forward(Q, K, V, NQ, NK, alpha, bias),) + oracle.backward(Q, K, V, DO, NQ, NK, alpha, bias)
    for name, got, ref, n in zip(("O", "dQ", "dK", "dV"), (o,) + tuple(g), refs, (NQ, NQ, NK, NK)):
        gv = host(got)
        if layout == "packed":
            gv = oracle.unpack(gv, _cu(n).numpy(), L)
        e = rel_err(gv, ref)
        assert e <= TOL, f"{name}: rel err {e:.3e}"
        for z in range(Z):
            assert np.all(gv[z, n[z]:] == 0.0), f"{name}: padded rows of sample {z} not exactly 0"


@pytest.mark.parametrize("D", [64, 128])
def test_softmax_every_remainder(D):
    import padding_aware_sigmoid_amd as sa

    Z, H = len(NQ), 2
    note(f"tile loops softmax D={D} nq={NQ} nk={NK}")
    q, k, v, do = workloads.make_tensors(Z, L, H, D, "bf16", seed=62)
    dq_, dk_, dv_, ddo, dnq, dnk = device_inputs(q, k, v, do, NQ, NK)
    alpha = 1.0 / np.sqrt(D)
    o, lse = sa.sigattn_softmax_fwd(dq_, dk_, dv_, dnq, dnk, alpha)
    g = sa.sigattn_softmax_bwd(dq_, dk_, dv_, o, ddo, lse, dnq, dnk, alpha)
    torch.cuda.synchronize()
    SM = oracle.softmax_attention
    Q, K, V, DO = (f64(t) for t in (q, k, v, do))
    ro, _ = SM.forward(Q, K, V, NQ, NK, alpha)
    refs = (ro,) + SM.backward(Q, K, V, DO, NQ, NK, alpha)
    for name, got, ref in zip(("O", "dQ", "dK", "dV"), (o,) + tuple(g), refs):
        e = rel_err(host(got), ref)
        assert e <= TOL, f"softmax {name}: rel err {e:.3e}"


@pytest.mark.parametrize("D", [64, 128])
def test_fp8_every_remainder(D):
    import padding_aware_sigmoid_amd as sa

    Z, H = len(NQ), 2
    note(f"tile loops fp8 D={D} nq={NQ} nk={NK}")
    q, k, v, do = workloads.make_tensors(Z, L, H, D, "bf16", seed=63)
    dq_, dk_, dv_, _, dnq, dnk = device_inputs(q, k, v, do, NQ, NK)
    alpha, bias = 1.0 / np.sqrt(D), -np.log(L)
    q8, sq = sa.sigattn_quantize_fp8(dq_, dnq)
    k8, sk = sa.sigattn_quantize_fp8(dk_, dnk)
    v8, sv = sa.sigattn_quantize_fp8(dv_, dnk)
    o = sa.sigattn_fwd_fp8(q8, k8, v8, sq, sk, sv, dnq, dnk, alpha, bias)
    torch.cuda.synchronize()
    got = host(o)
    args = [t.cpu().numpy() for t in (q8, k8, v8, sq, sk, sv)]
    r = fp8_bound.check_batch(got, *args, NQ, NK, alpha, bias, "fp8 O")
    note(f"  fp8 rel err vs oracle {r['oracle']:.2e}, vs MFMA-formed {r['hw']:.2e} "
         f"(bound use {r['hw_ratio']:.3f}), vs exact (bound use {r['exact_ratio']:.3f})")
    for z in range(Z):
        assert np.all(got[z, NQ[z]:] == 0.0)
