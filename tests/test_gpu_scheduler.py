"""The tile scheduler with many samples.

Each workgroup maps its index to (sample, head, row block): the samples are
ranked heaviest first when there are at most 256 of them, and the (sample,
head) pairs are dealt over the 8 XCDs when their count is a multiple of 8.
These cases cover the three regimes the mapping has:
  Z = 256, H = 8  ranked, dealt;
  Z = 300, H = 2  not ranked (more than 256 samples), dealt (600 pairs);
  Z = 301, H = 3  not ranked, not dealt (903 pairs).
The mapping decides only which workgroup computes which tile, so the outputs
must equal the oracle's whatever it does, with every padded row exactly 0
(a tile computed twice or never shows there), and the tile counters must
equal the oracle's tile plan entry for entry. The softmax kernels and the
FP8 forward share the mapping; one regime each checks them against their
oracles.
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
L, D = 160, 64


@pytest.mark.parametrize("Z,H", [(256, 8), (300, 2), (301, 3)])
def test_many_samples(Z, H):
    import padding_aware_sigmoid_amd as sa

    rng = np.random.default_rng(Z * 10 + H)
    nq = rng.integers(0, L + 1, Z)
    nk = rng.integers(0, L + 1, Z)
    nq[:3] = [0, L, 1]
    nk[:3] = [L, 0, 65]
    note(f"scheduler Z={Z} H={H} L={L} D={D}")
    q, k, v, do = workloads.make_tensors(Z, L, H, D, "bf16", seed=71)
    dq_, dk_, dv_, ddo, dnq, dnk = device_inputs(q, k, v, do, nq, nk)
    alpha, bias = 1.0 / np.sqrt(D), -np.log(L)
    tcs = {}
    for name, kern, axis in (("fwd", sa.KERNEL_FWD, 0), ("dq", sa.KERNEL_DQ, 0), ("dkdv", sa.KERNEL_DKDV, 1)):
        bq, bk = sa.sigattn_tile_config(kern, D, torch.bfloat16)
        tcs[name] = (bq, bk, torch.full((Z * H * -(-L // (bq if axis == 0 else bk)),), -7, dtype=torch.int32,
                                        device="cuda"))
    o = sa.sigattn_fwd(dq_, dk_, dv_, dnq, dnk, alpha, bias, tile_counts=tcs["fwd"][2])
    g = sa.sigattn_bwd(dq_, dk_, dv_, ddo, dnq, dnk, alpha, bias, tile_counts_dq=tcs["dq"][2],
                       tile_counts_dkdv=tcs["dkdv"][2])
    torch.cuda.synchronize()
    for name, (bq, bk, t) in tcs.items():
        by_q, by_k = oracle.tile_plan(nq, nk, L, bq, bk)
        want = by_k if name == "dkdv" else by_q
        got = t.cpu().numpy().reshape(Z, H, -1)
        for h in range(H):
            assert np.array_equal(got[:, h], want), f"{name}: tile counters differ from the plan (head {h})"
    Q, K, V, DO = (f64(t) for t in (q, k, v, do))
    refs = (oracle.forward(Q, K, V, nq, nk, alpha, bias),) + oracle.backward(Q, K, V, DO, nq, nk, alpha, bias)
    for name, got, ref, n in zip(("O", "dQ", "dK", "dV"), (o,) + tuple(g), refs, (nq, nq, nk, nk)):
        gv = host(got)
        e = rel_err(gv, ref)
        assert e <= TOL, f"{name}: rel err {e:.3e}"
        for z in range(Z):
            assert np.all(gv[z, n[z]:] == 0.0), f"{name}: padded rows of sample {z} not exactly 0"


def _lengths(Z, seed):
    rng = np.random.default_rng(seed)
    nq, nk = rng.integers(0, L + 1, Z), rng.integers(0, L + 1, Z)
    nq[:2] = [0, L]
    nk[:2] = [L, 0]
    return nq, nk


def test_many_samples_softmax():
    """Softmax forward and backward share the mapping: 300 samples (not ranked, dealt)."""
    import padding_aware_sigmoid_amd as sa

    Z, H = 300, 2
    nq, nk = _lengths(Z, 5)
    note(f"scheduler softmax Z={Z} H={H} L={L} D={D}")
    q, k, v, do = workloads.make_tensors(Z, L, H, D, "bf16", seed=72)
    dq_, dk_, dv_, ddo, dnq, dnk = device_inputs(q, k, v, do, nq, nk)
    alpha = 1.0 / np.sqrt(D)
    o, lse = sa.sigattn_softmax_fwd(dq_, dk_, dv_, dnq, dnk, alpha)
    g = sa.sigattn_softmax_bwd(dq_, dk_, dv_, o, ddo, lse, dnq, dnk, alpha)
    torch.cuda.synchronize()
    SM = oracle.softmax_attention
    Q, K, V, DO = (f64(t) for t in (q, k, v, do))
    ro, _ = SM.forward(Q, K, V, nq, nk, alpha)
    refs = (ro,) + SM.backward(Q, K, V, DO, nq, nk, alpha)
    for name, got, ref, n in zip(("O", "dQ", "dK", "dV"), (o,) + tuple(g), refs, (nq, nq, nk, nk)):
        gv = host(got)
        e = rel_err(gv, ref)
        assert e <= TOL, f"softmax {name}: rel err {e:.3e}"
        for z in range(Z):
            assert np.all(gv[z, n[z]:] == 0.0), f"softmax {name}: padded rows of sample {z} not exactly 0"


def test_many_samples_fp8():
    """The FP8 forward shares the mapping: 256 samples (ranked, dealt). Every slice is held
    to the bound against exact attention of tests/fp8_bound.py, and heads 0 and H - 1
    also to the tighter bound against the MFMA-formed FP8 forward."""
    import padding_aware_sigmoid_amd as sa

    Z, H = 256, 8
    nq, nk = _lengths(Z, 6)
    note(f"scheduler fp8 Z={Z} H={H} L={L} D={D}")
    q, k, v, do = workloads.make_tensors(Z, L, H, D, "bf16", seed=73)
    dq_, dk_, dv_, _, dnq, dnk = device_inputs(q, k, v, do, nq, nk)
    alpha, bias = 1.0 / np.sqrt(D), -np.log(L)
    q8, sq = sa.sigattn_quantize_fp8(dq_, dnq)
    k8, sk = sa.sigattn_quantize_fp8(dk_, dnk)
    v8, sv = sa.sigattn_quantize_fp8(dv_, dnk)
    o = sa.sigattn_fwd_fp8(q8, k8, v8, sq, sk, sv, dnq, dnk, alpha, bias)
    torch.cuda.synchronize()
    gv = host(o)
    args = [t.cpu().numpy() for t in (q8, k8, v8, sq, sk, sv)]
    r = fp8_bound.check_batch(gv, *args, nq, nk, alpha, bias, "fp8 O", hw_heads=(0, H - 1))
    note(f"  fp8 rel err vs oracle {r['oracle']:.2e}, vs MFMA-formed {r['hw']:.2e} "
         f"(bound use {r['hw_ratio']:.3f}), vs exact (bound use {r['exact_ratio']:.3f})")
    for z in range(Z):
        assert np.all(gv[z, nq[z]:] == 0.0), f"fp8 O: padded rows of sample {z} not exactly 0"
