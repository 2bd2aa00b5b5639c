"""GPU path (through the C ABI) against the CPU oracle, element by element.

Tolerances, chosen on the numerics of each path:
* bf16 I/O with fp32 accumulation: max|GPU - oracle| / max|oracle| <= 2e-2 for
  O, dQ, dK, dV. The GPU rounds P and dS to bf16 before each MFMA and rounds the
  outputs to bf16. The oracle rounds nothing.
* fp32 validation build: <= 1e-5.
* Padded output rows must be exactly 0 in every case.
Shapes span several tiles and ragged tails (L not a multiple of any tile).
"""

import math
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import assert_padding_zero, device_inputs, f64, host, note, rel_err

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
FP32_TOL = 1e-5


def _run(q, k, v, do, nq, nk, alpha, bias):
    import padding_aware_sigmoid_amd as sa

    dq_, dk_, dv_, ddo, dnq, dnk = device_inputs(q, k, v, do, nq, nk)
    o = sa.sigattn_fwd(dq_, dk_, dv_, dnq, dnk, alpha, bias)
    g = sa.sigattn_bwd(dq_, dk_, dv_, ddo, dnq, dnk, alpha, bias)
    torch.cuda.synchronize()
    return host(o), tuple(host(t) for t in g)


def _check_full(q, k, v, do, nq, nk, alpha, bias, tol, label):
    note(f"parity {label} shape={tuple(q.shape)} dtype={q.dtype} nq={list(nq)} nk={list(nk)}")
    o, (dq, dk, dv) = _run(q, k, v, do, nq, nk, alpha, bias)
    Q, K, V, DO = (f64(t) for t in (q, k, v, do))
    o_ref = oracle.forward(Q, K, V, nq, nk, alpha, bias)
    dq_ref, dk_ref, dv_ref = oracle.backward(Q, K, V, DO, nq, nk, alpha, bias)
    errs = {n: rel_err(a, b) for n, a, b in (("O", o, o_ref), ("dQ", dq, dq_ref), ("dK", dk, dk_ref),
                                             ("dV", dv, dv_ref))}
    for n, e in errs.items():
        assert e <= tol, f"{label}: {n} rel err {e:.3e} > {tol}"
    assert_padding_zero("O", o, nq)
    assert_padding_zero("dQ", dq, nq)
    assert_padding_zero("dK", dk, nk)
    assert_padding_zero("dV", dv, nk)
    return errs


CASES = [
    # (label, Z, L, H, D, nq, nk)
    ("ragged-d64", 3, 300, 2, 64, [300, 131, 7], [300, 131, 7]),
    ("ragged-d128", 2, 333, 2, 128, [333, 200], [333, 200]),
    ("nq!=nk", 2, 260, 1, 128, [260, 65], [129, 260]),
    ("edge-lengths", 4, 192, 1, 64, [0, 1, 128, 64], [192, 1, 0, 65]),
    ("single-tile", 1, 64, 3, 128, [40], [64]),
    # both sides of the fused dK/dV kernel's 128-row passes (a second pass
    # wholly in padding: n = 1, 127, 128) and of its 256-row workgroup tiles
    ("passes-d128", 6, 400, 1, 128, [385, 256, 129, 128, 127, 1], [1, 127, 128, 129, 256, 385]),
    ("passes-d64", 6, 400, 1, 64, [385, 256, 129, 128, 127, 1], [1, 127, 128, 129, 256, 385]),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bf16_parity(case):
    label, Z, L, H, D, nq, nk = case
    q, k, v, do = workloads.make_tensors(Z, L, H, D, "bf16", seed=zlib.crc32(label.encode()) % 1000)
    _check_full(q, k, v, do, np.array(nq), np.array(nk), 1 / math.sqrt(D), -math.log(L), BF16_TOL, label)


@pytest.mark.parametrize("D", [64, 128])
def test_many_samples(D):
    """More samples than the tile scheduler ranks (256): the unranked mapping,
    with lengths 0..L and Z * H not a multiple of 8."""
    Z, L, H = 301, 40, 1
    rng = np.random.default_rng(D)
    nq = rng.integers(0, L + 1, Z)
    nk = rng.integers(0, L + 1, Z)
    q, k, v, do = workloads.make_tensors(Z, L, H, D, "bf16", seed=77)
    _check_full(q, k, v, do, nq, nk, 1 / math.sqrt(D), -math.log(L), BF16_TOL, f"many-samples-D{D}")


@pytest.mark.parametrize("D", [64, 128])
def test_fp32_validation_build(D):
    """The tiny workload (Z=2, H=2, L=256, lengths [256, 160]) in fp32, at 1e-5."""
    w = workloads.WORKLOADS["tiny"]
    n = workloads.lengths(w)
    q, k, v, do = workloads.make_tensors(w.Z, w.L, w.H, D, "fp32", seed=0)
    _check_full(q, k, v, do, n, n, 1 / math.sqrt(D), w.bias, FP32_TOL, f"fp32-tiny-D{D}")


def test_tiny_workload_bf16():
    w = workloads.WORKLOADS["tiny"]
    n = workloads.lengths(w)
    q, k, v, do = workloads.make_tensors(w.Z, w.L, w.H, w.D, "bf16", seed=0)
    _check_full(q, k, v, do, n, n, w.alpha, w.bias, BF16_TOL, "tiny-bf16")


@pytest.mark.parametrize("scale", [4.0, 16.0])
def test_large_scores_bf16(scale):
    """The stress workload's score scale on a small shape: outputs finite and within tolerance."""
    q, k, v, do = workloads.make_tensors(2, 320, 2, 64, "bf16", seed=5, qk_scale=scale)
    n = np.array([320, 170])
    _check_full(q, k, v, do, n, n, 1 / 8, -math.log(320), BF16_TOL, f"stress-s{scale}")
    o, g = _run(q, k, v, do, n, n, 1 / 8, -math.log(320))
    assert np.all(np.isfinite(o)) and all(np.all(np.isfinite(t)) for t in g)
