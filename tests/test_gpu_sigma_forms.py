"""The forward's two forms of sigma, against the oracle.

The bf16 forward computes each 32 x 32 block of weights of a wave with
sigma(S) = t - t^2, t = e^S (one exponential per score; relative error t^2, at
most 2^-10 while t <= 2^-5, that is S <= -3.47), and keeps the largest t of the
block. If some score of the block lies outside that range, the wave
recomputes the whole block with the exact sigma = 1 / (1 + e^-S) before the
weights are used. A workgroup whose waves find a score above the range in
their first block of key tile 0 runs the exact form throughout, and so does
a launch whose bias is above -4.16 (where a zero-filled padded key alone
would leave the range).

* Every score in range (small-norm inputs, b = -ln L): the one-exponential
  result is within the bf16 tolerance of the exact oracle.
* One planted score far above 0 in the last or a middle key tile of a sample
  (a block recomputed inside the key loop), or in the first block of tile 0
  (the workgroup's vote): the form t - t^2 would make that weight a large
  negative number, so the output matches the oracle only if the exact form
  produced it.
* A bias that rules the one-exponential form out from the start.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import assert_padding_zero, device_inputs, f64, host, note, rel_err

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2


def _inputs(Z, L, H, D, seed, qk_scale):
    return workloads.make_tensors(Z, L, H, D, "bf16", seed=seed, qk_scale=qk_scale)


def _plant(q, k, z, h, i, j, alpha, target):
    """Make the raw score of query i and key j (sample z, head h) equal about
    target / alpha, by setting key j to a multiple of query i."""
    qi = q[z, i, h].float()
    beta = target / (alpha * float(qi @ qi))
    k[z, j, h] = (beta * qi).to(k.dtype)


def _forward_parity(q, k, v, n, alpha, bias, label):
    import padding_aware_sigmoid_amd as sa

    note(f"sigma forms {label} shape={tuple(q.shape)} n={list(n)} bias={bias:.3f}")
    dq_, dk_, dv_, _, dn, _ = device_inputs(q, k, v, v, n, n)
    o = sa.sigattn_fwd(dq_, dk_, dv_, dn, dn, alpha, bias)
    torch.cuda.synchronize()
    got = host(o)
    ref = oracle.forward(f64(q), f64(k), f64(v), n, n, alpha, bias)
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    err = rel_err(got, ref)
    assert err <= BF16_TOL, f"{label}: O rel err {err:.3e} > {BF16_TOL}"
    assert_padding_zero("O", got, n)
    return got, ref


@pytest.mark.parametrize("D", [64, 128])
def test_all_scores_in_the_one_exponential_range(D):
    Z, L, H = 2, 2048, 2
    n = np.array([2048, 1500])
    alpha, bias = 1 / math.sqrt(D), -math.log(L)
    q, k, v, _ = _inputs(Z, L, H, D, seed=40, qk_scale=0.5)
    got, ref = _forward_parity(q, k, v, n, alpha, bias, f"in range D={D}")
    # every score of these inputs is far inside the range
    s = np.einsum("zihd,zjhd->zhij", f64(q), f64(k)) * alpha + bias
    assert float(s.max()) < -3.47 - 1.0


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("where", ["last", "first", "middle"])
def test_planted_score_forces_the_exact_sigma(D, where):
    Z, L, H = 2, 2048, 2
    n = np.array([2048, 1500])
    alpha, bias = 1 / math.sqrt(D), -math.log(L)
    q, k, v, _ = _inputs(Z, L, H, D, seed=41, qk_scale=0.5)
    j = {"last": int(n[1]) - 3, "first": 5, "middle": 777}[where]
    i = 300
    _plant(q, k, 1, 1, i, j, alpha, 12.0)  # S = 12 + b = 4.4: sigma 0.988, e^S = 81
    s = float((q[1, i, 1].float() @ k[1, j, 1].float())) * alpha + bias
    assert s > 2.0, "the planted score must lie far outside the one-exponential range"
    got, ref = _forward_parity(q, k, v, n, alpha, bias, f"planted {where} D={D}")
    # the planted row itself, on its own scale
    row_err = float(np.max(np.abs(got[1, i, 1] - ref[1, i, 1])) / np.max(np.abs(ref[1, i, 1])))
    assert row_err <= BF16_TOL, f"planted row rel err {row_err:.3e}"


@pytest.mark.parametrize("D", [64, 128])
def test_bias_outside_the_range_runs_the_exact_sigma(D):
    Z, L, H = 2, 700, 1
    n = np.array([700, 333])
    alpha, bias = 1 / math.sqrt(D), -2.0
    q, k, v, _ = _inputs(Z, L, H, D, seed=42, qk_scale=1.0)
    _forward_parity(q, k, v, n, alpha, bias, f"bias -2 D={D}")


@pytest.mark.parametrize("D", [64, 128])
def test_one_exponential_form_every_tile_count(D):
    """Samples of 1 to 5 key tiles, full and partial, with scores inside the
    one-exponential range (so every workgroup takes that form): the prologue,
    the leftover iterations after the loop in rounds of three, and the last
    tile's epilogue each check their blocks. Tile counters equal the plan."""
    import padding_aware_sigmoid_amd as sa

    lengths = [1, 40, 64, 65, 100, 128, 129, 192, 200, 256, 300]
    Z, L, H = len(lengths), 320, 1
    n = np.array(lengths)
    alpha, bias = 1 / math.sqrt(D), -math.log(L)
    q, k, v, _ = _inputs(Z, L, H, D, seed=43, qk_scale=0.4)
    s = np.einsum("zihd,zjhd->zhij", f64(q), f64(k)) * alpha + bias
    # every workgroup's vote passes (t <= 2^-6, that is S <= -4.16), with room
    assert float(s.max()) < -4.16 - 0.5
    _forward_parity(q, k, v, n, alpha, bias, f"every tile count D={D}")
    dq_, dk_, dv_, _, dn, _ = device_inputs(q, k, v, v, n, n)
    bq, bk = sa.sigattn_tile_config(sa.KERNEL_FWD, D, dq_.dtype)
    tc = torch.full((Z * H * (-(-L // bq)),), -7, dtype=torch.int32, device=dq_.device)
    sa.sigattn_fwd(dq_, dk_, dv_, dn, dn, alpha, bias, tile_counts=tc)
    torch.cuda.synchronize()
    by_q, _ = oracle.tile_plan(n, n, L, bq, bk)
    assert np.array_equal(tc.cpu().numpy().reshape(Z, H, -1)[:, 0, :], by_q)
