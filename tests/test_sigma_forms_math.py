"""The numbers behind the forward's one-transcendental sigma, checked on the CPU.

The bf16 forward takes sigma(S) = t - t^2 with t = e^S on every block of
scores whose t stays at or below 2^-5, and the exact logistic elsewhere; a
workgroup whose first block has a score with t above 2^-6 runs the exact
form throughout. These tests pin the claims the kernel's comments and the
design notes rest on, against the oracle's logistic in float64:

* the error of t - t^2 is t^3 / (1 + t), that is a relative error below t^2,
  at most 2^-10 over the whole range S <= -5 ln 2;
* in bf16 (the precision P enters the MFMA in) the two forms round to the
  same value almost everywhere and never more than one bf16 step apart;
* the bounds as the kernel encodes them: the bit pattern of 2^-5 in float32,
  the score at which t = 2^-5 (-3.47), and the vote's -6 on the log2 scale of
  the exponent's argument (S = -4.16).
"""

import numpy as np
import torch

from oracle import sigmoid_attention as osa

T_MAX = 2.0 ** -5


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)


def test_relative_error_of_the_one_transcendental_form():
    s = np.linspace(-40.0, -5.0 * np.log(2.0), 200001)
    t = np.exp(s)
    exact = osa.sigmoid(s)
    fast = t - t * t
    rel = np.abs(fast - exact) / exact
    u64 = 2.0 ** -53  # float64 rounding of both sides, which dominates for tiny t
    assert np.all(rel <= t * t * (1 + 1e-9) + 4 * u64)
    assert float(rel.max()) <= 2.0 ** -10 * (1 + 1e-9)  # t^2 exactly, at t = 2^-5
    # the error is one-sided (t - t^2 undershoots) and its size is t^3 / (1 + t)
    big = t > 1e-3  # where t^3 stands clear of float64 rounding
    assert np.all(fast[big] < exact[big])
    np.testing.assert_allclose((exact - fast)[big], (t ** 3 / (1 + t))[big], rtol=1e-6, atol=0)


def test_bf16_roundings_agree_or_differ_by_one_step():
    s = np.linspace(-30.0, -5.0 * np.log(2.0), 100001)
    t = np.exp(s)
    exact = _bf16(osa.sigmoid(s))
    fast = _bf16(t - t * t)
    differ = exact != fast
    assert differ.mean() < 0.01
    # where they differ, they are neighbours: one bf16 step (2^-7 relative at most) apart
    assert np.all(np.abs(exact[differ] - fast[differ]) <= exact[differ] * 2.0 ** -7 * (1 + 1e-9))


def test_the_bounds_as_encoded():
    assert np.float32(T_MAX).view(np.uint32) == 0x3D000000
    assert abs(np.log(T_MAX) - (-3.4657)) < 1e-4
    # the vote: exponent argument y = S log2(e) <= -6, i.e. t <= 2^-6, S <= -4.16
    assert abs(-6.0 / np.log2(np.e) - (-4.1589)) < 1e-4
    # a zero-filled padded key scores S = b; launches try the form only when
    # c0 = -b log2(e) >= 6, so such a key's t = 2^-c0 <= 2^-6 < 2^-5
    assert 2.0 ** -6 < T_MAX
