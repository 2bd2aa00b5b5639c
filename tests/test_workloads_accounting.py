"""Input generators and FLOP accounting, against what the pages fix."""

import math

import numpy as np

import workloads
from padding_aware_sigmoid_amd import accounting


def test_lengths_are_seeded_and_in_range():
    for name, w in workloads.WORKLOADS.items():
        a, b = workloads.lengths(w, 0), workloads.lengths(w, 0)
        assert np.array_equal(a, b) and a.dtype == np.int32 and a.shape == (w.Z,)
        assert np.all(a >= 0) and np.all(a <= w.L)


def test_pad25_totals_exactly_a_quarter():
    w = workloads.WORKLOADS["pad25_16k"]
    for seed in range(20):
        n = workloads.lengths(w, seed)
        assert int((w.L - n).sum()) == w.Z * w.L // 4


def test_cell_length_model_matches_the_page_cdf():
    """Gene counts per cell: 57.7/82.0/96.6% at or below 2048/4096/8192 (rainbus.top figure notes).
    The two-parameter log-normal matches the 2048 and 8192 points to within 1 point. It cannot also hit 4096
    (it gives 84.5%), so that point is held to 3 points."""
    rng = np.random.default_rng(0)
    x = rng.lognormal(workloads.CELL_LOGNORMAL_MU, workloads.CELL_LOGNORMAL_SIGMA, 400_000)
    x = x[(x >= workloads.CELL_MIN) & (x <= workloads.CELL_MAX)]
    for cut, frac, tol in ((2048, 0.577, 0.01), (4096, 0.820, 0.03), (8192, 0.966, 0.01)):
        assert abs(np.mean(x <= cut) - frac) < tol, (cut, np.mean(x <= cut))
    w = workloads.WORKLOADS["cellbatch8k"]
    n = workloads.lengths(w, 0)
    assert np.all(n >= 200) and np.all(n <= 8192)


def test_stress_lengths_and_scales():
    w = workloads.WORKLOADS["stress8k"]
    n = workloads.lengths(w, 0)
    assert np.all(n >= 1024) and np.all(n <= 8192)
    assert w.qk_scales == (1.0, 4.0, 16.0)
    q, k, v, do = workloads.make_tensors(1, 64, 1, 64, "fp32", seed=1, qk_scale=16.0)
    q1, k1, v1, _ = workloads.make_tensors(1, 64, 1, 64, "fp32", seed=1, qk_scale=1.0)
    assert np.array_equal(q.numpy(), 16 * q1.numpy()) and np.array_equal(v.numpy(), v1.numpy())


def test_bf16_rounding_is_exact_in_fp64():
    q, _, _, _ = workloads.make_tensors(1, 8, 1, 64, "bf16", seed=3)
    f = workloads.to_f64(q)
    bits = f.astype(np.float32).view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)


def test_flop_rule():
    """The FLOP rule of paperlayer.ai section A.2: 4*D per valid pair forward, backward 2.5x."""
    f = accounting.attention_flops(2, 256, 2, 64, [256, 160], [256, 160])
    assert f["fwd_padded"] == 4 * 64 * 2 * 2 * 256 * 256
    assert f["fwd_valid"] == 4 * 64 * 2 * (256 * 256 + 160 * 160)
    assert math.isclose(f["fwd_padded"] / 1e6, 67.1, rel_tol=1e-3)
    assert math.isclose(f["fwd_valid"] / 1e6, 46.7, rel_tol=2e-3)
    assert f["bwd_valid"] == 2.5 * f["fwd_valid"] and f["total_valid"] == 3.5 * f["fwd_valid"]
    g = accounting.attention_flops(1, 16384, 16, 128)
    assert math.isclose(g["fwd_padded"], 2.199e12, rel_tol=1e-3)
    w = workloads.WORKLOADS["pad25_16k"]
    n = workloads.lengths(w, 0)
    h = accounting.attention_flops(w.Z, w.L, w.H, w.D, n, n)
    assert math.isclose(h["fwd_valid"] / 1e12, 5.157, rel_tol=1e-3)


def test_profile_kernel_names():
    from padding_aware_sigmoid_amd.profiling import short_name

    cases = {
        "void sigattn::fwd_bf16_kernel<128>(...)": "fwd",
        "void sigattn::fwd_bf16_kernel<128, true>(...)": "fwd",
        "void sigattn::fwd_bf16_kernel<64, false>(...)": "fwd",
        "_ZN7sigattn15fwd_bf16_kernelILi128ELb1EEEvPKDF16bS2_S2_PDF16bNS_9SeqLayoutEiiffPi": "fwd",
        "void sigattn::dkdv_bf16_kernel<128, 1, 0>(...)": "dk",
        "void sigattn::dkdv_bf16_kernel<128, 2, 1>(...)": "sm_dv",
        "void sigattn::dkdv_bf16_kernel<64, 0, 0>(...)": "dkdv",
        "void sigattn::dkdv_bf16_kernel<64, 1, 0, true>(...)": "dq",
        "_ZN7sigattn16dkdv_bf16_kernelILi64ELi1ELi0ELb1EEEvPKDF16b": "dq",
        "_ZN7sigattn16dkdv_bf16_kernelILi64ELi1ELi0ELb0EEEvPKDF16b": "dk",
        "void sigattn::dq_bf16_kernel<128, 1>(...)": "sm_dq",
        "void sigattn::dq_bf16_kernel<64, 0>(...)": "dq",
        "void sigattn::sm_fwd_bf16_kernel<128>(...)": "sm_fwd",
        "void sigattn::sm_rowstats_kernel<__bf16, 128>(...)": "sm_rowstats",
        "void sigattn::sm_rowstats_kernel<float, 64>(...)": "sm_rowstats_fp32",
        "void sigattn::dq_fp32_kernel<64>(...)": "dq_fp32",
        "void sigattn::sm_dkdv_fp32_kernel<128>(...)": "sm_dkdv_fp32",
        "_ZN7sigattn16dkdv_bf16_kernelILi128ELi1ELi1EEEvPKDF16b": "sm_dk",
        "_ZN7sigattn16dkdv_bf16_kernelILi128ELi2ELi0EEEvPKDF16b": "dv",
        "_ZN7sigattn14dq_bf16_kernelILi128ELi0EEEvPKDF16b": "dq",
        "_ZN7sigattn18sm_rowstats_kernelIDF16bLi128EEEvPKT_": "sm_rowstats",
        "_ZN7sigattn18sm_fwd_bf16_kernelILi64EEEvPKDF16b": "sm_fwd",
        "void sigattn::fwd_fp8_kernel<128>(...)": "fp8_fwd",
        "void sigattn::quantize_fp8_kernel<64>(...)": "fp8_quantize",
        "_ZN7sigattn14fwd_fp8_kernelILi128EEEvPKhS2_S2_S2_S2_S2_PDF16b": "fp8_fwd",
        "__amd_rocclr_copyBuffer": None,
    }
    for name, want in cases.items():
        assert short_name(name) == want, name
