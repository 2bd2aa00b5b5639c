"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
rejects bad arguments with status codes without launching anything."""

import ctypes
import pathlib
import re

import pytest

ROOT = pathlib.Path(__file__).resolve().parents[1]
HEADER = ROOT / "include" / "sigattn.h"


def _declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sigattn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from padding_aware_sigmoid_amd import _lib

    if not _lib.lib_path().exists():
        pytest.skip("libsigattn.so not built")
    return _lib.load()


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("sigattn_fwd", "sigattn_bwd", "sigattn_bwd_dkdv", "sigattn_bwd_dq", "sigattn_bwd_dk",
              "sigattn_bwd_dv", "sigattn_fwd_ex", "sigattn_bwd_ex", "sigattn_tile_config",
              "sigattn_strerror", "sigattn_last_error", "sigattn_version"):
        assert n in names
    assert "sigattn_workspace_size" not in names


def test_every_declared_symbol_is_exported(lib):
    from padding_aware_sigmoid_amd import _lib

    for name in _declared_functions():
        assert hasattr(lib, name), f"{name} declared in sigattn.h but not exported"
    assert set(_lib.EXPORTED_SYMBOLS) == set(_declared_functions())


def test_argument_errors_need_no_gpu(lib):
    null = None
    # D not 64/128
    assert lib.sigattn_fwd(null, null, null, null, null, null, 1, 8, 1, 96, 1.0, 0.0, 0, null, null) == -1
    assert b"D must be" in lib.sigattn_last_error()
    # unknown dtype
    assert lib.sigattn_fwd(null, null, null, null, null, null, 1, 8, 1, 64, 1.0, 0.0, 9, null, null) == -2
    # negative sizes
    assert lib.sigattn_bwd(null, null, null, null, null, null, null, null, null, -1, 8, 1, 64, 1.0, 0.0, 0, null,
                           null, null) == -1
    # non-finite scalars
    assert lib.sigattn_bwd_dq(null, null, null, null, null, null, null, 1, 8, 1, 64, float("inf"), 0.0, 0, null,
                              null) == -1
    # NULL lengths with a non-empty batch
    assert lib.sigattn_bwd_dkdv(null, null, null, null, null, null, null, null, 1, 8, 1, 64, 1.0, 0.0, 0, null,
                                null) == -1
    assert lib.sigattn_bwd_dk(null, null, null, null, null, null, null, 1, 8, 1, 128, 1.0, 0.0, 0, null, null) == -1
    # dv needs no v: only q, k, dout and dv are checked
    fake0 = ctypes.c_void_p(16)
    assert lib.sigattn_bwd_dv(fake0, fake0, fake0, null, fake0, fake0, 1, 8, 1, 128, 1.0, 0.0, 0, null, null) == -1
    assert b"tensor dv is NULL" in lib.sigattn_last_error()
    assert lib.sigattn_bwd_dv(null, null, null, null, null, null, 0, 8, 1, 128, 1.0, 0.0, 0, null, null) == 0
    # layout and bias mode of the _ex entry points
    assert lib.sigattn_fwd_ex(null, null, null, null, null, null, 2, 0, 1, 8, 1, 64, 1.0, 0.0, 0, null, null) == -1
    assert b"layout" in lib.sigattn_last_error()
    assert lib.sigattn_fwd_ex(null, null, null, null, null, null, 1, 7, 1, 8, 1, 64, 1.0, 0.0, 0, null, null) == -1
    assert b"bias mode" in lib.sigattn_last_error()
    assert lib.sigattn_bwd_ex(null, null, null, null, null, null, null, null, null, 1, 1, 1, 8, 1, 96, 1.0, 0.0, 0,
                              null, null, null) == -1
    assert b"D must be" in lib.sigattn_last_error()
    # an empty packed batch is a no-op success
    assert lib.sigattn_fwd_ex(null, null, null, null, null, null, 1, 1, 0, 8, 1, 64, 1.0, 0.0, 0, null, null) == 0
    # NULL tensors (lengths non-NULL but never dereferenced on the host)
    fake = ctypes.c_void_p(16)
    assert lib.sigattn_fwd(null, null, null, null, fake, fake, 1, 8, 1, 64, 1.0, 0.0, 0, null, null) == -1
    assert b"is NULL" in lib.sigattn_last_error()
    # misaligned tensor
    assert lib.sigattn_fwd(ctypes.c_void_p(18), fake, fake, fake, fake, fake, 1, 8, 1, 64, 1.0, 0.0, 0, null,
                           null) == -1
    assert b"aligned" in lib.sigattn_last_error()
    # an empty batch is a no-op success, even with NULL pointers
    assert lib.sigattn_fwd(null, null, null, null, null, null, 0, 8, 1, 64, 1.0, 0.0, 0, null, null) == 0


def test_strings_and_configs(lib):
    from padding_aware_sigmoid_amd import _lib

    assert lib.sigattn_strerror(0) == b"ok"
    assert lib.sigattn_strerror(-3) == b"HIP error"
    assert b"gfx950" in lib.sigattn_version()
    for kern in (0, 1, 2):
        for d in (64, 128):
            for dt in (0, 1):
                bq, bk = _lib.tile_config(kern, d, dt)
                assert bq > 0 and bk > 0 and bq % 32 == 0 and bk % 32 == 0
    with pytest.raises(_lib.SigattnError):
        _lib.tile_config(5, 64, 0)


def test_softmax_argument_errors_need_no_gpu(lib):
    null, f = None, ctypes.c_void_p(16)
    fwd = lib.sigattn_softmax_fwd
    bwd = lib.sigattn_softmax_bwd
    # alpha must be > 0 (the running row maximum assumes it)
    for a in (0.0, -1.0, float("nan")):
        assert fwd(f, f, f, f, f, f, f, 0, 1, 8, 1, 64, a, 0, null) == -1
        assert b"alpha > 0" in lib.sigattn_last_error()
    assert fwd(f, f, f, f, f, f, f, 2, 1, 8, 1, 64, 1.0, 0, null) == -1
    assert b"layout" in lib.sigattn_last_error()
    assert fwd(f, f, f, f, f, f, f, 0, 1, 8, 1, 96, 1.0, 0, null) == -1
    assert fwd(f, f, f, f, f, f, f, 0, 1, 8, 1, 64, 1.0, 7, null) == -2
    # NULL lse
    assert fwd(f, f, f, f, null, f, f, 0, 1, 8, 1, 64, 1.0, 0, null) == -1
    assert b"lse" in lib.sigattn_last_error()
    # empty batch: nothing to do
    assert fwd(null, null, null, null, null, null, null, 0, 0, 8, 1, 64, 1.0, 0, null) == 0
    # backward: NULL workspace, then one too small for Z * L * H rows (padded)
    assert bwd(f, f, f, f, f, f, f, f, f, f, f, 0, 2, 8, 3, 64, 1.0, 0, null, 0, null) == -1
    assert b"workspace" in lib.sigattn_last_error()
    assert bwd(f, f, f, f, f, f, f, f, f, f, f, 0, 2, 8, 3, 64, 1.0, 0, f, 2 * 8 * 3 * 8 - 1, null) == -4
    assert bwd(f, f, f, f, f, f, f, f, f, f, f, 0, 2, 8, 3, 64, 0.0, 0, f, 1 << 20, null) == -1
    assert lib.sigattn_softmax_bwd_workspace_size(2 * 8, 3) == 2 * 8 * 3 * 8
    assert lib.sigattn_softmax_bwd_workspace_size(0, 3) == 0


def test_grid_limit(lib):
    null, f = None, ctypes.c_void_p(16)
    # 2^20 samples of 2^16 rows: more work-items than one dispatch holds
    assert lib.sigattn_fwd(f, f, f, f, f, f, 1 << 20, 1 << 16, 1, 64, 1.0, 0.0, 0, null, null) == -1
    assert b"too large" in lib.sigattn_last_error()
    # The bound follows the smallest workgroup tile (128 rows of 256
    # work-items, the fused dK/dV kernel). 2^23 - 1 pairs of 384 rows take
    # 3 such workgroups each, 1.5 * 2^32 work-items, but fit with 256-row
    # workgroups (2^32 - 512). Rejected before any launch.
    Z = (1 << 23) - 1
    assert lib.sigattn_bwd_dkdv(f, f, f, f, f, f, f, f, Z, 384, 1, 128, 1.0, 0.0, 0, null, null) == -1
    assert b"too large" in lib.sigattn_last_error()


def test_fp8_argument_errors_need_no_gpu(lib):
    null, f = None, ctypes.c_void_p(16)
    q, fwd = lib.sigattn_quantize_fp8, lib.sigattn_fwd_fp8
    assert q(f, f, null, f, 0, 1, 64, 1, 128, null) == -1
    assert b"scales" in lib.sigattn_last_error()
    assert q(f, f, f, f, 3, 1, 64, 1, 128, null) == -1
    assert q(f, f, f, f, 0, 1, 64, 1, 96, null) == -1
    assert q(null, null, null, null, 0, 0, 64, 1, 128, null) == 0   # empty batch
    for a in (0.0, -0.5):
        assert fwd(f, f, f, f, f, f, f, f, f, 0, 0, 1, 64, 1, 128, a, 0.0, null) == -1
        assert b"alpha > 0" in lib.sigattn_last_error()
    assert fwd(f, f, f, f, f, f, f, f, f, 0, 0, 1, 262144 + 64, 1, 128, 0.1, 0.0, null) == -1
    assert b"262144" in lib.sigattn_last_error()
    assert fwd(f, f, f, null, f, f, f, f, f, 0, 0, 1, 64, 1, 128, 0.1, 0.0, null) == -1
    assert b"scale" in lib.sigattn_last_error()
    assert fwd(f, f, f, f, f, f, f, f, f, 0, 5, 1, 64, 1, 128, 0.1, 0.0, null) == -1


def _declared_prototypes():
    """{name: parameter count} of every function sigattn.h declares."""
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    out = {}
    for m in re.finditer(r"\b(sigattn_[a-z0-9_]+)\s*\(([^)]*)\)\s*;", text):
        params = [x.strip() for x in m.group(2).split(",") if x.strip()]
        out[m.group(1)] = 0 if params in ([], ["void"]) else len(params)
    return out


def test_binding_signatures_match_the_header(lib):
    """Every prototype in sigattn.h has as many parameters as the ctypes
    binding passes, so no header parameter is dropped or padded on the way."""
    protos = _declared_prototypes()
    assert set(protos) == set(_declared_functions())
    for name, nparams in protos.items():
        assert len(getattr(lib, name).argtypes) == nparams, f"{name}: header {nparams} parameters, binding differs"


def test_enum_parameters_are_typed():
    """dtype, layout, bias mode and kernel arguments carry their enum types;
    no entry point takes workspace arguments it would ignore."""
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    assert not re.search(r"\bint\s+(dtype|layout|bias_mode|kernel)\b", text)
    assert "sigattn_dtype dtype" in text and "sigattn_layout layout" in text
    fwd = re.search(r"int sigattn_fwd\(([^)]*)\)", text).group(1)
    bwd = re.search(r"int sigattn_bwd\(([^)]*)\)", text).group(1)
    assert "workspace" not in fwd and "workspace" not in bwd


def test_unknown_enum_values_are_rejected(lib):
    null, f = None, ctypes.c_void_p(16)
    assert lib.sigattn_fwd(f, f, f, f, f, f, 1, 8, 1, 64, 1.0, 0.0, 0x7fffffff, null, null) == -2
    assert lib.sigattn_fwd_ex(f, f, f, f, f, f, -1, 0, 1, 8, 1, 64, 1.0, 0.0, 0, null, null) == -1
    assert lib.sigattn_fwd_ex(f, f, f, f, f, f, 0, 0x7fffffff, 1, 8, 1, 64, 1.0, 0.0, 0, null, null) == -1
    bq, bk = ctypes.c_int(), ctypes.c_int()
    assert lib.sigattn_tile_config(0x7fffffff, 64, 0, ctypes.byref(bq), ctypes.byref(bk)) == -1


def test_packed_offsets_are_checked_on_the_host():
    """The binding rejects offsets the kernels would trust: not starting at 0,
    decreasing, past the tensor, or a sample longer than max_len."""
    from padding_aware_sigmoid_amd.ops import check_offsets

    check_offsets([0, 3, 3, 10], 10, 7)
    check_offsets([0], 0, 1)
    for cu, rows, L, what in (([1, 3], 10, 8, "start at 0"), ([0, 5, 4], 10, 8, "non-decreasing"),
                              ([0, 4, 11], 10, 8, "past the tensor"), ([0, 9, 10], 10, 8, "more than max_len"),
                              ([], 0, 8, r"Z \+ 1")):
        with pytest.raises(ValueError, match=what):
            check_offsets(cu, rows, L)
