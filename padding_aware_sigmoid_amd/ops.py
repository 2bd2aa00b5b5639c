"""Torch-facing binding of the C ABI. It marshals tensors to pointers and sizes.

The functions carry the C entry points' names. torch supplies device memory
and the current HIP stream, and nothing else: every step of the attention runs
in libsigattn.so's kernels. There is no CPU path. A missing library raises.
"""

from __future__ import annotations

import math

import torch

from . import _lib

_DTYPES = {torch.bfloat16: _lib.BF16, torch.float32: _lib.FP32}


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"sigattn supports bfloat16 and float32 tensors, got {t.dtype}") from None


def _check_tensors(ref: torch.Tensor, named: dict) -> None:
    if ref.dim() != 4:
        raise ValueError("tensors must be [Z, L, H, D]")
    if ref.device.type != "cuda":
        raise ValueError("sigattn tensors must live on a HIP device")
    for name, t in named.items():
        if t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device:
            raise ValueError(f"{name} must match q in shape, dtype and device")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous [Z, L, H, D]")


def _lengths(n, Z: int, device) -> torch.Tensor:
    if isinstance(n, torch.Tensor):
        if n.dtype != torch.int32 or n.device != device or n.numel() != Z or not n.is_contiguous():
            raise ValueError("sequence lengths must be a contiguous int32[Z] tensor on the tensors' device")
        return n
    t = torch.as_tensor(n, dtype=torch.int32).reshape(-1)
    if t.numel() != Z:
        raise ValueError(f"expected {Z} sequence lengths")
    return t.to(device)


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def default_alpha(D: int) -> float:
    return 1.0 / math.sqrt(D)


def default_bias(L: int, bias_mode: int = _lib.BIAS_CONSTANT) -> float:
    """-ln L with one bias for every sample; 0 when the bias is per sample
    (b_z = bias - ln n_k[z])."""
    return 0.0 if bias_mode == _lib.BIAS_NEG_LOG_NK else -math.log(L)


_BIAS_MODES = {"constant": _lib.BIAS_CONSTANT, "neg_log_nk": _lib.BIAS_NEG_LOG_NK}


def _bias_mode(mode) -> int:
    if isinstance(mode, str):
        try:
            return _BIAS_MODES[mode]
        except KeyError:
            raise ValueError(f"bias_mode must be one of {sorted(_BIAS_MODES)}") from None
    return int(mode)


def sigattn_fwd(q, k, v, seqlens_q, seqlens_k, alpha=None, bias=None, out=None, tile_counts=None,
                bias_mode="constant"):
    """O = sigma(alpha q k^T + b) v with padding. Wraps the C entry point sigattn_fwd
    (sigattn_fwd_ex when the bias is per sample).

    q, k, v: [Z, L, H, D] bf16 or fp32 on the device. seqlens_*: int32[Z].
    alpha defaults to 1/sqrt(D). bias_mode "constant": b = bias, default -ln L;
    "neg_log_nk": b_z = bias - ln n_k[z], bias default 0.
    tile_counts, if given, is an int32 device tensor of Z*H*ceil(L/BQ) entries.
    """
    _check_tensors(q, {"k": k, "v": v})
    Z, L, H, D = q.shape
    mode = _bias_mode(bias_mode)
    alpha = default_alpha(D) if alpha is None else float(alpha)
    bias = default_bias(L, mode) if bias is None else float(bias)
    nq, nk = _lengths(seqlens_q, Z, q.device), _lengths(seqlens_k, Z, q.device)
    o = torch.empty_like(q) if out is None else out
    _check_tensors(q, {"out": o})
    lib = _lib.load()
    tc = None if tile_counts is None else tile_counts.data_ptr()
    if mode == _lib.BIAS_CONSTANT:
        _lib.check(lib.sigattn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), nq.data_ptr(),
                                   nk.data_ptr(), Z, L, H, D, alpha, bias, _dtype_code(q), tc, _stream(q.device)))
    else:
        _lib.check(lib.sigattn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), nq.data_ptr(),
                                      nk.data_ptr(), _lib.LAYOUT_PADDED, mode, Z, L, H, D, alpha, bias,
                                      _dtype_code(q), tc, _stream(q.device)))
    return o


def sigattn_bwd(q, k, v, dout, seqlens_q, seqlens_k, alpha=None, bias=None, dq=None, dk=None, dv=None,
                tile_counts_dq=None, tile_counts_dkdv=None, bias_mode="constant"):
    """(dq, dk, dv) of sigmoid attention. Wraps the C entry point sigattn_bwd
    (sigattn_bwd_ex when the bias is per sample). Arguments as for sigattn_fwd."""
    _check_tensors(q, {"k": k, "v": v, "dout": dout})
    Z, L, H, D = q.shape
    mode = _bias_mode(bias_mode)
    alpha = default_alpha(D) if alpha is None else float(alpha)
    bias = default_bias(L, mode) if bias is None else float(bias)
    nq, nk = _lengths(seqlens_q, Z, q.device), _lengths(seqlens_k, Z, q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    _check_tensors(q, {"dq": dq, "dk": dk, "dv": dv})
    lib = _lib.load()
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    if mode == _lib.BIAS_CONSTANT:
        _lib.check(lib.sigattn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), dq.data_ptr(),
                                   dk.data_ptr(), dv.data_ptr(), nq.data_ptr(), nk.data_ptr(), Z, L, H, D, alpha,
                                   bias, _dtype_code(q), ptr(tile_counts_dq), ptr(tile_counts_dkdv),
                                   _stream(q.device)))
    else:
        _lib.check(lib.sigattn_bwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), dq.data_ptr(),
                                      dk.data_ptr(), dv.data_ptr(), nq.data_ptr(), nk.data_ptr(), _lib.LAYOUT_PADDED,
                                      mode, Z, L, H, D, alpha, bias, _dtype_code(q), ptr(tile_counts_dq),
                                      ptr(tile_counts_dkdv), _stream(q.device)))
    return dq, dk, dv


def _check_packed(q, k, named_q: dict, named_k: dict) -> None:
    if q.dim() != 3 or k.dim() != 3:
        raise ValueError("packed tensors must be [T, H, D]")
    if q.device.type != "cuda":
        raise ValueError("sigattn tensors must live on a HIP device")
    if k.shape[1:] != q.shape[1:] or k.dtype != q.dtype or k.device != q.device:
        raise ValueError("k must match q in H, D, dtype and device")
    for ref, named in ((q, named_q), (k, named_k)):
        for name, t in named.items():
            if t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device:
                raise ValueError(f"{name} must match {'q' if ref is q else 'k'} in shape, dtype and device")
    for t in (q, k, *named_q.values(), *named_k.values()):
        if not t.is_contiguous():
            raise ValueError("packed tensors must be contiguous [T, H, D]")


def _offsets(cu, device) -> torch.Tensor:
    t = cu if isinstance(cu, torch.Tensor) else torch.as_tensor(cu, dtype=torch.int32)
    if t.dtype != torch.int32 or t.dim() != 1 or t.numel() < 1:
        raise ValueError("cumulative offsets must be an int32[Z + 1] tensor")
    return t.to(device).contiguous()


def check_offsets(cu, rows: int, max_len: int, name: str = "cu_seqlens") -> None:
    """The packed layout's contract, checked on the host: offsets start at 0,
    never decrease, end at or below the tensor's row count, and give no sample
    more than max_len rows. The kernels read the offsets from device memory and
    trust them (an offset past the tensor would make them read and write out of
    bounds; a sample longer than max_len would leave its rows past max_len
    unwritten), so every packed entry point calls this first. A device tensor
    is copied to the host for the check, which synchronises with its stream."""
    c = (cu.detach().cpu() if isinstance(cu, torch.Tensor) else torch.as_tensor(cu)).to(torch.int64).reshape(-1)
    if c.numel() < 1:
        raise ValueError(f"{name} must hold Z + 1 offsets")
    if int(c[0]) != 0:
        raise ValueError(f"{name} must start at 0, got {int(c[0])}")
    d = c[1:] - c[:-1]
    if d.numel() and int(d.min()) < 0:
        raise ValueError(f"{name} must be non-decreasing")
    if int(c[-1]) > rows:
        raise ValueError(f"{name} ends at {int(c[-1])}, past the tensor's {rows} rows")
    if d.numel() and int(d.max()) > max_len:
        raise ValueError(f"{name}: a sample has {int(d.max())} rows, more than max_len = {max_len}")


def sigattn_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_len, alpha=None, bias=None, out=None,
                       tile_counts=None, bias_mode="constant"):
    """Sigmoid attention over packed sequences. Wraps sigattn_fwd_ex with the packed layout.

    q: [Tq, H, D], k and v: [Tk, H, D]; sample z owns rows cu_seqlens[z] ..
    cu_seqlens[z+1]-1. max_len bounds every length. alpha defaults to
    1/sqrt(D); bias as in sigattn_fwd, with L = max_len.
    """
    _check_packed(q, k, {}, {"v": v})
    H, D = q.shape[1], q.shape[2]
    cq, ck = _offsets(cu_seqlens_q, q.device), _offsets(cu_seqlens_k, q.device)
    if cq.numel() != ck.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold Z + 1 offsets")
    Z, L = cq.numel() - 1, int(max_len)
    check_offsets(cq, q.shape[0], L, "cu_seqlens_q")
    check_offsets(ck, k.shape[0], L, "cu_seqlens_k")
    mode = _bias_mode(bias_mode)
    alpha = default_alpha(D) if alpha is None else float(alpha)
    bias = default_bias(max(L, 1), mode) if bias is None else float(bias)
    o = torch.empty_like(q) if out is None else out
    _check_packed(q, k, {"out": o}, {})
    _lib.check(_lib.load().sigattn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), cq.data_ptr(),
                                          ck.data_ptr(), _lib.LAYOUT_PACKED, mode, Z, L, H, D, alpha, bias,
                                          _dtype_code(q), None if tile_counts is None else tile_counts.data_ptr(),
                                          _stream(q.device)))
    return o


def sigattn_bwd_varlen(q, k, v, dout, cu_seqlens_q, cu_seqlens_k, max_len, alpha=None, bias=None, dq=None, dk=None,
                       dv=None, tile_counts_dq=None, tile_counts_dkdv=None, bias_mode="constant"):
    """(dq, dk, dv) over packed sequences. Wraps sigattn_bwd_ex with the packed layout."""
    _check_packed(q, k, {"dout": dout}, {"v": v})
    H, D = q.shape[1], q.shape[2]
    cq, ck = _offsets(cu_seqlens_q, q.device), _offsets(cu_seqlens_k, q.device)
    if cq.numel() != ck.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold Z + 1 offsets")
    Z, L = cq.numel() - 1, int(max_len)
    check_offsets(cq, q.shape[0], L, "cu_seqlens_q")
    check_offsets(ck, k.shape[0], L, "cu_seqlens_k")
    mode = _bias_mode(bias_mode)
    alpha = default_alpha(D) if alpha is None else float(alpha)
    bias = default_bias(max(L, 1), mode) if bias is None else float(bias)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(k) if dv is None else dv
    _check_packed(q, k, {"dq": dq}, {"dk": dk, "dv": dv})
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    _lib.check(_lib.load().sigattn_bwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), dq.data_ptr(),
                                          dk.data_ptr(), dv.data_ptr(), cq.data_ptr(), ck.data_ptr(),
                                          _lib.LAYOUT_PACKED, mode, Z, L, H, D, alpha, bias, _dtype_code(q),
                                          ptr(tile_counts_dq), ptr(tile_counts_dkdv), _stream(q.device)))
    return dq, dk, dv


def sigattn_bwd_dkdv(q, k, v, dout, seqlens_q, seqlens_k, alpha=None, bias=None, dk=None, dv=None,
                     tile_counts_dkdv=None):
    """(dk, dv) only: one kernel launch. Wraps the C entry point sigattn_bwd_dkdv."""
    _check_tensors(q, {"k": k, "v": v, "dout": dout})
    Z, L, H, D = q.shape
    alpha = default_alpha(D) if alpha is None else float(alpha)
    bias = default_bias(L) if bias is None else float(bias)
    nq, nk = _lengths(seqlens_q, Z, q.device), _lengths(seqlens_k, Z, q.device)
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    _check_tensors(q, {"dk": dk, "dv": dv})
    lib = _lib.load()
    _lib.check(lib.sigattn_bwd_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), dk.data_ptr(),
                                    dv.data_ptr(), nq.data_ptr(), nk.data_ptr(), Z, L, H, D, alpha, bias,
                                    _dtype_code(q), None if tile_counts_dkdv is None else tile_counts_dkdv.data_ptr(),
                                    _stream(q.device)))
    return dk, dv


def sigattn_bwd_dq(q, k, v, dout, seqlens_q, seqlens_k, alpha=None, bias=None, dq=None, tile_counts_dq=None):
    """dq only: one kernel launch. Wraps the C entry point sigattn_bwd_dq."""
    _check_tensors(q, {"k": k, "v": v, "dout": dout})
    Z, L, H, D = q.shape
    alpha = default_alpha(D) if alpha is None else float(alpha)
    bias = default_bias(L) if bias is None else float(bias)
    nq, nk = _lengths(seqlens_q, Z, q.device), _lengths(seqlens_k, Z, q.device)
    dq = torch.empty_like(q) if dq is None else dq
    _check_tensors(q, {"dq": dq})
    lib = _lib.load()
    _lib.check(lib.sigattn_bwd_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), dq.data_ptr(),
                                  nq.data_ptr(), nk.data_ptr(), Z, L, H, D, alpha, bias, _dtype_code(q),
                                  None if tile_counts_dq is None else tile_counts_dq.data_ptr(), _stream(q.device)))
    return dq


def sigattn_bwd_dk(q, k, v, dout, seqlens_q, seqlens_k, alpha=None, bias=None, dk=None, tile_counts_dkdv=None):
    """dk only: one kernel launch. Wraps the C entry point sigattn_bwd_dk."""
    _check_tensors(q, {"k": k, "v": v, "dout": dout})
    Z, L, H, D = q.shape
    alpha = default_alpha(D) if alpha is None else float(alpha)
    bias = default_bias(L) if bias is None else float(bias)
    nq, nk = _lengths(seqlens_q, Z, q.device), _lengths(seqlens_k, Z, q.device)
    dk = torch.empty_like(q) if dk is None else dk
    _check_tensors(q, {"dk": dk})
    lib = _lib.load()
    _lib.check(lib.sigattn_bwd_dk(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), dk.data_ptr(),
                                  nq.data_ptr(), nk.data_ptr(), Z, L, H, D, alpha, bias, _dtype_code(q),
                                  None if tile_counts_dkdv is None else tile_counts_dkdv.data_ptr(),
                                  _stream(q.device)))
    return dk


def sigattn_bwd_dv(q, k, dout, seqlens_q, seqlens_k, alpha=None, bias=None, dv=None, tile_counts_dkdv=None):
    """dv only (v is not needed): one kernel launch. Wraps the C entry point sigattn_bwd_dv."""
    _check_tensors(q, {"k": k, "dout": dout})
    Z, L, H, D = q.shape
    alpha = default_alpha(D) if alpha is None else float(alpha)
    bias = default_bias(L) if bias is None else float(bias)
    nq, nk = _lengths(seqlens_q, Z, q.device), _lengths(seqlens_k, Z, q.device)
    dv = torch.empty_like(q) if dv is None else dv
    _check_tensors(q, {"dv": dv})
    lib = _lib.load()
    _lib.check(lib.sigattn_bwd_dv(q.data_ptr(), k.data_ptr(), dout.data_ptr(), dv.data_ptr(), nq.data_ptr(),
                                  nk.data_ptr(), Z, L, H, D, alpha, bias, _dtype_code(q),
                                  None if tile_counts_dkdv is None else tile_counts_dkdv.data_ptr(),
                                  _stream(q.device)))
    return dv


def sigattn_tile_config(kernel: int, D: int, dtype) -> tuple:
    code = dtype if isinstance(dtype, int) else _DTYPES[dtype]
    return _lib.tile_config(kernel, D, code)


class SigmoidAttention(torch.autograd.Function):
    """Autograd wrapper. The forward saves only its inputs, since the backward
    recomputes P and needs neither O nor any row statistic."""

    @staticmethod
    def forward(ctx, q, k, v, seqlens_q, seqlens_k, alpha=None, bias=None, bias_mode="constant"):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        Z, L, H, D = q.shape
        nq = _lengths(seqlens_q, Z, q.device)
        nk = _lengths(seqlens_k, Z, q.device)
        mode = _bias_mode(bias_mode)
        alpha = default_alpha(D) if alpha is None else float(alpha)
        bias = default_bias(L, mode) if bias is None else float(bias)
        ctx.save_for_backward(q, k, v, nq, nk)
        ctx.scalars = (alpha, bias, mode)
        return sigattn_fwd(q, k, v, nq, nk, alpha, bias, bias_mode=mode)

    @staticmethod
    def backward(ctx, grad_out):
        q, k, v, nq, nk = ctx.saved_tensors
        alpha, bias, mode = ctx.scalars
        dq, dk, dv = sigattn_bwd(q, k, v, grad_out.contiguous(), nq, nk, alpha, bias, bias_mode=mode)
        return dq, dk, dv, None, None, None, None, None


def sigmoid_attention(q, k, v, seqlens_q, seqlens_k, alpha=None, bias=None, bias_mode="constant"):
    """Differentiable padding-aware sigmoid attention over [Z, L, H, D] tensors."""
    return SigmoidAttention.apply(q, k, v, seqlens_q, seqlens_k, alpha, bias, bias_mode)


class SigmoidAttentionVarlen(torch.autograd.Function):
    """Autograd wrapper over packed [T, H, D] sequences."""

    @staticmethod
    def forward(ctx, q, k, v, cu_seqlens_q, cu_seqlens_k, max_len, alpha=None, bias=None, bias_mode="constant"):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        cq, ck = _offsets(cu_seqlens_q, q.device), _offsets(cu_seqlens_k, q.device)
        mode = _bias_mode(bias_mode)
        alpha = default_alpha(q.shape[2]) if alpha is None else float(alpha)
        bias = default_bias(max(int(max_len), 1), mode) if bias is None else float(bias)
        ctx.save_for_backward(q, k, v, cq, ck)
        ctx.scalars = (int(max_len), alpha, bias, mode)
        return sigattn_fwd_varlen(q, k, v, cq, ck, max_len, alpha, bias, bias_mode=mode)

    @staticmethod
    def backward(ctx, grad_out):
        q, k, v, cq, ck = ctx.saved_tensors
        max_len, alpha, bias, mode = ctx.scalars
        dq, dk, dv = sigattn_bwd_varlen(q, k, v, grad_out.contiguous(), cq, ck, max_len, alpha, bias,
                                        bias_mode=mode)
        return dq, dk, dv, None, None, None, None, None, None


def sigmoid_attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_len, alpha=None, bias=None,
                             bias_mode="constant"):
    """Differentiable sigmoid attention over packed [T, H, D] sequences."""
    return SigmoidAttentionVarlen.apply(q, k, v, cu_seqlens_q, cu_seqlens_k, max_len, alpha, bias, bias_mode)


# ------------------------------------------------------------------------------------- softmax attention


def _softmax_layout(q, k, seq_q, seq_k, max_len, named_q: dict, named_k: dict):
    """(layout, Z, L, seq_q, seq_k): padded [Z, L, H, D] tensors with lengths, or
    packed [T, H, D] tensors with int32[Z + 1] offsets and max_len."""
    if q.dim() == 4:
        _check_tensors(q, {"k": k, **named_q, **named_k})
        Z, L = q.shape[0], q.shape[1]
        return _lib.LAYOUT_PADDED, Z, L, _lengths(seq_q, Z, q.device), _lengths(seq_k, Z, q.device)
    if max_len is None:
        raise ValueError("packed [T, H, D] tensors need max_len")
    _check_packed(q, k, named_q, named_k)
    cq, ck = _offsets(seq_q, q.device), _offsets(seq_k, q.device)
    if cq.numel() != ck.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold Z + 1 offsets")
    check_offsets(cq, q.shape[0], int(max_len), "cu_seqlens_q")
    check_offsets(ck, k.shape[0], int(max_len), "cu_seqlens_k")
    return _lib.LAYOUT_PACKED, cq.numel() - 1, int(max_len), cq, ck


def _check_lse(lse, q):
    want = q.shape[:-1]
    if lse.shape != want or lse.dtype != torch.float32 or lse.device != q.device or not lse.is_contiguous():
        raise ValueError(f"lse must be a contiguous float32 tensor of shape {tuple(want)} on q's device")


def sigattn_softmax_fwd(q, k, v, seq_q, seq_k, alpha=None, out=None, lse=None, max_len=None):
    """(O, LSE) of padding-aware softmax attention. Wraps sigattn_softmax_fwd.

    Padded: q, k, v [Z, L, H, D], seq_* int32[Z] lengths. Packed: q [Tq, H, D],
    k, v [Tk, H, D], seq_* int32[Z + 1] offsets, max_len bounding every length.
    LSE (natural log, fp32) has q's shape without D. alpha defaults to 1/sqrt(D).
    """
    layout, Z, L, sq, sk = _softmax_layout(q, k, seq_q, seq_k, max_len, {}, {"v": v})
    H, D = q.shape[-2], q.shape[-1]
    alpha = default_alpha(D) if alpha is None else float(alpha)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty(q.shape[:-1], dtype=torch.float32, device=q.device) if lse is None else lse
    if o.shape != q.shape or o.dtype != q.dtype or o.device != q.device or not o.is_contiguous():
        raise ValueError("out must match q in shape, dtype and device and be contiguous")
    _check_lse(lse, q)
    _lib.check(_lib.load().sigattn_softmax_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                               lse.data_ptr(), sq.data_ptr(), sk.data_ptr(), layout, Z, L, H, D,
                                               alpha, _dtype_code(q), _stream(q.device)))
    return o, lse


def sigattn_softmax_bwd(q, k, v, o, dout, lse, seq_q, seq_k, alpha=None, dq=None, dk=None, dv=None, max_len=None,
                        workspace=None):
    """(dq, dk, dv) of padding-aware softmax attention from the forward's O and
    LSE. Wraps sigattn_softmax_bwd; layouts as for sigattn_softmax_fwd. The
    workspace (rows_q * H * 8 bytes) is allocated here unless given."""
    layout, Z, L, sq, sk = _softmax_layout(q, k, seq_q, seq_k, max_len, {"o": o, "dout": dout}, {"v": v})
    H, D = q.shape[-2], q.shape[-1]
    alpha = default_alpha(D) if alpha is None else float(alpha)
    _check_lse(lse, q)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(k) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, k)):
        if t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device or not t.is_contiguous():
            raise ValueError(f"{name} must match {'q' if ref is q else 'k'} in shape, dtype and device")
    lib = _lib.load()
    rows = q.shape[0] * q.shape[1] if layout == _lib.LAYOUT_PADDED else q.shape[0]
    nbytes = lib.sigattn_softmax_bwd_workspace_size(rows, H)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    elif workspace.numel() * workspace.element_size() < nbytes:
        raise ValueError(f"workspace needs {nbytes} bytes")
    _lib.check(lib.sigattn_softmax_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                                       lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), sq.data_ptr(),
                                       sk.data_ptr(), layout, Z, L, H, D, alpha, _dtype_code(q),
                                       workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                       _stream(q.device)))
    return dq, dk, dv


def sigattn_softmax_bwd_noalloc(q, k, v, o, dout, lse, seq_q, seq_k, alpha=None, dq=None, dk=None, dv=None,
                                max_len=None):
    """sigattn_softmax_bwd with the library's fixed device buffer for the row
    statistics instead of a workspace (wraps sigattn_softmax_bwd_noalloc): the
    C call allocates nothing. Z * L * H must not exceed NOALLOC_ROWS, and calls
    that overlap on one GPU race. Pass dq, dk and dv to allocate nothing here
    either."""
    layout, Z, L, sq, sk = _softmax_layout(q, k, seq_q, seq_k, max_len, {"o": o, "dout": dout}, {"v": v})
    H, D = q.shape[-2], q.shape[-1]
    alpha = default_alpha(D) if alpha is None else float(alpha)
    _check_lse(lse, q)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(k) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, k)):
        if t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device or not t.is_contiguous():
            raise ValueError(f"{name} must match {'q' if ref is q else 'k'} in shape, dtype and device")
    _lib.check(_lib.load().sigattn_softmax_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                                       dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                                       dv.data_ptr(), sq.data_ptr(), sk.data_ptr(), layout, Z, L, H, D,
                                                       alpha, _dtype_code(q), _stream(q.device)))
    return dq, dk, dv


class SoftmaxAttention(torch.autograd.Function):
    """Autograd wrapper of the softmax path. The forward saves its inputs, O and
    LSE; the backward recomputes P from them."""

    @staticmethod
    def forward(ctx, q, k, v, seq_q, seq_k, alpha=None, max_len=None):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        layout, _, _, sq, sk = _softmax_layout(q, k, seq_q, seq_k, max_len, {}, {"v": v})
        alpha = default_alpha(q.shape[-1]) if alpha is None else float(alpha)
        o, lse = sigattn_softmax_fwd(q, k, v, sq, sk, alpha, max_len=max_len)
        ctx.save_for_backward(q, k, v, o, lse, sq, sk)
        ctx.scalars = (alpha, max_len)
        ctx.mark_non_differentiable(lse)
        return o, lse

    @staticmethod
    def backward(ctx, grad_out, grad_lse):
        q, k, v, o, lse, sq, sk = ctx.saved_tensors
        alpha, max_len = ctx.scalars
        dq, dk, dv = sigattn_softmax_bwd(q, k, v, o, grad_out.contiguous(), lse, sq, sk, alpha, max_len=max_len)
        return dq, dk, dv, None, None, None, None


def softmax_attention(q, k, v, seq_q, seq_k, alpha=None, max_len=None):
    """Differentiable padding-aware softmax attention: returns O (LSE is not
    differentiated). Padded [Z, L, H, D] with lengths, or packed [T, H, D] with
    offsets and max_len."""
    return SoftmaxAttention.apply(q, k, v, seq_q, seq_k, alpha, max_len)[0]


# ------------------------------------------------------------------------------------------ FP8 path

_FP8_TILE = 64


def _fp8_layout(x, seq, max_len):
    """(layout, Z, L, seq tensor) of an FP8-path tensor: padded [Z, L, H, D] with
    int32[Z] lengths, or packed [T, H, D] with int32[Z + 1] offsets and max_len."""
    if x.device.type != "cuda":
        raise ValueError("sigattn tensors must live on a HIP device")
    if x.dim() == 4:
        if not x.is_contiguous():
            raise ValueError("tensors must be contiguous [Z, L, H, D]")
        return _lib.LAYOUT_PADDED, x.shape[0], x.shape[1], _lengths(seq, x.shape[0], x.device)
    if x.dim() != 3 or not x.is_contiguous():
        raise ValueError("packed tensors must be contiguous [T, H, D]")
    if max_len is None:
        raise ValueError("packed [T, H, D] tensors need max_len")
    cu = _offsets(seq, x.device)
    check_offsets(cu, x.shape[0], int(max_len))
    return _lib.LAYOUT_PACKED, cu.numel() - 1, int(max_len), cu


def sigattn_quantize_fp8(x, seq, max_len=None, out=None, scales=None):
    """(codes, scales) of a bf16 tensor: OCP E4M3 codes (uint8, x's layout) and
    one E8M0 scale byte per (sample, head, 64-row tile), uint8 [Z, H, ceil(L/64)].
    Wraps sigattn_quantize_fp8. Padded [Z, L, H, D] with lengths, or packed
    [T, H, D] with offsets and max_len."""
    if x.dtype != torch.bfloat16:
        raise TypeError("sigattn_quantize_fp8 takes a bfloat16 tensor")
    layout, Z, L, sq = _fp8_layout(x, seq, max_len)
    H, D = x.shape[-2], x.shape[-1]
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if out is None else out
    nt = -(-L // _FP8_TILE)
    sc = torch.empty((Z, H, nt), dtype=torch.uint8, device=x.device) if scales is None else scales
    if codes.shape != x.shape or codes.dtype != torch.uint8 or not codes.is_contiguous():
        raise ValueError("out must be a contiguous uint8 tensor of x's shape")
    if sc.shape != (Z, H, nt) or sc.dtype != torch.uint8 or not sc.is_contiguous():
        raise ValueError(f"scales must be a contiguous uint8 tensor of shape {(Z, H, nt)}")
    _lib.check(_lib.load().sigattn_quantize_fp8(x.data_ptr(), codes.data_ptr(), sc.data_ptr(), sq.data_ptr(),
                                                layout, Z, L, H, D, _stream(x.device)))
    return codes, sc


def sigattn_fwd_fp8(q8, k8, v8, sq, sk, sv, seq_q, seq_k, alpha=None, bias=None, out=None, max_len=None,
                    bias_mode="constant"):
    """O (bf16) = sigma(alpha Q K^T + b) V on E4M3 operands with per-tile E8M0
    scales (as sigattn_quantize_fp8 returns them), P quantised per query row and
    64-key tile. Wraps sigattn_fwd_fp8. alpha defaults to 1/sqrt(D); bias as in
    sigattn_fwd, with L = max_len for packed tensors."""
    layout, Z, L, cq = _fp8_layout(q8, seq_q, max_len)
    _, _, _, ck = _fp8_layout(k8, seq_k, max_len)
    H, D = q8.shape[-2], q8.shape[-1]
    for name, t, ref in (("k8", k8, k8), ("v8", v8, k8)):
        if t.dtype != torch.uint8 or t.shape != ref.shape or t.shape[-2:] != q8.shape[-2:]:
            raise ValueError(f"{name} must be uint8 codes of k's shape with q's H and D")
    if q8.dtype != torch.uint8:
        raise ValueError("q8 must hold uint8 codes")
    nt = -(-L // _FP8_TILE)
    for name, t in (("sq", sq), ("sk", sk), ("sv", sv)):
        if t.shape != (Z, H, nt) or t.dtype != torch.uint8 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous uint8 tensor of shape {(Z, H, nt)}")
    mode = _bias_mode(bias_mode)
    alpha = default_alpha(D) if alpha is None else float(alpha)
    bias = default_bias(max(L, 1), mode) if bias is None else float(bias)
    o = torch.empty(q8.shape, dtype=torch.bfloat16, device=q8.device) if out is None else out
    if o.shape != q8.shape or o.dtype != torch.bfloat16 or not o.is_contiguous():
        raise ValueError("out must be a contiguous bfloat16 tensor of q's shape")
    _lib.check(_lib.load().sigattn_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), sq.data_ptr(),
                                           sk.data_ptr(), sv.data_ptr(), o.data_ptr(), cq.data_ptr(), ck.data_ptr(),
                                           layout, mode, Z, L, H, D, alpha, bias, _stream(q8.device)))
    return o
