"""CPU oracle for the FP8 forward of padding-aware sigmoid attention.

TEST INFRASTRUCTURE. Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The library's HIP
path never imports, links or calls it, and this module imports nothing from
the library. It shares no code with the GPU path.

Plain NumPy in float64.

Sources: the pages name FP8/INT8 quantisation as future work for the kernel
(rainbus.top summary of arXiv:2604.27124, section "未来方向"; paperlayer.ai
summary, section 5) and give no scheme. The forward computed here is the
sigmoid forward of the rest of the oracle (gist.science summary, section 2.A;
rainbus.top summary, "方法步骤详情", steps 1-3) on quantised operands.

Readings taken where the pages are silent:

* Format: OCP FP8 E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7,
  3 mantissa bits, subnormals with step 2^-9, largest finite value 448, no
  infinities (code 0x7f / 0xff is NaN).
* Rounding: to nearest, ties to even, in every conversion.
* Inputs Q, K, V are quantised per tile of 64 rows of one (sample, head),
  rows counted from the sample's first row, valid rows only. A tile's scale
  is a power of two 2^E with E = floor(log2 amax) - 7, so the largest
  magnitude maps into [128, 256) and no code overflows; E = 0 for an all-zero
  tile; E >= -127. The scale is stored as the byte E + 127 (the E8M0
  encoding). Codes of padded rows are 0.
* The forward dequantises exactly (code value * 2^E), forms S = alpha Q K^T +
  b and P = sigma(S) as the sigmoid oracle does, then quantises P once more
  before P V: per query row and per tile of 64 keys, with the power-of-two
  scale 2^e, e = floor(log2 m) - 7, m the largest P over the valid keys of
  that tile (e = 0 when m = 0). O = sum over tiles of 2^e * e4m3(P 2^-e) V.
  Rows i >= n_q of O are 0.

Parity status: every public function here is pinned by tests/oracle_pins.py
(format values from the OCP definition, closed forms, exact scaling laws and
the quantisation error bound).
"""

from __future__ import annotations

import numpy as np

from .sigmoid_attention import _check_lengths, _check_qkv, sigmoid

E4M3_MAX = 448.0
TILE = 64  # rows per quantisation tile, and keys per P tile


def e4m3_round(x):
    """x rounded to the nearest OCP E4M3 value, ties to even (float64 in, float64 out).

    |x| must not exceed 448 after rounding. Normal values 2^E * 1.mmm have a
    step of 2^(E-3); below the smallest normal 2^-6 the step is 2^-9."""
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    _, ex = np.frexp(a)  # a = f * 2^ex, f in [0.5, 1): floor(log2 a) = ex - 1
    step = np.where(a >= 2.0**-6, np.ldexp(1.0, ex - 1 - 3), 2.0**-9)
    q = np.rint(a / step) * step  # np.rint rounds half to even; a / step is exact (power of two)
    if np.any(q > E4M3_MAX):
        raise ValueError("value outside the E4M3 range")
    return np.copysign(q, x)


def e4m3_decode(code):
    """float64 values of E4M3 codes (uint8). NaN codes (0x7f, 0xff) give NaN."""
    c = np.asarray(code, np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0**-9, np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e4m3_encode(x):
    """E4M3 codes (uint8) of values that are already on the E4M3 grid (e4m3_round output)."""
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    _, ex = np.frexp(a)
    normal = a >= 2.0**-6
    e = np.where(normal, ex - 1 + 7, 0)
    m = np.where(normal, np.rint((a / np.ldexp(1.0, ex - 1) - 1.0) * 8.0), np.rint(a / 2.0**-9))
    code = (e.astype(np.int64) << 3) | m.astype(np.int64)
    code = np.where(a == 0, 0, code)
    code = code | np.where(np.signbit(x), 0x80, 0)
    return code.astype(np.uint8)


def tile_exponent(amax):
    """E = floor(log2 amax) - 7 (amax * 2^-E in [128, 256)), 0 for amax = 0, never below -127."""
    amax = np.asarray(amax, np.float64)
    _, ex = np.frexp(amax)
    e = np.where(amax > 0, ex - 1 - 7, 0)
    return np.maximum(e, -127).astype(np.int64)


def quantize(x, seqlens, tile=TILE):
    """Per-tile E4M3 quantisation of a [Z, L, H, D] tensor.

    Returns (codes uint8 [Z, L, H, D], scale bytes uint8 [Z, H, ceil(L / tile)]).
    Tile m of (z, h) holds rows m*tile .. m*tile + tile - 1 below n[z]; its
    byte is E + 127. Codes of rows >= n[z] are 0."""
    x = np.asarray(x, np.float64)
    Z, L, H, D = x.shape
    n = _check_lengths(seqlens, Z, L, "seqlens")
    nt = -(-L // tile)
    codes = np.zeros((Z, L, H, D), np.uint8)
    sbytes = np.full((Z, H, nt), 127, np.uint8)
    for z in range(Z):
        for h in range(H):
            for m in range(nt):
                r0, r1 = m * tile, min((m + 1) * tile, int(n[z]))
                if r1 <= r0:
                    continue
                blk = x[z, r0:r1, h]
                e = int(tile_exponent(np.max(np.abs(blk))))
                codes[z, r0:r1, h] = e4m3_encode(e4m3_round(np.ldexp(blk, -e)))
                sbytes[z, h, m] = e + 127
    return codes, sbytes


def dequantize(codes, sbytes, tile=TILE):
    """float64 [Z, L, H, D] values of per-tile E4M3 codes."""
    v = e4m3_decode(codes)
    Z, L, H, D = v.shape
    e = np.asarray(sbytes, np.int64) - 127                      # [Z, H, nt]
    rows = np.repeat(e, tile, axis=2)[:, :, :L]                 # [Z, H, L]
    return np.ldexp(v, rows.transpose(0, 2, 1)[..., None])


def quantize_p(p, tile=TILE):
    """P of one query row block [rows, n_k] quantised per row and per tile of
    `tile` keys: 2^e * e4m3(P 2^-e), e from the tile's largest P."""
    p = np.asarray(p, np.float64)
    out = np.empty_like(p)
    for t0 in range(0, p.shape[1], tile):
        blk = p[:, t0:t0 + tile]
        e = tile_exponent(blk.max(axis=1))[:, None]
        out[:, t0:t0 + tile] = np.ldexp(e4m3_round(np.ldexp(blk, -e)), e)
    return out


def head_forward(qv, kv, vv, alpha, bias):
    """O of one (sample, head) slice: dequantised operands (float64), P = sigma(S)
    over the valid keys, quantised per query row and key tile, then P V."""
    qv, kv, vv = (np.asarray(t, np.float64) for t in (qv, kv, vv))
    if kv.shape[0] == 0:
        return np.zeros((qv.shape[0], vv.shape[1]))
    p = sigmoid(alpha * (qv @ kv.T) + bias)
    return quantize_p(p) @ vv


def forward(q8, k8, v8, sq, sk, sv, seqlens_q, seqlens_k, alpha, bias):
    """FP8 forward over the batch: O float64 [Z, L, H, D] from E4M3 codes and
    per-tile scale bytes (as `quantize` returns them). bias: a scalar or one
    per sample. Rows i >= n_q are 0."""
    Q, K, V = dequantize(q8, sq), dequantize(k8, sk), dequantize(v8, sv)
    Z, L, H, D = _check_qkv(Q, K, V)
    nq = _check_lengths(seqlens_q, Z, L, "seqlens_q")
    nk = _check_lengths(seqlens_k, Z, L, "seqlens_k")
    b = np.broadcast_to(np.asarray(bias, np.float64), (Z,))
    o = np.zeros((Z, L, H, D), np.float64)
    for z in range(Z):
        a, c = int(nq[z]), int(nk[z])
        for h in range(H):
            if a > 0:
                o[z, :a, h] = head_forward(Q[z, :a, h], K[z, :c, h], V[z, :c, h], alpha, b[z])
    return o


def forward_rows(q8, k8, v8, sq, sk, sv, seqlens_q, seqlens_k, alpha, bias, z, h, rows):
    """O[z, rows, h, :] exactly; rows >= n_q give 0."""
    Z, L, H, D = np.asarray(q8).shape
    nq = _check_lengths(seqlens_q, Z, L, "seqlens_q")
    nk = _check_lengths(seqlens_k, Z, L, "seqlens_k")
    b = np.broadcast_to(np.asarray(bias, np.float64), (Z,))
    rows = np.asarray(rows, np.int64)
    out = np.zeros((rows.shape[0], D), np.float64)
    live = rows < nq[z]
    if live.any():
        c = int(nk[z])
        qz = dequantize(np.asarray(q8)[z:z + 1], np.asarray(sq)[z:z + 1])[0]
        kz = dequantize(np.asarray(k8)[z:z + 1], np.asarray(sk)[z:z + 1])[0]
        vz = dequantize(np.asarray(v8)[z:z + 1], np.asarray(sv)[z:z + 1])[0]
        out[live] = head_forward(qz[rows[live], h], kz[:c, h], vz[:c, h], alpha, b[z])
    return out
