"""Plant plausible mistakes in the CPU oracle and check that some pin catches each.

The mistakes are planted with monkeypatch on the CPU. Each one is a slip a
person could make writing the oracle: a dropped term, a wrong sign, a wrong
index, a transposed or swapped operand, an off-by-one in the mask. Every
mutant must make at least one pin in tests/oracle_pins.py fail.
"""

import math

import numpy as np
import pytest

import oracle_pins
from oracle import fp8_attention as f8a
from oracle import sigmoid_attention as osa
from oracle import softmax_attention as sma

_orig_scores = osa.scores
_orig_sigmoid = osa.sigmoid
_orig_head_backward = osa.head_backward
_orig_forward = osa.forward
_orig_backward = osa.backward
_orig_tile_plan = osa.tile_plan
_orig_bias_at = osa._bias_at
_orig_per_sample_bias = osa.per_sample_bias
_orig_forward_varlen = osa.forward_varlen
_orig_backward_varlen = osa.backward_varlen
_orig_sm_head_forward = sma.head_forward
_orig_sm_dkdv = sma._dkdv_by_key_blocks


def _sm_forward(variant):
    def f(qv, kv, vv, alpha):
        qv, kv, vv = (np.asarray(t, np.float64) for t in (qv, kv, vv))
        if kv.shape[0] == 0:
            return np.zeros((qv.shape[0], vv.shape[1])), np.zeros(qv.shape[0])
        s = alpha * (qv @ kv.T)
        if variant == "softmax over queries":
            m = s.max(axis=0, keepdims=True)
            e = np.exp(s - m)
            p = e / e.sum(axis=0, keepdims=True)
            return p @ vv, (m.max() + np.log(e.sum(axis=1)))
        m = s.max(axis=1, keepdims=True) if variant != "softmax without max" else 0.0
        e = np.exp(s - m)
        den = e.sum(axis=1, keepdims=True)
        lse = np.log(den)[:, 0] if variant == "LSE without max" else (m + np.log(den))[:, 0]
        return (e / den) @ vv, lse

    return f


def _sm_dkdv(variant):
    def f(qv, kv, vv, dov, alpha, lse, dvec):
        a, b = qv.shape[0], kv.shape[0]
        dk = np.zeros(kv.shape)
        dv = np.zeros(vv.shape)
        for c0, c1 in osa._row_blocks(b, a):
            s = alpha * (qv @ kv[c0:c1].T)
            if variant == "key blocks renormalised":
                e = np.exp(s - s.max(axis=1, keepdims=True))
                p = e / e.sum(axis=1, keepdims=True)
            else:
                p = np.exp(s - lse[:, None])
            dp = dov @ vv[c0:c1].T
            ds = p * dp if variant == "dS drops D" else p * (dp - dvec[:, None])
            dk[c0:c1] = alpha * (ds.T @ qv)
            dv[c0:c1] = p.T @ dov
        return dk, dv

    return f


def _varlen_fwd(variant):
    """A packed forward that gets the offsets wrong."""

    def f(q, k, v, cu_q, cu_k, alpha, bias):
        q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
        cu_q, cu_k = np.asarray(cu_q).astype(int), np.asarray(cu_k).astype(int)
        o = np.zeros(q.shape)
        Z = cu_q.shape[0] - 1
        for z in range(Z):
            q0, q1, k0, k1 = cu_q[z], cu_q[z + 1], cu_k[z], cu_k[z + 1]
            if variant == "varlen keys use query offsets":
                k0, k1 = min(cu_q[z], k.shape[0]), min(cu_q[z + 1], k.shape[0])
            if variant == "varlen keys shifted by one":
                k0, k1 = min(k0 + 1, k.shape[0]), min(k1 + 1, k.shape[0])
            for h in range(q.shape[1]):
                if q1 > q0:
                    o[q0:q1, h] = osa.head_forward(q[q0:q1, h], k[k0:k1, h], v[k0:k1, h], alpha,
                                                   osa._bias_at(bias, z, Z))
        return o

    return f


def _hb(variant):
    """A head_backward with one planted mistake."""

    def f(qv, kv, vv, dov, alpha, bias, return_intermediates=False, dtype=np.float64):
        qv, kv, vv, dov = (np.asarray(t, np.float64) for t in (qv, kv, vv, dov))
        s = osa.scores(qv, kv, alpha, bias)
        p = osa.sigmoid(s)
        dp = dov @ (kv.T if variant == "dP uses K" else vv.T)
        if variant == "dS drops (1-P)":
            ds = p * dp
        elif variant == "dS sign":
            ds = -p * (1.0 - p) * dp
        else:
            ds = p * (1.0 - p) * dp
        dq = (1.0 if variant == "dQ drops alpha" else alpha) * (ds @ (vv if variant == "dQ uses V" else kv))
        dk = alpha * (ds.T @ (dov if variant == "dK uses dO" else qv))
        if variant == "dV uses 1-P":
            dv = (1.0 - p).T @ dov
        elif variant == "dV uses Q":
            dv = p.T @ qv
        else:
            dv = p.T @ dov
        if variant == "dK scaled by alpha twice":
            dk = alpha * dk
        if return_intermediates:
            return dq, dk, dv, {"S": s, "P": p, "dP": dp, "dS": ds}
        return dq, dk, dv

    return f


def _forward_mask(variant):
    """A full-batch forward that gets the padding wrong."""

    def f(q, k, v, seqlens_q, seqlens_k, alpha, bias, dtype=np.float64):
        Z, L, H, D = np.asarray(q).shape
        nq = np.asarray(seqlens_q).astype(int)
        nk = np.asarray(seqlens_k).astype(int)
        o = np.zeros((Z, L, H, D))
        for z in range(Z):
            a = L if variant == "padded queries not zeroed" else nq[z]
            b = {"keys masked with n_q": nq[z], "one padded key read": min(L, nk[z] + 1)}.get(variant, nk[z])
            for h in range(H):
                o[z, :a, h] = osa.head_forward(q[z, :a, h], k[z, :b, h], v[z, :b, h], alpha, bias)
        return o

    return f


def _backward_mask(variant):
    def f(q, k, v, do, seqlens_q, seqlens_k, alpha, bias, dtype=np.float64):
        Z, L, H, D = np.asarray(q).shape
        nq = np.asarray(seqlens_q).astype(int)
        nk = np.asarray(seqlens_k).astype(int)
        out = [np.zeros((Z, L, H, D)) for _ in range(3)]
        for z in range(Z):
            a, b = nq[z], nk[z]
            bk = L if variant == "padded keys get gradients" else b
            for h in range(H):
                dq, _, _ = osa.head_backward(q[z, :a, h], k[z, :b, h], v[z, :b, h], do[z, :a, h], alpha, bias)
                _, dk, dv = osa.head_backward(q[z, :a, h], k[z, :bk, h], v[z, :bk, h], do[z, :a, h], alpha, bias)
                out[0][z, :a, h] = dq
                out[1][z, :bk, h] = dk
                out[2][z, :bk, h] = dv
        return tuple(out)

    return f


def _tile_plan_off_by_one(seqlens_q, seqlens_k, L, block_q, block_k):
    nq = np.asarray(seqlens_q).reshape(-1)
    nk = np.asarray(seqlens_k).reshape(-1)
    n_qt, n_kt = -(-L // block_q), -(-L // block_k)
    by_q = np.zeros((nq.shape[0], n_qt), np.int64)
    by_k = np.zeros((nq.shape[0], n_kt), np.int64)
    for z in range(nq.shape[0]):
        for m in range(n_qt):
            for t in range(n_kt):
                if m * block_q <= nq[z] and t * block_k <= nk[z]:  # "<=" instead of "<"
                    by_q[z, m] += 1
                    by_k[z, t] += 1
    return by_q, by_k


# ------------------------------------------------------------------ FP8 path mutants
_orig_quantize_p = f8a.quantize_p
_orig_dequantize = f8a.dequantize
_orig_quantize = f8a.quantize
_orig_e4m3_round = f8a.e4m3_round
_orig_tile_exponent = f8a.tile_exponent


def _round_ties_away(x):
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    _, ex = np.frexp(a)
    step = np.where(a >= 2.0**-6, np.ldexp(1.0, ex - 1 - 3), 2.0**-9)
    return np.copysign(np.floor(a / step + 0.5) * step, x)


def _round_no_subnormals(x):
    r = _orig_e4m3_round(x)
    return np.where(np.abs(r) < 2.0**-6, 0.0, r)


def _dequantize_tile32(codes, sbytes, tile=64):
    return _orig_dequantize(codes, sbytes, 32)


def _quantize_padding_too(x, seqlens, tile=64):
    x = np.asarray(x, np.float64)
    full = np.full(x.shape[0], x.shape[1])
    return _orig_quantize(x, full, tile)


def _fp8_forward_keys_by_nq(q8, k8, v8, sq, sk, sv, seqlens_q, seqlens_k, alpha, bias):
    return _orig_fp8_forward(q8, k8, v8, sq, sk, sv, seqlens_q, seqlens_q, alpha, bias)


_orig_fp8_forward = f8a.forward


MUTANTS = {
    "bias dropped": ("scores", lambda qv, kv, a, b, dtype=np.float64: a * (np.asarray(qv, float) @ np.asarray(kv, float).T)),
    "alpha dropped": ("scores", lambda qv, kv, a, b, dtype=np.float64: (np.asarray(qv, float) @ np.asarray(kv, float).T) + b),
    "bias sign": ("scores", lambda qv, kv, a, b, dtype=np.float64: a * (np.asarray(qv, float) @ np.asarray(kv, float).T) - b),
    "scores use Q Q^T": ("scores", lambda qv, kv, a, b, dtype=np.float64: a * (np.asarray(qv, float) @ np.asarray(qv, float).T[:, : np.asarray(kv).shape[0]]) + b
                         if np.asarray(qv).shape[0] >= np.asarray(kv).shape[0] else _orig_scores(qv, kv, a, b) * 1.01),
    "sigma sign": ("sigmoid", lambda x, dtype=np.float64: _orig_sigmoid(-np.asarray(x, float))),
    "sigma of 2x (tanh slip)": ("sigmoid", lambda x, dtype=np.float64: _orig_sigmoid(2.0 * np.asarray(x, float))),
    "sigma without exp": ("sigmoid", lambda x, dtype=np.float64: 1.0 / (1.0 + np.abs(np.asarray(x, float)))),
    "dS drops (1-P)": ("head_backward", _hb("dS drops (1-P)")),
    "dS sign": ("head_backward", _hb("dS sign")),
    "dP uses K": ("head_backward", _hb("dP uses K")),
    "dQ drops alpha": ("head_backward", _hb("dQ drops alpha")),
    "dQ uses V": ("head_backward", _hb("dQ uses V")),
    "dK uses dO": ("head_backward", _hb("dK uses dO")),
    "dK scaled by alpha twice": ("head_backward", _hb("dK scaled by alpha twice")),
    "dV uses 1-P": ("head_backward", _hb("dV uses 1-P")),
    "dV uses Q": ("head_backward", _hb("dV uses Q")),
    "padded queries not zeroed": ("forward", _forward_mask("padded queries not zeroed")),
    "keys masked with n_q": ("forward", _forward_mask("keys masked with n_q")),
    "one padded key read": ("forward", _forward_mask("one padded key read")),
    "padded keys get gradients": ("backward", _backward_mask("padded keys get gradients")),
    "tile plan off by one": ("tile_plan", _tile_plan_off_by_one),
    "per-sample bias sign": ("per_sample_bias", lambda n, bias=0.0: float(bias) + np.log(np.maximum(
        np.asarray(n, float).reshape(-1), 1.0))),
    "per-sample bias log2": ("per_sample_bias", lambda n, bias=0.0: float(bias) - np.log2(np.maximum(
        np.asarray(n, float).reshape(-1), 1.0))),
    "bias of the wrong sample": ("_bias_at", lambda bias, z, Z: _orig_bias_at(bias, (z + 1) % Z, Z)),
    "varlen keys use query offsets": ("forward_varlen", _varlen_fwd("varlen keys use query offsets")),
    "varlen keys shifted by one": ("forward_varlen", _varlen_fwd("varlen keys shifted by one")),
    "softmax over queries": ("sm:head_forward", _sm_forward("softmax over queries")),
    "softmax without max": ("sm:head_forward", _sm_forward("softmax without max")),
    "LSE without max": ("sm:head_forward", _sm_forward("LSE without max")),
    "key blocks renormalised": ("sm:_dkdv_by_key_blocks", _sm_dkdv("key blocks renormalised")),
    "dS drops D": ("sm:_dkdv_by_key_blocks", _sm_dkdv("dS drops D")),
    "P not quantised": ("f8:quantize_p", lambda p, tile=64: np.asarray(p, np.float64)),
    "P tiles of 32 keys": ("f8:quantize_p", lambda p, tile=64: _orig_quantize_p(p, 32)),
    "P scaled over the whole row": ("f8:quantize_p", lambda p, tile=64: _orig_quantize_p(p, max(1, np.shape(p)[1]))),
    "e4m3 ties away from zero": ("f8:e4m3_round", _round_ties_away),
    "e4m3 flushes subnormals": ("f8:e4m3_round", _round_no_subnormals),
    "tile scale one binade low": ("f8:tile_exponent", lambda amax: _orig_tile_exponent(amax) + 1),
    "dequantised by 32-row tiles": ("f8:dequantize", _dequantize_tile32),
    "padded rows quantised": ("f8:quantize", _quantize_padding_too),
    "fp8 keys masked with n_q": ("f8:forward", _fp8_forward_keys_by_nq),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    module = osa
    if attr.startswith("sm:"):
        module, attr = sma, attr[3:]
    elif attr.startswith("f8:"):
        module, attr = f8a, attr[3:]
    monkeypatch.setattr(module, attr, fn)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake '{name}'"


def test_unmutated_oracle_passes_every_pin():
    for pin in oracle_pins.ALL_PINS:
        pin()
    assert math.isfinite(float(osa.sigmoid(np.array([0.0]))[0]))
