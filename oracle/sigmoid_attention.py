"""CPU oracle for fused, padding-aware, non-causal sigmoid attention.

TEST INFRASTRUCTURE. Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The library's
HIP path never imports, links or calls it, and this module imports nothing
from the library. It shares no code with the GPU path.

Plain NumPy in float64. Inputs in any float dtype are upcast exactly.

Sources. Every formula below is restated from these summary pages of
"Better Models, Faster Training: Sigmoid Attention for single-cell Foundation
Models" (arXiv:2604.27124):

* rainbus.top summary, section "方法步骤详情" (method steps), steps 1-5:
  - the Z x L x H x D tensors and per-sample lengths n_q, n_k (step 1);
  - the scores S = alpha * Q K^T + b (step 2);
  - -inf at padded key positions, and wholly padded query blocks written as
    zeros (step 2);
  - the elementwise sigmoid, then accumulation into the output (step 3);
  - the backward dS = P (1 - P) (dO V^T), with dK/dV taken in the
    transposed view (step 4).
* gist.science summary, section 2.A: the logistic function
  sigma(x) = 1 / (1 + e^{-x}) and the forward sigma(Q K^T / sqrt(d) + b) V.
* paperlayer.ai summary, section 3: the bias b = -log(n), taken either as one
  scalar for the batch or per sample, b_z = -log(n_k[z]).
* Per-sample lengths (rainbus.top summary, "方法步骤详情" step 1), and cells
  attended one by one, never split or concatenated with other cells
  (paperlayer.ai summary, section 1). The packed (varlen) layout used by
  forward_varlen and backward_varlen stores the samples' valid rows back to
  back, with cumulative offsets, in place of padding. That storage variant is
  this library's own; the pages do not describe it. Attention stays per sample,
  so the results are those of the padded layout on the same valid rows.

Readings taken where the pages are silent:

* A key j >= n_k gets weight exactly 0. The -inf score is read as a select,
  not an addition.
* Query rows i >= n_q are outputs defined as the constant 0. dO on those rows
  therefore has no effect, and their dQ rows are 0.
* dK and dV rows j >= n_k are 0.
* dQ = alpha dS K, dK = alpha dS^T Q and dV = P^T dO come from the chain rule
  applied to the forward above.
* Padding is a suffix: positions [0, n) are valid.
* Padded inputs are never read, so their contents, even NaN, cannot matter.

Parity status: every public function here is pinned by tests that check it
against closed forms, finite differences, a hand-worked example, torch's
autograd and the pages' invariants. See tests/test_oracle_pins.py.
"""

from __future__ import annotations

import math

import numpy as np

# Arithmetic the oracle can run in. float64 is the oracle: every parity check
# and pin uses it. float32 is a timing mode for the CPU baseline only (the
# same steps in single precision, a fairer CPU number than float64).
TIMING_DTYPES = (np.float64, np.float32)

# Rows per dense block when a head is too large to hold its full n_q x n_k
# score matrix. Each block is the dense definition applied to a slice of
# independent rows, so no sum is split or reordered.
_MAX_BLOCK_ELEMS = 1 << 24


def sigmoid(x, dtype=np.float64):
    """Logistic function sigma(x) = 1 / (1 + e^{-x}), elementwise, float64.

    The formula is the one in the gist.science summary, section 2.A. It is
    evaluated in the two algebraically equal forms that never overflow:
    1 / (1 + e^{-x}) for x >= 0 and e^{x} / (1 + e^{x}) for x < 0.
    dtype float32 is the CPU-timing mode (see TIMING_DTYPES); every check
    uses float64.
    """
    x = np.asarray(x, dtype=dtype)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def scores(qv, kv, alpha, bias, dtype=np.float64):
    """Scores S = alpha * Q K^T + b for one (sample, head), valid rows only.

    From the rainbus.top summary, "方法步骤详情" step 2, and the gist.science
    summary, section 2.A. qv is [n_q, D] and kv is [n_k, D]. Returns [n_q, n_k].
    """
    return dtype(alpha) * (np.asarray(qv, dtype) @ np.asarray(kv, dtype).T) + dtype(bias)


def head_forward(qv, kv, vv, alpha, bias, dtype=np.float64):
    """O = sigma(S) V for one (sample, head) on its valid rows.

    From the rainbus.top summary, "方法步骤详情" steps 2-3. There is no row
    normalisation: each weight is an independent sigmoid (paperlayer.ai
    summary, section 3).
    """
    p = sigmoid(scores(qv, kv, alpha, bias, dtype=dtype), dtype=dtype)
    return p @ np.asarray(vv, dtype)


def head_backward(qv, kv, vv, dov, alpha, bias, return_intermediates=False, dtype=np.float64):
    """Gradients of O = sigma(alpha Q K^T + b) V for one (sample, head).

    The forward is recomputed (P = sigma(S)), as in the rainbus.top summary,
    "方法步骤详情" step 5. Then:
      dP = dO V^T
      dS = P * (1 - P) * dP                    (step 4)
      dQ = alpha dS K                          (chain rule)
      dK = alpha dS^T Q                        (step 4, the transposed view)
      dV = P^T dO                              (chain rule)
    All inputs cover valid rows only: qv, dov are [n_q, D]; kv, vv are [n_k, D].
    """
    qv = np.asarray(qv, dtype)
    kv = np.asarray(kv, dtype)
    vv = np.asarray(vv, dtype)
    dov = np.asarray(dov, dtype)
    s = scores(qv, kv, alpha, bias, dtype=dtype)
    p = sigmoid(s, dtype=dtype)
    dp = dov @ vv.T
    ds = p * (1.0 - p) * dp
    dq = dtype(alpha) * (ds @ kv)
    dk = dtype(alpha) * (ds.T @ qv)
    dv = p.T @ dov
    if return_intermediates:
        return dq, dk, dv, {"S": s, "P": p, "dP": dp, "dS": ds}
    return dq, dk, dv


def per_sample_bias(seqlens_k, bias=0.0):
    """b_z = bias - ln(n_k[z]) for every sample z (paperlayer.ai summary,
    section 3: b = -log n with n the sample's own length). A sample with no
    key gets bias (ln 1), which no score ever uses."""
    n = np.asarray(seqlens_k, dtype=np.float64).reshape(-1)
    return float(bias) - np.log(np.maximum(n, 1.0))


def _bias_at(bias, z, Z):
    """The bias of sample z: bias is one scalar, or an array of Z per-sample values."""
    b = np.asarray(bias, dtype=np.float64)
    if b.ndim == 0:
        return float(b)
    b = b.reshape(-1)
    if b.shape[0] != Z:
        raise ValueError(f"a per-sample bias needs Z={Z} values, got {b.shape[0]}")
    return float(b[z])


def _check_lengths(seqlens, Z, L, name):
    n = np.asarray(seqlens, dtype=np.int64).reshape(-1)
    if n.shape[0] != Z:
        raise ValueError(f"{name} has {n.shape[0]} entries, expected Z={Z}")
    if (n < 0).any() or (n > L).any():
        raise ValueError(f"{name} must lie in [0, L={L}]")
    return n


def _check_qkv(q, k, v):
    q = np.asarray(q)
    if q.ndim != 4:
        raise ValueError("q must be [Z, L, H, D]")
    for t in (k, v):
        if np.asarray(t).shape != q.shape:
            raise ValueError("q, k and v must share the shape [Z, L, H, D]")
    return q.shape


def _row_blocks(n_rows, n_other):
    step = max(1, _MAX_BLOCK_ELEMS // max(1, n_other))
    return [(s, min(s + step, n_rows)) for s in range(0, n_rows, step)]


def forward(q, k, v, seqlens_q, seqlens_k, alpha, bias, dtype=np.float64):
    """Padding-aware forward over the whole batch: O[z, :, h, :] for every z, h.

    Q, K, V are [Z, L, H, D] (rainbus.top summary, "方法步骤详情" step 1).
    For sample z only the prefixes Q[z, :n_q[z]], K[z, :n_k[z]] and
    V[z, :n_k[z]] are read. Rows i >= n_q[z] of O are 0. bias is one scalar
    or Z per-sample values (see per_sample_bias). Returns float64 (dtype:
    the CPU-timing mode, see TIMING_DTYPES).
    """
    Z, L, H, D = _check_qkv(q, k, v)
    nq = _check_lengths(seqlens_q, Z, L, "seqlens_q")
    nk = _check_lengths(seqlens_k, Z, L, "seqlens_k")
    o = np.zeros((Z, L, H, D), dtype)
    for z in range(Z):
        a, b = int(nq[z]), int(nk[z])
        for h in range(H):
            kv = k[z, :b, h, :]
            vv = v[z, :b, h, :]
            for r0, r1 in _row_blocks(a, b):
                o[z, r0:r1, h, :] = head_forward(q[z, r0:r1, h, :], kv, vv, alpha, _bias_at(bias, z, Z), dtype=dtype)
    return o


def backward(q, k, v, do, seqlens_q, seqlens_k, alpha, bias, dtype=np.float64):
    """Padding-aware backward over the whole batch. Returns (dQ, dK, dV), float64.

    Each dQ row depends on its own query row and on all valid keys, so dQ is
    taken in blocks of query rows. Each dK/dV row depends on its own key row
    and on all valid queries, so dK and dV are taken in blocks of key rows.
    Every block applies head_backward's dense definition to its slice, and no
    sum is split. dQ rows >= n_q and dK, dV rows >= n_k are 0.
    """
    Z, L, H, D = _check_qkv(q, k, v)
    if np.asarray(do).shape != (Z, L, H, D):
        raise ValueError("do must be [Z, L, H, D]")
    nq = _check_lengths(seqlens_q, Z, L, "seqlens_q")
    nk = _check_lengths(seqlens_k, Z, L, "seqlens_k")
    dq = np.zeros((Z, L, H, D), dtype)
    dk = np.zeros((Z, L, H, D), dtype)
    dv = np.zeros((Z, L, H, D), dtype)
    for z in range(Z):
        a, b = int(nq[z]), int(nk[z])
        for h in range(H):
            qv, kv, vv, dov = q[z, :a, h, :], k[z, :b, h, :], v[z, :b, h, :], do[z, :a, h, :]
            bz = _bias_at(bias, z, Z)
            for r0, r1 in _row_blocks(a, b):
                dq[z, r0:r1, h, :] = head_backward(qv[r0:r1], kv, vv, dov[r0:r1], alpha, bz, dtype=dtype)[0]
            for c0, c1 in _row_blocks(b, a):
                _, dkb, dvb = head_backward(qv, kv[c0:c1], vv[c0:c1], dov, alpha, bz, dtype=dtype)
                dk[z, c0:c1, h, :] = dkb
                dv[z, c0:c1, h, :] = dvb
    return dq, dk, dv


def forward_rows(q, k, v, seqlens_q, seqlens_k, alpha, bias, z, h, rows):
    """O[z, rows, h, :] exactly, without computing the other rows.

    Each output row depends only on its own query row, so this is the dense
    definition applied to the selected rows. Rows >= n_q[z] give 0.
    """
    Z, L, H, D = _check_qkv(q, k, v)
    nq = _check_lengths(seqlens_q, Z, L, "seqlens_q")
    nk = _check_lengths(seqlens_k, Z, L, "seqlens_k")
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.shape[0], D), np.float64)
    live = rows < nq[z]
    if live.any():
        b = int(nk[z])
        out[live] = head_forward(q[z, rows[live], h, :], k[z, :b, h, :], v[z, :b, h, :], alpha,
                                 _bias_at(bias, z, Z))
    return out


def backward_rows(q, k, v, do, seqlens_q, seqlens_k, alpha, bias, z, h, q_rows, k_rows):
    """dQ[z, q_rows, h], dK[z, k_rows, h] and dV[z, k_rows, h] exactly.

    dQ row i needs only query row i and every valid key. dK/dV row j needs
    only key row j and every valid query. Rows past the valid prefix give 0.
    """
    Z, L, H, D = _check_qkv(q, k, v)
    nq = _check_lengths(seqlens_q, Z, L, "seqlens_q")
    nk = _check_lengths(seqlens_k, Z, L, "seqlens_k")
    a, b = int(nq[z]), int(nk[z])
    q_rows = np.asarray(q_rows, dtype=np.int64)
    k_rows = np.asarray(k_rows, dtype=np.int64)
    dq = np.zeros((q_rows.shape[0], D), np.float64)
    dk = np.zeros((k_rows.shape[0], D), np.float64)
    dv = np.zeros((k_rows.shape[0], D), np.float64)
    qv, kv, vv, dov = q[z, :a, h, :], k[z, :b, h, :], v[z, :b, h, :], do[z, :a, h, :]
    bz = _bias_at(bias, z, Z)
    lq = q_rows < a
    if lq.any():
        dq[lq] = head_backward(q[z, q_rows[lq], h, :], kv, vv, do[z, q_rows[lq], h, :], alpha, bz)[0]
    lk = k_rows < b
    if lk.any():
        _, dkb, dvb = head_backward(qv, k[z, k_rows[lk], h, :], v[z, k_rows[lk], h, :], dov, alpha, bz)
        dk[lk] = dkb
        dv[lk] = dvb
    return dq, dk, dv


def tile_plan(seqlens_q, seqlens_k, L, block_q, block_k):
    """Which tile pairs a padding-aware kernel computes.

    A tile is skipped when it lies wholly in padding, for query blocks and key
    blocks alike (rainbus.top summary, "方法步骤详情" step 2; gist.science
    summary, section 2.C). A block is live when at least one of its rows is
    valid. Tiles are found here by walking the rows of each block.

    Returns (pairs_per_qtile, pairs_per_ktile):
    * pairs_per_qtile[z, m] counts the live key blocks paired with query
      block m, or is 0 when query block m is wholly padding;
    * pairs_per_ktile[z, t] is the same with the roles swapped.
    """
    nq = np.asarray(seqlens_q, dtype=np.int64).reshape(-1)
    nk = np.asarray(seqlens_k, dtype=np.int64).reshape(-1)
    Z = nq.shape[0]
    n_qt = -(-L // block_q)
    n_kt = -(-L // block_k)
    by_q = np.zeros((Z, n_qt), np.int64)
    by_k = np.zeros((Z, n_kt), np.int64)
    for z in range(Z):
        q_live = [any(r < nq[z] for r in range(m * block_q, min(L, (m + 1) * block_q))) for m in range(n_qt)]
        k_live = [any(r < nk[z] for r in range(t * block_k, min(L, (t + 1) * block_k))) for t in range(n_kt)]
        for m in range(n_qt):
            for t in range(n_kt):
                if q_live[m] and k_live[t]:
                    by_q[z, m] += 1
                    by_k[z, t] += 1
    return by_q, by_k


def _check_offsets(cu, name):
    cu = np.asarray(cu, dtype=np.int64).reshape(-1)
    if cu.shape[0] < 1 or cu[0] != 0 or (np.diff(cu) < 0).any():
        raise ValueError(f"{name} must be non-decreasing offsets starting at 0")
    return cu


def pack(x, seqlens):
    """The packed layout of a padded [Z, L, ...] array: the valid prefixes
    x[z, :n[z]] back to back, [sum n, ...]. Data movement only."""
    x = np.asarray(x)
    n = np.asarray(seqlens, dtype=np.int64).reshape(-1)
    return np.concatenate([x[z, : int(n[z])] for z in range(x.shape[0])], axis=0)


def unpack(xp, cu, L):
    """The padded layout of a packed array: [Z, L, ...] with sample z's rows
    cu[z] .. cu[z+1]-1 at positions 0 .. n-1 and zeros after. Data movement only."""
    xp = np.asarray(xp)
    cu = _check_offsets(cu, "cu")
    out = np.zeros((cu.shape[0] - 1, L) + xp.shape[1:], np.float64)
    for z in range(cu.shape[0] - 1):
        n = int(cu[z + 1] - cu[z])
        if n > L:
            raise ValueError(f"sample {z} has {n} rows, more than L={L}")
        out[z, :n] = xp[int(cu[z]) : int(cu[z + 1])]
    return out


def forward_varlen(q, k, v, cu_q, cu_k, alpha, bias):
    """The forward over packed sequences. q is [Tq, H, D] and k, v are
    [Tk, H, D]. Sample z's queries are rows cu_q[z] .. cu_q[z+1]-1 and its keys
    rows cu_k[z] .. cu_k[z+1]-1, all valid. Each (z, h) slice is the dense
    definition. bias is one scalar or Z per-sample values. Returns float64
    [Tq, H, D]."""
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    cu_q, cu_k = _check_offsets(cu_q, "cu_q"), _check_offsets(cu_k, "cu_k")
    Z, H = cu_q.shape[0] - 1, q.shape[1]
    o = np.zeros(q.shape, np.float64)
    for z in range(Z):
        q0, q1, k0, k1 = int(cu_q[z]), int(cu_q[z + 1]), int(cu_k[z]), int(cu_k[z + 1])
        for h in range(H):
            for r0, r1 in _row_blocks(q1 - q0, k1 - k0):
                o[q0 + r0 : q0 + r1, h] = head_forward(q[q0 + r0 : q0 + r1, h], k[k0:k1, h], v[k0:k1, h], alpha,
                                                        _bias_at(bias, z, Z))
    return o


def backward_varlen(q, k, v, do, cu_q, cu_k, alpha, bias):
    """The backward over packed sequences: (dQ [Tq, H, D], dK and dV [Tk, H, D]),
    float64. Layout and bias as in forward_varlen."""
    q, k, v, do = np.asarray(q), np.asarray(k), np.asarray(v), np.asarray(do)
    cu_q, cu_k = _check_offsets(cu_q, "cu_q"), _check_offsets(cu_k, "cu_k")
    Z, H = cu_q.shape[0] - 1, q.shape[1]
    dq = np.zeros(q.shape, np.float64)
    dk = np.zeros(k.shape, np.float64)
    dv = np.zeros(k.shape, np.float64)
    for z in range(Z):
        q0, q1, k0, k1 = int(cu_q[z]), int(cu_q[z + 1]), int(cu_k[z]), int(cu_k[z + 1])
        bz = _bias_at(bias, z, Z)
        for h in range(H):
            qv, kv, vv, dov = q[q0:q1, h], k[k0:k1, h], v[k0:k1, h], do[q0:q1, h]
            for r0, r1 in _row_blocks(q1 - q0, k1 - k0):
                dq[q0 + r0 : q0 + r1, h] = head_backward(qv[r0:r1], kv, vv, dov[r0:r1], alpha, bz)[0]
            for c0, c1 in _row_blocks(k1 - k0, q1 - q0):
                _, dkb, dvb = head_backward(qv, kv[c0:c1], vv[c0:c1], dov, alpha, bz)
                dk[k0 + c0 : k0 + c1, h] = dkb
                dv[k0 + c0 : k0 + c1, h] = dvb
    return dq, dk, dv


def default_scalars(D, L):
    """alpha = 1/sqrt(D) (gist.science summary, section 2.A) and b = -log(L).

    b = -log(n) comes from the paperlayer.ai summary, section 3. n is read
    here as the padded length L, with a natural log.
    """
    return 1.0 / math.sqrt(D), -math.log(L)
