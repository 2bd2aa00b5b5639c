"""CPU oracle for padding-aware, non-causal softmax attention.

TEST INFRASTRUCTURE. Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The library's HIP
path never imports, links or calls it, and this module imports nothing from
the library. It shares no code with the GPU path.

Plain NumPy in float64. Inputs in any float dtype are upcast exactly.

Sources (summary pages of "Better Models, Faster Training: Sigmoid Attention
for single-cell Foundation Models", arXiv:2604.27124):

* rainbus.top summary, "前置知识" (prerequisites), entries "自注意力机制" and
  "Softmax 归一化": attention weights are the softmax over keys of the scaled
  scores Q K^T / sqrt(d), softmax(a)_i = e^{a_i} / sum_j e^{a_j}, and the output
  is the weighted sum of V.
* rainbus.top summary, "未来方向": carrying the padding-aware kernel design
  over to softmax attention. The padding semantics are therefore those of the
  sigmoid oracle: only keys j < n_k[z] take part, query rows i >= n_q[z] are
  outputs defined as 0, and padded inputs are never read.

Readings taken where the pages are silent:

* A score bias b adds the same constant to a whole row, which softmax removes,
  so the softmax path has no bias argument.
* The row's log-sum-exp LSE_i = log sum_{j < n_k} e^{S_ij} is an output of the
  forward (the backward needs it). A row with no key (n_k = 0) has no
  distribution: its output row and its LSE are 0, and so are its gradients.
  Padded query rows have LSE 0.
* The backward is the chain rule through the softmax:
  dP = dO V^T, D_i = sum_d dO_id O_id (= sum_j P_ij dP_ij),
  dS = P (dP - D), dQ = alpha dS K, dK = alpha dS^T Q, dV = P^T dO.

Parity status: every public function here is pinned by tests/oracle_pins.py
(closed forms, torch's softmax, finite differences, row-sum invariants).
"""

from __future__ import annotations

import numpy as np

from .sigmoid_attention import _check_lengths, _check_qkv, _row_blocks


def head_forward(qv, kv, vv, alpha):
    """(O, LSE) of one (sample, head) slice over its valid rows.

    S = alpha Q K^T; each row's weights are softmax(S_i) over the keys
    (rainbus.top summary, 前置知识, "Softmax 归一化"), taken with the row
    maximum subtracted first so that e^x never overflows; O = P V;
    LSE_i = max_i + log sum_j e^{S_ij - max_i}. With no key, O and LSE are 0.
    """
    qv, kv, vv = (np.asarray(t, np.float64) for t in (qv, kv, vv))
    if kv.shape[0] == 0:
        return np.zeros((qv.shape[0], vv.shape[1])), np.zeros(qv.shape[0])
    s = alpha * (qv @ kv.T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    den = e.sum(axis=1, keepdims=True)
    p = e / den
    return p @ vv, (m + np.log(den))[:, 0]


def head_backward(qv, kv, vv, dov, alpha):
    """(dQ, dK, dV) of one slice: P recomputed from the scores, then the chain
    rule through the row softmax with D_i = sum_j P_ij dP_ij."""
    qv, kv, vv, dov = (np.asarray(t, np.float64) for t in (qv, kv, vv, dov))
    if kv.shape[0] == 0 or qv.shape[0] == 0:
        return np.zeros(qv.shape), np.zeros(kv.shape), np.zeros(vv.shape)
    s = alpha * (qv @ kv.T)
    e = np.exp(s - s.max(axis=1, keepdims=True))
    p = e / e.sum(axis=1, keepdims=True)
    dp = dov @ vv.T
    d = (p * dp).sum(axis=1, keepdims=True)
    ds = p * (dp - d)
    return alpha * (ds @ kv), alpha * (ds.T @ qv), p.T @ dov


def forward(q, k, v, seqlens_q, seqlens_k, alpha):
    """Padding-aware softmax forward over the batch: (O [Z, L, H, D], LSE [Z, H, L]).

    For sample z only Q[z, :n_q], K[z, :n_k] and V[z, :n_k] are read. Rows
    i >= n_q of O and LSE are 0. Each output row depends only on its own query
    row, so rows are taken in blocks with no sum split."""
    Z, L, H, D = _check_qkv(q, k, v)
    nq = _check_lengths(seqlens_q, Z, L, "seqlens_q")
    nk = _check_lengths(seqlens_k, Z, L, "seqlens_k")
    o = np.zeros((Z, L, H, D), np.float64)
    lse = np.zeros((Z, H, L), np.float64)
    for z in range(Z):
        a, b = int(nq[z]), int(nk[z])
        for h in range(H):
            for r0, r1 in _row_blocks(a, b):
                o[z, r0:r1, h], lse[z, h, r0:r1] = head_forward(q[z, r0:r1, h], k[z, :b, h], v[z, :b, h], alpha)
    return o, lse


def _dkdv_by_key_blocks(qv, kv, vv, dov, alpha, lse, dvec):
    """dK and dV of one slice, taken in blocks of key rows. A softmax row spans
    every key, so each block uses the row statistics instead of renormalising:
    P_ij = e^{S_ij - LSE_i} (the definition of LSE), and D_i = dO_i . O_i
    (= sum_j P_ij dP_ij, since O_i = sum_j P_ij V_j). Then dS = P (dP - D),
    dK = alpha dS^T Q and dV = P^T dO, block by block with no sum split."""
    a, b = qv.shape[0], kv.shape[0]
    dk = np.zeros(kv.shape, np.float64)
    dv = np.zeros(vv.shape, np.float64)
    for c0, c1 in _row_blocks(b, a):
        s = alpha * (qv @ kv[c0:c1].T)
        p = np.exp(s - lse[:, None])
        dp = dov @ vv[c0:c1].T
        ds = p * (dp - dvec[:, None])
        dk[c0:c1] = alpha * (ds.T @ qv)
        dv[c0:c1] = p.T @ dov
    return dk, dv


def _slice_stats(qv, kv, vv, dov, alpha):
    """(LSE, D) of every valid query row of one slice, from the forward in row blocks."""
    a, b = qv.shape[0], kv.shape[0]
    lse = np.zeros(a, np.float64)
    o = np.zeros((a, vv.shape[1]), np.float64)
    for r0, r1 in _row_blocks(a, b):
        o[r0:r1], lse[r0:r1] = head_forward(qv[r0:r1], kv, vv, alpha)
    return lse, (dov * o).sum(axis=1)


def backward(q, k, v, do, seqlens_q, seqlens_k, alpha):
    """Padding-aware softmax backward: (dQ, dK, dV), float64, [Z, L, H, D].

    dQ rows depend on their own query row and all valid keys: query-row blocks
    of the dense definition. dK/dV rows depend on their own key row and on
    every valid query's whole softmax row: key-row blocks through the row
    statistics (see _dkdv_by_key_blocks). Padded rows are 0."""
    Z, L, H, D = _check_qkv(q, k, v)
    nq = _check_lengths(seqlens_q, Z, L, "seqlens_q")
    nk = _check_lengths(seqlens_k, Z, L, "seqlens_k")
    dq = np.zeros((Z, L, H, D), np.float64)
    dk = np.zeros((Z, L, H, D), np.float64)
    dv = np.zeros((Z, L, H, D), np.float64)
    for z in range(Z):
        a, b = int(nq[z]), int(nk[z])
        if a == 0 or b == 0:
            continue
        for h in range(H):
            qv, kv, vv, dov = (np.asarray(t[z, :n, h], np.float64) for t, n in ((q, a), (k, b), (v, b), (do, a)))
            for r0, r1 in _row_blocks(a, b):
                dq[z, r0:r1, h] = head_backward(qv[r0:r1], kv, vv, dov[r0:r1], alpha)[0]
            lse, dvec = _slice_stats(qv, kv, vv, dov, alpha)
            dk[z, :b, h], dv[z, :b, h] = _dkdv_by_key_blocks(qv, kv, vv, dov, alpha, lse, dvec)
    return dq, dk, dv


def forward_rows(q, k, v, seqlens_q, seqlens_k, alpha, z, h, rows):
    """(O[z, rows, h, :], LSE[z, h, rows]) exactly; rows >= n_q give 0."""
    Z, L, H, D = _check_qkv(q, k, v)
    nq = _check_lengths(seqlens_q, Z, L, "seqlens_q")
    nk = _check_lengths(seqlens_k, Z, L, "seqlens_k")
    rows = np.asarray(rows, dtype=np.int64)
    o = np.zeros((rows.shape[0], D), np.float64)
    lse = np.zeros(rows.shape[0], np.float64)
    live = rows < nq[z]
    if live.any():
        b = int(nk[z])
        o[live], lse[live] = head_forward(q[z, rows[live], h], k[z, :b, h], v[z, :b, h], alpha)
    return o, lse


def backward_rows(q, k, v, do, seqlens_q, seqlens_k, alpha, z, h, q_rows, k_rows):
    """dQ[z, q_rows, h], dK[z, k_rows, h] and dV[z, k_rows, h] exactly. dK/dV
    rows need every valid query's row statistics, taken over the whole slice."""
    Z, L, H, D = _check_qkv(q, k, v)
    nq = _check_lengths(seqlens_q, Z, L, "seqlens_q")
    nk = _check_lengths(seqlens_k, Z, L, "seqlens_k")
    a, b = int(nq[z]), int(nk[z])
    q_rows = np.asarray(q_rows, dtype=np.int64)
    k_rows = np.asarray(k_rows, dtype=np.int64)
    dq = np.zeros((q_rows.shape[0], D), np.float64)
    dk = np.zeros((k_rows.shape[0], D), np.float64)
    dv = np.zeros((k_rows.shape[0], D), np.float64)
    if a == 0 or b == 0:
        return dq, dk, dv
    qv, kv, vv, dov = (np.asarray(t[z, :n, h], np.float64) for t, n in ((q, a), (k, b), (v, b), (do, a)))
    lq = q_rows < a
    if lq.any():
        dq[lq] = head_backward(qv[q_rows[lq]], kv, vv, dov[q_rows[lq]], alpha)[0]
    lk = k_rows < b
    if lk.any():
        lse, dvec = _slice_stats(qv, kv, vv, dov, alpha)
        dk[lk], dv[lk] = _dkdv_by_key_blocks(qv, kv[k_rows[lk]], vv[k_rows[lk]], dov, alpha, lse, dvec)
    return dq, dk, dv
