"""Pins that tie the CPU oracle to something other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with:
* a closed form;
* the hand-worked example under tests/golden;
* finite differences;
* torch's autograd;
* an invariant the pages state.

The functions reach the oracle only through module attribute lookups
(``osa.forward`` etc.). tests/test_oracle_mutations.py can therefore
monkeypatch a planted mistake into the oracle and check that some pin fails.
"""

from __future__ import annotations

import json
import math
import pathlib

import numpy as np

from oracle import fp8_attention as f8a
from oracle import sigmoid_attention as osa
from oracle import softmax_attention as sma

GOLDEN = pathlib.Path(__file__).parent / "golden"


def _close(a, b, rtol=1e-12, atol=1e-12, what=""):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    assert np.allclose(a, b, rtol=rtol, atol=atol), f"{what}: max diff {np.max(np.abs(a - b))}"


def _case(rng, Z, L, H, D, nq, nk, scale=1.0):
    q = rng.standard_normal((Z, L, H, D)) * scale
    k = rng.standard_normal((Z, L, H, D)) * scale
    v = rng.standard_normal((Z, L, H, D))
    do = rng.standard_normal((Z, L, H, D))
    return q, k, v, do, np.array(nq), np.array(nk)


# --------------------------------------------------------------------------- sigma
def pin_sigmoid_closed_forms():
    """sigma(0) = 1/2 and sigma(+-ln 3) = 3/4, 1/4. It saturates to exactly 0
    or 1 without overflow. sigma(-x) = 1 - sigma(x)."""
    l3 = math.log(3.0)
    x = np.array([0.0, l3, -l3, 800.0, -800.0, 30.0, -30.0])
    want = [0.5, 0.75, 0.25, 1.0, 0.0, 1.0 / (1.0 + math.exp(-30.0)), math.exp(-30.0) / (1.0 + math.exp(-30.0))]
    _close(osa.sigmoid(x), want, rtol=1e-15, atol=0, what="sigma closed forms")
    r = np.random.default_rng(1).standard_normal(1000) * 8
    _close(osa.sigmoid(-r), 1.0 - osa.sigmoid(r), rtol=0, atol=2e-16, what="sigma symmetry")
    assert np.all(np.diff(osa.sigmoid(np.linspace(-50, 50, 2001))) >= 0), "sigma not monotone"


def pin_derivative_bound():
    """sigma' = sigma (1 - sigma) <= 1/4. So every |dS_ij| <= |dP_ij| / 4,
    including at huge scores (rainbus.top summary, 核心方法; paperlayer.ai §3)."""
    rng = np.random.default_rng(2)
    for scale in (1.0, 4.0, 16.0):
        qv = rng.standard_normal((40, 8)) * scale
        kv = rng.standard_normal((33, 8)) * scale
        vv = rng.standard_normal((33, 8))
        dov = rng.standard_normal((40, 8))
        _, _, _, it = osa.head_backward(qv, kv, vv, dov, 0.35, -2.0, return_intermediates=True)
        p = it["P"]
        assert np.all(p * (1 - p) <= 0.25), "sigma' above 1/4"
        assert np.all(np.abs(it["dS"]) <= np.abs(it["dP"]) / 4 + 1e-300), "|dS| above |dP|/4"
        _close(it["S"], 0.35 * qv @ kv.T - 2.0, rtol=1e-13, atol=1e-13, what="scores")


def pin_lipschitz_quarter():
    """sigma is 1/4-Lipschitz in the scores: ||sigma(S1)-sigma(S2)||_F <= ||S1-S2||_F / 4
    (paperlayer.ai summary, A.1.2)."""
    rng = np.random.default_rng(3)
    for _ in range(50):
        s1 = rng.standard_normal((16, 16)) * rng.uniform(0.1, 20)
        s2 = s1 + rng.standard_normal((16, 16)) * rng.uniform(1e-3, 5)
        lhs = np.linalg.norm(osa.sigmoid(s1) - osa.sigmoid(s2))
        assert lhs <= 0.25 * np.linalg.norm(s1 - s2) * (1 + 1e-12), "sigma not 1/4-Lipschitz"


# --------------------------------------------------------------------------- closed forms
def pin_q_zero_closed_form():
    """With Q = 0 every score equals b. Then, for i < n_q and j < n_k:
      O_i  = sigma(b) * sum_j V_j
      dK_j = 0
      dV_j = sigma(b) * sum_i dO_i
      dQ_i = alpha sigma(b)(1 - sigma(b)) * sum_j (dO_i . V_j) K_j
    Every padded row is 0."""
    rng = np.random.default_rng(4)
    Z, L, H, D = 2, 12, 2, 3
    nq, nk = [12, 7], [9, 12]
    alpha, bias = 0.7, -1.3
    _, k, v, do, nq, nk = _case(rng, Z, L, H, D, nq, nk)
    q = np.zeros_like(k)
    sb = 1.0 / (1.0 + math.exp(1.3))
    o_w = np.zeros((Z, L, H, D))
    dq_w = np.zeros((Z, L, H, D))
    dv_w = np.zeros((Z, L, H, D))
    for z in range(Z):
        for h in range(H):
            a, b = nq[z], nk[z]
            o_w[z, :a, h] = sb * v[z, :b, h].sum(0)
            dv_w[z, :b, h] = sb * do[z, :a, h].sum(0)
            for i in range(a):
                acc = np.zeros(D)
                for j in range(b):
                    acc += float(do[z, i, h] @ v[z, j, h]) * k[z, j, h]
                dq_w[z, i, h] = alpha * sb * (1 - sb) * acc
    _close(osa.forward(q, k, v, nq, nk, alpha, bias), o_w, what="O with Q=0")
    dq, dk, dv = osa.backward(q, k, v, do, nq, nk, alpha, bias)
    _close(dq, dq_w, what="dQ with Q=0")
    _close(dk, np.zeros_like(dk), what="dK with Q=0")
    _close(dv, dv_w, what="dV with Q=0")


def pin_k_zero_closed_form():
    """With K = 0 every score equals b. Then, for i < n_q and j < n_k:
      O_i  = sigma(b) * sum_j V_j
      dQ_i = 0
      dK_j = alpha sigma(b)(1 - sigma(b)) * sum_i (dO_i . V_j) Q_i
      dV_j = sigma(b) * sum_i dO_i"""
    rng = np.random.default_rng(5)
    Z, L, H, D = 2, 10, 1, 4
    q, _, v, do, nq, nk = _case(rng, Z, L, H, D, [6, 10], [10, 3])
    k = np.zeros_like(q)
    alpha, bias = 0.5, 0.8
    sb = 1.0 / (1.0 + math.exp(-0.8))
    o_w = np.zeros((Z, L, H, D))
    dk_w = np.zeros((Z, L, H, D))
    dv_w = np.zeros((Z, L, H, D))
    for z in range(Z):
        a, b = nq[z], nk[z]
        o_w[z, :a, 0] = sb * v[z, :b, 0].sum(0)
        dv_w[z, :b, 0] = sb * do[z, :a, 0].sum(0)
        for j in range(b):
            acc = np.zeros(D)
            for i in range(a):
                acc += float(do[z, i, 0] @ v[z, j, 0]) * q[z, i, 0]
            dk_w[z, j, 0] = alpha * sb * (1 - sb) * acc
    _close(osa.forward(q, k, v, nq, nk, alpha, bias), o_w, what="O with K=0")
    dq, dk, dv = osa.backward(q, k, v, do, nq, nk, alpha, bias)
    _close(dq, np.zeros_like(dq), what="dQ with K=0")
    _close(dk, dk_w, what="dK with K=0")
    _close(dv, dv_w, what="dV with K=0")


def pin_single_key():
    """With n_k = 1: O_i = sigma(alpha q_i . k_0 + b) v_0, element by element, using math.exp."""
    rng = np.random.default_rng(6)
    Z, L, H, D = 1, 5, 2, 3
    q, k, v, _, nq, nk = _case(rng, Z, L, H, D, [4], [1])
    alpha, bias = 0.9, -0.4
    o = osa.forward(q, k, v, nq, nk, alpha, bias)
    for h in range(H):
        for i in range(L):
            if i < 4:
                s = alpha * sum(q[0, i, h, d] * k[0, 0, h, d] for d in range(D)) + bias
                w = 1.0 / (1.0 + math.exp(-s))
                want = [w * v[0, 0, h, d] for d in range(D)]
            else:
                want = [0.0] * D
            _close(o[0, i, h], want, rtol=1e-13, atol=1e-15, what="O with n_k=1")


def pin_worked_example():
    """The hand-worked example in tests/golden/worked_example.json."""
    g = json.loads((GOLDEN / "worked_example.json").read_text())
    alpha = bias = math.log(3.0) / 2.0
    q = np.array(g["q"], np.float64)[None, :, None, :]
    k = np.array(g["k"], np.float64)[None, :, None, :]
    v = np.array(g["v"], np.float64)[None, :, None, :]
    do = np.array(g["do"], np.float64)[None, :, None, :]
    for c in g["cases"]:
        nq, nk = np.array([c["n_q"]]), np.array([c["n_k"]])
        o = osa.forward(q, k, v, nq, nk, alpha, bias)
        _close(o[0, :, 0], c["o"], rtol=1e-14, atol=1e-14, what=f"worked O ({c['name']})")
        dq, dk, dv = osa.backward(q, k, v, do, nq, nk, alpha, bias)
        _close(dq[0, :, 0] / alpha, c["dq_over_alpha"], rtol=1e-14, atol=1e-14, what=f"worked dQ ({c['name']})")
        _close(dk[0, :, 0] / alpha, c["dk_over_alpha"], rtol=1e-14, atol=1e-14, what=f"worked dK ({c['name']})")
        _close(dv[0, :, 0], c["dv"], rtol=1e-14, atol=1e-14, what=f"worked dV ({c['name']})")


# --------------------------------------------------------------------------- gradients
def _loss(q, k, v, do, nq, nk, alpha, bias):
    return float(np.sum(osa.forward(q, k, v, nq, nk, alpha, bias) * do))


def pin_finite_differences():
    """Central differences in fp64 of L = sum(O * dO) against the backward, entry by
    entry. The shape is tiny: Z=2, H=1, L=8, D=4. The length pairs are (n_q, n_k) =
    ([8,5],[8,5]) and ([6,3],[8,5]). Perturbing a padded entry must change nothing,
    so its difference must be exactly 0."""
    rng = np.random.default_rng(7)
    alpha, bias = 0.6, -1.1
    for nq_, nk_ in (([8, 5], [8, 5]), ([6, 3], [8, 5])):
        q, k, v, do, nq, nk = _case(rng, 2, 8, 1, 4, nq_, nk_)
        grads = osa.backward(q, k, v, do, nq, nk, alpha, bias)
        hstep = 1e-6
        for t_idx, (t, g) in enumerate(zip((q, k, v), grads)):
            n_valid = nq if t_idx == 0 else nk
            for idx in np.ndindex(t.shape):
                orig = t[idx]
                t[idx] = orig + hstep
                lp = _loss(q, k, v, do, nq, nk, alpha, bias)
                t[idx] = orig - hstep
                lm = _loss(q, k, v, do, nq, nk, alpha, bias)
                t[idx] = orig
                fd = (lp - lm) / (2 * hstep)
                if idx[1] >= n_valid[idx[0]]:
                    assert lp == lm, f"padded entry {idx} of tensor {t_idx} changed the loss"
                    assert g[idx] == 0.0, f"padded gradient {idx} of tensor {t_idx} is {g[idx]}"
                else:
                    assert abs(fd - g[idx]) <= 1e-6 * max(1.0, abs(fd)), (
                        f"FD mismatch tensor {t_idx} at {idx}: fd={fd} grad={g[idx]}")


def pin_torch_autograd():
    """The dense torch form of the pages' "PyTorch sigmoid attention" gives the same
    results. It uses torch.sigmoid on the full padded score matrix, zeroes the
    weights of padded keys, zeroes padded query rows, and differentiates with
    autograd in float64 on the CPU."""
    import torch

    rng = np.random.default_rng(8)
    Z, L, H, D = 3, 24, 2, 8
    q, k, v, do, nq, nk = _case(rng, Z, L, H, D, [24, 13, 0], [17, 24, 9])
    alpha, bias = 1.0 / math.sqrt(D), -math.log(L)
    tq, tk, tv = (torch.tensor(t, dtype=torch.float64, requires_grad=True) for t in (q, k, v))
    tdo = torch.tensor(do, dtype=torch.float64)
    outs = []
    for z in range(Z):
        kmask = (torch.arange(L) < int(nk[z])).to(torch.float64)
        qmask = (torch.arange(L) < int(nq[z])).to(torch.float64)
        heads = []
        for h in range(H):
            s = alpha * tq[z, :, h, :] @ tk[z, :, h, :].T + bias
            p = torch.sigmoid(s) * kmask[None, :]
            heads.append((p @ tv[z, :, h, :]) * qmask[:, None])
        outs.append(torch.stack(heads, dim=1))
    o_t = torch.stack(outs, dim=0)
    (o_t * tdo).sum().backward()
    _close(osa.forward(q, k, v, nq, nk, alpha, bias), o_t.detach().numpy(), rtol=1e-11, atol=1e-13, what="O vs torch")
    dq, dk, dv = osa.backward(q, k, v, do, nq, nk, alpha, bias)
    _close(dq, tq.grad.numpy(), rtol=1e-11, atol=1e-13, what="dQ vs autograd")
    _close(dk, tk.grad.numpy(), rtol=1e-11, atol=1e-13, what="dK vs autograd")
    _close(dv, tv.grad.numpy(), rtol=1e-11, atol=1e-13, what="dV vs autograd")


def pin_gradient_identities():
    """Two exact identities of the chain rule:
    sum <dQ, Q> = sum <dK, K> (both equal alpha * sum dS * QK^T), and
    sum <dV, V> = sum <dO, O>."""
    rng = np.random.default_rng(9)
    q, k, v, do, nq, nk = _case(rng, 2, 20, 3, 5, [20, 11], [15, 20])
    alpha, bias = 0.45, -2.0
    o = osa.forward(q, k, v, nq, nk, alpha, bias)
    dq, dk, dv = osa.backward(q, k, v, do, nq, nk, alpha, bias)
    do_valid = do.copy()
    for z in range(2):
        do_valid[z, nq[z]:] = 0.0
    _close(np.sum(dq * q), np.sum(dk * k), rtol=1e-12, atol=1e-12, what="<dQ,Q> = <dK,K>")
    _close(np.sum(dv * v), np.sum(do_valid * o), rtol=1e-12, atol=1e-12, what="<dV,V> = <dO,O>")


# --------------------------------------------------------------------------- padding and symmetries
def pin_padding_semantics():
    """The padding semantics (rainbus.top summary, 方法步骤详情 step 2):
    * every padded output row is exactly 0;
    * valid outputs are bitwise unchanged when the padded inputs hold garbage or NaN;
    * valid outputs are bitwise unchanged when L grows."""
    rng = np.random.default_rng(10)
    Z, L, H, D = 3, 16, 2, 4
    q, k, v, do, nq, nk = _case(rng, Z, L, H, D, [16, 9, 0], [11, 16, 5])
    alpha, bias = 0.5, -1.0
    o = osa.forward(q, k, v, nq, nk, alpha, bias)
    g = osa.backward(q, k, v, do, nq, nk, alpha, bias)
    for z in range(Z):
        assert np.all(o[z, nq[z]:] == 0.0), "padded O row not 0"
        assert np.all(g[0][z, nq[z]:] == 0.0), "padded dQ row not 0"
        assert np.all(g[1][z, nk[z]:] == 0.0) and np.all(g[2][z, nk[z]:] == 0.0), "padded dK/dV row not 0"
    for fill in (np.nan, 1e30):
        q2, k2, v2, do2 = (t.copy() for t in (q, k, v, do))
        for z in range(Z):
            q2[z, nq[z]:] = fill
            do2[z, nq[z]:] = fill
            k2[z, nk[z]:] = fill
            v2[z, nk[z]:] = fill
        assert np.array_equal(osa.forward(q2, k2, v2, nq, nk, alpha, bias), o), f"O depends on padding ({fill})"
        g2 = osa.backward(q2, k2, v2, do2, nq, nk, alpha, bias)
        for a, b in zip(g2, g):
            assert np.array_equal(a, b), f"grads depend on padding ({fill})"
    grow = lambda t: np.concatenate([t, rng.standard_normal((Z, 7, H, D))], axis=1)  # noqa: E731
    o3 = osa.forward(grow(q), grow(k), grow(v), nq, nk, alpha, bias)
    assert np.array_equal(o3[:, :L], o) and np.all(o3[:, L:] == 0), "O changes when L grows"
    g3 = osa.backward(grow(q), grow(k), grow(v), grow(do), nq, nk, alpha, bias)
    for a, b in zip(g3, g):
        assert np.array_equal(a[:, :L], b) and np.all(a[:, L:] == 0), "grads change when L grows"


def pin_symmetries():
    """O is linear in V. Permuting the valid keys together with their values:
    * leaves O and dQ unchanged (up to rounding);
    * permutes the rows of dK and dV the same way.
    Scaling alpha by c while scaling Q by 1/c leaves every output unchanged."""
    rng = np.random.default_rng(11)
    Z, L, H, D = 1, 14, 2, 5
    q, k, v, do, nq, nk = _case(rng, Z, L, H, D, [12], [10])
    alpha, bias = 0.3, -0.7
    v2 = rng.standard_normal(v.shape)
    o1 = osa.forward(q, k, v, nq, nk, alpha, bias)
    o2 = osa.forward(q, k, v2, nq, nk, alpha, bias)
    _close(osa.forward(q, k, 2.0 * v - 3.0 * v2, nq, nk, alpha, bias), 2.0 * o1 - 3.0 * o2, what="linearity in V")
    perm = np.concatenate([rng.permutation(10), np.arange(10, L)])
    kp, vp = k[:, perm], v[:, perm]
    _close(osa.forward(q, kp, vp, nq, nk, alpha, bias), o1, what="key permutation O")
    dq, dk, dv = osa.backward(q, k, v, do, nq, nk, alpha, bias)
    dqp, dkp, dvp = osa.backward(q, kp, vp, do, nq, nk, alpha, bias)
    _close(dqp, dq, what="key permutation dQ")
    _close(dkp, dk[:, perm], what="key permutation dK")
    _close(dvp, dv[:, perm], what="key permutation dV")
    dqs, dks, dvs = osa.backward(q / 4.0, k, v, do, nq, nk, alpha * 4.0, bias)
    _close(osa.forward(q / 4.0, k, v, nq, nk, alpha * 4.0, bias), o1, what="alpha/Q scaling O")
    _close(dqs, dq * 4.0, what="alpha/Q scaling dQ")
    _close(dks, dk, what="alpha/Q scaling dK")


def pin_large_scores():
    """At very large scores (std of alpha q.k about 256, as in the stress shape):
    * every output is finite;
    * P saturates to exactly 0 and exactly 1;
    * dS is exactly 0 wherever P does."""
    rng = np.random.default_rng(12)
    qv = rng.standard_normal((64, 16)) * 16 * 2
    kv = rng.standard_normal((48, 16)) * 16 * 2
    vv = rng.standard_normal((48, 16))
    dov = rng.standard_normal((64, 16))
    dq, dk, dv, it = osa.head_backward(qv, kv, vv, dov, 0.25, -math.log(8192), return_intermediates=True)
    assert all(np.all(np.isfinite(t)) for t in (dq, dk, dv, it["P"], it["dS"])), "non-finite at large scores"
    p = it["P"]
    assert np.any(p == 0.0) and np.any(p == 1.0), "no saturation at |S| ~ 1e3"
    assert np.all(it["dS"][(p == 0.0) | (p == 1.0)] == 0.0), "dS not 0 where P saturates"
    assert np.all(np.isfinite(osa.head_forward(qv, kv, vv, 0.25, -math.log(8192))))


def pin_row_sampling():
    """forward_rows / backward_rows give the same rows as the full-tensor functions."""
    rng = np.random.default_rng(13)
    q, k, v, do, nq, nk = _case(rng, 2, 30, 2, 6, [30, 17], [22, 30])
    alpha, bias = 0.4, -1.5
    o = osa.forward(q, k, v, nq, nk, alpha, bias)
    dq, dk, dv = osa.backward(q, k, v, do, nq, nk, alpha, bias)
    rows = np.array([0, 5, 16, 17, 21, 22, 29])
    for z in range(2):
        for h in range(2):
            _close(osa.forward_rows(q, k, v, nq, nk, alpha, bias, z, h, rows), o[z, rows, h], what="forward_rows")
            a, b, c = osa.backward_rows(q, k, v, do, nq, nk, alpha, bias, z, h, rows, rows)
            _close(a, dq[z, rows, h], what="backward_rows dQ")
            _close(b, dk[z, rows, h], what="backward_rows dK")
            _close(c, dv[z, rows, h], what="backward_rows dV")


def pin_tile_plan():
    """The skip plan equals its closed form: query tile m pairs with ceil(n_k/BN)
    key tiles when m*BM < n_q, and with none otherwise. The same holds for key
    tiles with the roles swapped. Edge lengths are covered: 0, L, multiples of
    the tile, and L not a multiple of the tile."""
    rng = np.random.default_rng(14)
    for L, bm, bn in ((256, 64, 64), (300, 128, 64), (1000, 64, 128), (17, 16, 32)):
        n = np.concatenate([[0, L, bm, bn, 1, L - 1], rng.integers(0, L + 1, 6)])
        nq, nk = n, np.roll(n, 3)
        by_q, by_k = osa.tile_plan(nq, nk, L, bm, bn)
        n_qt, n_kt = -(-L // bm), -(-L // bn)
        for z in range(n.shape[0]):
            for m in range(n_qt):
                want = -(-int(nk[z]) // bn) if m * bm < nq[z] else 0
                assert by_q[z, m] == want, f"tile plan q L={L} z={z} m={m}: {by_q[z, m]} != {want}"
            for t in range(n_kt):
                want = -(-int(nq[z]) // bm) if t * bn < nk[z] else 0
                assert by_k[z, t] == want, f"tile plan k L={L} z={z} t={t}: {by_k[z, t]} != {want}"


def pin_default_scalars():
    """alpha = 1/sqrt(D) (gist.science §2.A) and b = -ln(L) (paperlayer.ai §3, n = L)."""
    a, b = osa.default_scalars(64, 256)
    assert a == 0.125 and abs(b + math.log(256)) < 1e-15


# ------------------------------------------------------------- per-sample bias, packed layout
def pin_per_sample_bias_closed_form():
    """With Q = 0 and the per-sample bias b_z = -ln n_k[z] (paperlayer.ai §3,
    b = -log n), every score of sample z is b_z, so every weight is exactly
    sigma(-ln n) = 1/(1 + n), taken here from the integers alone. For i < n_q
    and j < n_k:
      O_i  = sum_j V_j / (1 + n_k)
      dV_j = sum_i dO_i / (1 + n_k)
      dQ_i = alpha n_k / (1 + n_k)^2 * sum_j (dO_i . V_j) K_j
      dK_j = 0
    The same holds in the packed layout, sample by sample."""
    rng = np.random.default_rng(14)
    Z, L, H, D = 3, 10, 2, 3
    nq, nk = [10, 4, 7], [6, 10, 1]
    alpha = 0.9
    _, k, v, do, nq, nk = _case(rng, Z, L, H, D, nq, nk)
    q = np.zeros_like(k)
    bias = osa.per_sample_bias(nk, 0.0)
    o_w, dq_w, dv_w = (np.zeros((Z, L, H, D)) for _ in range(3))
    for z in range(Z):
        a, b = int(nq[z]), int(nk[z])
        w = 1.0 / (1 + b)
        for h in range(H):
            o_w[z, :a, h] = w * v[z, :b, h].sum(0)
            dv_w[z, :b, h] = w * do[z, :a, h].sum(0)
            for i in range(a):
                acc = np.zeros(D)
                for j in range(b):
                    acc += float(do[z, i, h] @ v[z, j, h]) * k[z, j, h]
                dq_w[z, i, h] = alpha * b / (1 + b) ** 2 * acc
    _close(osa.forward(q, k, v, nq, nk, alpha, bias), o_w, what="O, per-sample bias, Q=0")
    dq, dk, dv = osa.backward(q, k, v, do, nq, nk, alpha, bias)
    _close(dq, dq_w, what="dQ, per-sample bias, Q=0")
    _close(dk, np.zeros_like(dk), what="dK, per-sample bias, Q=0")
    _close(dv, dv_w, what="dV, per-sample bias, Q=0")
    cu_q = np.concatenate([[0], np.cumsum(nq)])
    cu_k = np.concatenate([[0], np.cumsum(nk)])
    qp, kp, vp, dop = (np.concatenate([t[z, : int(n[z])] for z in range(Z)]) for t, n in
                       ((q, nq), (k, nk), (v, nk), (do, nq)))
    _close(osa.forward_varlen(qp, kp, vp, cu_q, cu_k, alpha, bias),
           np.concatenate([o_w[z, : int(nq[z])] for z in range(Z)]), what="packed O, per-sample bias, Q=0")
    dqp, dkp, dvp = osa.backward_varlen(qp, kp, vp, dop, cu_q, cu_k, alpha, bias)
    _close(dqp, np.concatenate([dq_w[z, : int(nq[z])] for z in range(Z)]), what="packed dQ, Q=0")
    _close(dkp, np.zeros_like(dkp), what="packed dK, Q=0")
    _close(dvp, np.concatenate([dv_w[z, : int(nk[z])] for z in range(Z)]), what="packed dV, Q=0")


def pin_varlen_matches_padded():
    """The packed layout is the padded one with the padding removed: on the
    same valid rows, forward_varlen and backward_varlen (which slice the packed
    arrays by offsets) equal forward and backward on the padded arrays (which
    slice by lengths), for one bias and for per-sample biases, with n_q != n_k
    and an empty sample."""
    rng = np.random.default_rng(15)
    Z, L, H, D = 4, 9, 2, 4
    nq, nk = np.array([9, 3, 0, 5]), np.array([4, 9, 2, 1])
    q, k, v, do, nq, nk = _case(rng, Z, L, H, D, nq, nk, scale=0.8)
    cu_q = np.concatenate([[0], np.cumsum(nq)])
    cu_k = np.concatenate([[0], np.cumsum(nk)])
    qp, dop = osa.pack(q, nq), osa.pack(do, nq)
    kp, vp = osa.pack(k, nk), osa.pack(v, nk)
    assert qp.shape == (int(nq.sum()), H, D) and kp.shape == (int(nk.sum()), H, D)
    for bias in (-1.1, osa.per_sample_bias(nk, 0.3)):
        o = osa.forward(q, k, v, nq, nk, 0.6, bias)
        _close(osa.forward_varlen(qp, kp, vp, cu_q, cu_k, 0.6, bias), osa.pack(o, nq), what="packed O")
        dq, dk, dv = osa.backward(q, k, v, do, nq, nk, 0.6, bias)
        dqp, dkp, dvp = osa.backward_varlen(qp, kp, vp, dop, cu_q, cu_k, 0.6, bias)
        _close(dqp, osa.pack(dq, nq), what="packed dQ")
        _close(dkp, osa.pack(dk, nk), what="packed dK")
        _close(dvp, osa.pack(dv, nk), what="packed dV")


def pin_pack_roundtrip():
    """unpack(pack(x)) keeps the valid prefixes and zeroes the rest."""
    rng = np.random.default_rng(16)
    x = rng.standard_normal((3, 5, 2))
    n = np.array([5, 0, 2])
    xp = osa.pack(x, n)
    assert xp.shape == (7, 2)
    y = osa.unpack(xp, np.concatenate([[0], np.cumsum(n)]), 5)
    want = x.copy()
    want[1, :] = 0
    want[2, 2:] = 0
    _close(y, want, rtol=0, atol=0, what="pack/unpack")


# ------------------------------------------------------------------------------ softmax path
def pin_softmax_q_zero_closed_form():
    """With Q = 0 every score of a row is 0, so every weight is exactly 1/n_k
    (rainbus.top summary, 前置知识, "Softmax 归一化": e^0 / sum e^0). For
    i < n_q, j < n_k:
      O_i = sum_j V_j / n_k,  LSE_i = ln n_k,
      dV_j = sum_i dO_i / n_k,  dK_j = 0,
      dQ_i = alpha / n_k * sum_j (dO_i . V_j - dO_i . O_i) K_j."""
    rng = np.random.default_rng(30)
    Z, L, H, D = 2, 11, 2, 3
    nq, nk = [11, 5], [7, 11]
    alpha = 0.8
    _, k, v, do, nq, nk = _case(rng, Z, L, H, D, nq, nk)
    q = np.zeros_like(k)
    o_w, dq_w, dv_w = (np.zeros((Z, L, H, D)) for _ in range(3))
    lse_w = np.zeros((Z, H, L))
    for z in range(Z):
        a, b = int(nq[z]), int(nk[z])
        for h in range(H):
            mean_v = v[z, :b, h].sum(0) / b
            o_w[z, :a, h] = mean_v
            lse_w[z, h, :a] = math.log(b)
            dv_w[z, :b, h] = do[z, :a, h].sum(0) / b
            for i in range(a):
                acc = np.zeros(D)
                for j in range(b):
                    acc += (float(do[z, i, h] @ v[z, j, h]) - float(do[z, i, h] @ mean_v)) * k[z, j, h]
                dq_w[z, i, h] = alpha / b * acc
    o, lse = sma.forward(q, k, v, nq, nk, alpha)
    _close(o, o_w, what="softmax O with Q=0")
    _close(lse, lse_w, what="softmax LSE with Q=0")
    dq, dk, dv = sma.backward(q, k, v, do, nq, nk, alpha)
    _close(dq, dq_w, what="softmax dQ with Q=0")
    _close(dk, np.zeros_like(dk), what="softmax dK with Q=0")
    _close(dv, dv_w, what="softmax dV with Q=0")


def _torch_softmax_reference(q, k, v, do, nq, nk, alpha):
    import torch

    Z, L, H, D = q.shape
    outs = [np.zeros((Z, L, H, D)) for _ in range(4)]
    lse = np.zeros((Z, H, L))
    for z in range(Z):
        a, b = int(nq[z]), int(nk[z])
        if a == 0 or b == 0:
            continue
        for h in range(H):
            tq, tk, tv = (torch.tensor(t[z, :, h], dtype=torch.float64, requires_grad=True) for t in (q, k, v))
            s = alpha * tq @ tk.T
            s = s.masked_fill(torch.arange(L)[None, :] >= b, float("-inf"))
            w = torch.softmax(s, dim=1)
            o = w @ tv
            o = o.masked_fill(torch.arange(L)[:, None] >= a, 0.0)
            (o * torch.tensor(do[z, :, h])).sum().backward()
            outs[0][z, :, h] = o.detach().numpy()
            outs[1][z, :, h] = tq.grad.numpy()
            outs[2][z, :, h] = tk.grad.numpy()
            outs[3][z, :, h] = tv.grad.numpy()
            lse[z, h, :a] = torch.logsumexp(s, dim=1).detach().numpy()[:a]
    return outs, lse


def pin_softmax_torch():
    """Dense torch.softmax / logsumexp / autograd in float64, padded keys masked
    with -inf and padded query rows zeroed, against the oracle's forward and
    backward (which take dK/dV through the row statistics)."""
    rng = np.random.default_rng(31)
    Z, L, H, D = 3, 13, 2, 4
    q, k, v, do, nq, nk = _case(rng, Z, L, H, D, [13, 6, 9], [9, 13, 1], scale=1.5)
    (o_t, dq_t, dk_t, dv_t), lse_t = _torch_softmax_reference(q, k, v, do, nq, nk, 0.7)
    o, lse = sma.forward(q, k, v, nq, nk, 0.7)
    _close(o, o_t, rtol=1e-10, atol=1e-12, what="softmax O vs torch")
    _close(lse, lse_t, rtol=1e-10, atol=1e-12, what="softmax LSE vs torch")
    dq, dk, dv = sma.backward(q, k, v, do, nq, nk, 0.7)
    _close(dq, dq_t, rtol=1e-10, atol=1e-12, what="softmax dQ vs torch")
    _close(dk, dk_t, rtol=1e-10, atol=1e-12, what="softmax dK vs torch")
    _close(dv, dv_t, rtol=1e-10, atol=1e-12, what="softmax dV vs torch")


def pin_softmax_small_blocks():
    """The backward again, with blocks of a few rows: the key-block route
    (P = e^{S - LSE}, D = dO . O) must not renormalise inside a block."""
    from oracle import sigmoid_attention as base

    rng = np.random.default_rng(32)
    q, k, v, do, nq, nk = _case(rng, 2, 12, 1, 3, [12, 5], [12, 9], scale=2.0)
    (_, dq_t, dk_t, dv_t), _ = _torch_softmax_reference(q, k, v, do, nq, nk, 0.9)
    saved = base._MAX_BLOCK_ELEMS
    base._MAX_BLOCK_ELEMS = 30  # blocks of 2-3 rows
    try:
        dq, dk, dv = sma.backward(q, k, v, do, nq, nk, 0.9)
        o_r, lse_r = sma.forward_rows(q, k, v, nq, nk, 0.9, 0, 0, np.arange(12))
        bq, bk, bv = sma.backward_rows(q, k, v, do, nq, nk, 0.9, 1, 0, np.arange(12), np.arange(12))
    finally:
        base._MAX_BLOCK_ELEMS = saved
    for n, a, b in (("dQ", dq, dq_t), ("dK", dk, dk_t), ("dV", dv, dv_t)):
        _close(a, b, rtol=1e-10, atol=1e-12, what=f"softmax {n}, small blocks")
    o, lse = sma.forward(q, k, v, nq, nk, 0.9)
    _close(o_r, o[0, :, 0], what="softmax forward_rows")
    _close(lse_r, lse[0, 0], what="softmax forward_rows LSE")
    _close(bq, dq_t[1, :, 0], rtol=1e-10, atol=1e-12, what="softmax backward_rows dQ")
    _close(bk, dk_t[1, :, 0], rtol=1e-10, atol=1e-12, what="softmax backward_rows dK")
    _close(bv, dv_t[1, :, 0], rtol=1e-10, atol=1e-12, what="softmax backward_rows dV")


def pin_softmax_invariants():
    """Each valid row's weights sum to 1 (V = 1 gives O = 1); a row with no
    key gives 0; huge scores do not overflow, and a key that leads every other
    by far takes all the weight."""
    rng = np.random.default_rng(33)
    Z, L, H, D = 2, 9, 1, 3
    q, k, _, do, nq, nk = _case(rng, Z, L, H, D, [9, 4], [6, 0], scale=3.0)
    ones = np.ones((Z, L, H, D))
    o, lse = sma.forward(q, k, ones, nq, nk, 1.0)
    _close(o[0, :9], np.ones((9, H, D)), what="softmax rows sum to 1")
    assert np.all(o[1] == 0) and np.all(lse[1] == 0), "a row with no key must give 0"
    # one dominating key: scores 0 except key 3 at 1000
    q1 = np.zeros((1, 5, 1, 2)); q1[0, :, 0, 0] = 1.0
    k1 = np.zeros((1, 5, 1, 2)); k1[0, 3, 0, 0] = 1000.0
    v1 = rng.standard_normal((1, 5, 1, 2))
    o1, lse1 = sma.forward(q1, k1, v1, [5], [5], 1.0)
    assert np.all(np.isfinite(o1)) and np.all(np.isfinite(lse1)), "softmax overflowed"
    _close(o1[0, :, 0], np.repeat(v1[0, 3:4, 0], 5, axis=0), rtol=0, atol=1e-12, what="dominating key")
    _close(lse1[0, 0], np.full(5, 1000.0), rtol=1e-15, atol=1e-12, what="LSE of a dominating key")
    dq, dk, dv = sma.backward(q1 * 50, k1, v1, rng.standard_normal((1, 5, 1, 2)), [5], [5], 1.0)
    assert all(np.all(np.isfinite(t)) for t in (dq, dk, dv)), "softmax gradients overflowed"


def pin_softmax_finite_differences():
    """dQ, dK and dV against central differences of sum(O * G), entry by entry."""
    rng = np.random.default_rng(34)
    q, k, v, g, nq, nk = _case(rng, 1, 5, 1, 2, [4], [5])
    alpha, eps = 0.6, 1e-6
    dq, dk, dv = sma.backward(q, k, v, g, nq, nk, alpha)
    loss = lambda qq, kk, vv: float((sma.forward(qq, kk, vv, nq, nk, alpha)[0] * g).sum())  # noqa: E731
    for name, t, grad in (("dQ", q, dq), ("dK", k, dk), ("dV", v, dv)):
        for idx in np.ndindex(t.shape):
            tp, tm = t.copy(), t.copy()
            tp[idx] += eps
            tm[idx] -= eps
            args_p = {"dQ": (tp, k, v), "dK": (q, tp, v), "dV": (q, k, tp)}[name]
            args_m = {"dQ": (tm, k, v), "dK": (q, tm, v), "dV": (q, k, tm)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - grad[idx]) < 1e-7, f"softmax {name}{idx}: fd {fd} vs {grad[idx]}"


# ------------------------------------------------------------------------------ FP8 path
# OCP 8-bit floating point, E4M3: bias 7, 3 mantissa bits, subnormals m * 2^-9,
# largest finite 1.75 * 2^8 = 448, code 0x7f NaN (the OCP FP8 specification's
# E4M3 table). Every expected value below is read off that definition.
def pin_e4m3_format():
    """Known codes of the E4M3 table, an exact round trip of every finite code,
    a strictly increasing grid, and round-to-nearest-even at every midpoint."""
    table = {0x00: 0.0, 0x01: 2.0**-9, 0x07: 7 * 2.0**-9, 0x08: 2.0**-6, 0x38: 1.0, 0x3A: 1.25, 0x40: 2.0,
             0x70: 128.0, 0x77: 240.0, 0x7E: 448.0, 0xC2: -2.5, 0xB8: -1.0, 0xFE: -448.0}
    for code, val in table.items():
        assert f8a.e4m3_decode(np.uint8(code)) == val, f"decode 0x{code:02x}"
        assert int(f8a.e4m3_encode(val)) == code, f"encode {val}"
    assert np.isnan(f8a.e4m3_decode(np.uint8(0x7F))) and np.isnan(f8a.e4m3_decode(np.uint8(0xFF)))
    assert int(f8a.e4m3_encode(-0.0)) == 0x80
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    assert np.array_equal(f8a.e4m3_encode(f8a.e4m3_decode(codes)), codes), "codes do not round-trip"
    pos = f8a.e4m3_decode(np.arange(0x00, 0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0), "grid not increasing"
    lo, hi = pos[:-1], pos[1:]
    mid = (lo + hi) / 2
    even = np.where(np.arange(0x00, 0x7E) % 2 == 0, lo, hi)   # the neighbour with an even code
    _close(f8a.e4m3_round(mid), even, rtol=0, atol=0, what="ties to even")
    _close(f8a.e4m3_round(-mid), -even, rtol=0, atol=0, what="ties to even, negative")
    _close(f8a.e4m3_round(mid - (hi - lo) / 8), lo, rtol=0, atol=0, what="below a midpoint")
    _close(f8a.e4m3_round(mid + (hi - lo) / 8), hi, rtol=0, atol=0, what="above a midpoint")
    _close(f8a.e4m3_round([1.0625, 1.1875, 1.5 * 2.0**-9, 2.0**-10]), [1.0, 1.25, 2.0**-8, 0.0], rtol=0, atol=0,
           what="rounding examples")


def pin_fp8_quantize():
    """Per-tile power-of-two quantisation: a hand-worked tile, exact round trips
    of representable values, the E4M3 error bound, per-tile independence, and
    zero codes for padding."""
    Z, L, H, D = 2, 150, 2, 8
    n = [150, 70]
    x = np.zeros((Z, L, H, D))
    # tile 0 of (0, 0): amax 1 -> E = -7 (1 * 2^7 = 128 in [128, 256)), byte 120
    x[0, 0:64, 0, 0] = 1.0
    x[0, 0:64, 0, 1] = 0.5          # 64 -> code 0x68
    x[0, 0:64, 0, 2] = -3 / 128     # -3 = -1.5 * 2^1 -> exponent field 8, mantissa 4: code 0xc4
    codes, sb = f8a.quantize(x, n)
    assert sb[0, 0, 0] == 120, f"scale byte {sb[0, 0, 0]}"
    assert codes[0, 5, 0, 0] == 0x70 and codes[0, 5, 0, 1] == 0x68 and codes[0, 5, 0, 2] == 0xC4
    # all-zero tiles: E = 0, byte 127, codes 0
    assert sb[0, 1, 0] == 127 and not codes[0, :64, 1].any()
    # representable values round-trip exactly; others stay within 2^-4 (normal) or 2^-10 2^E (subnormal)
    rng = np.random.default_rng(80)
    y = rng.standard_normal((Z, L, H, D)) * np.exp(rng.uniform(-6, 6, (Z, 1, H, 1)))
    cy, sy = f8a.quantize(y, n)
    dy = f8a.dequantize(cy, sy)
    again, s_again = f8a.quantize(dy, n)
    for z in range(Z):
        for h in range(H):
            for m in range(-(-n[z] // 64)):
                r0, r1 = 64 * m, min(64 * m + 64, n[z])
                e = int(sy[z, h, m]) - 127
                blk, got = y[z, r0:r1, h], dy[z, r0:r1, h]
                assert 128 <= np.max(np.abs(blk)) * 2.0**-e < 256, "amax not mapped into [128, 256)"
                tol = np.where(np.abs(blk) * 2.0**-e >= 2.0**-6, 2.0**-4 * np.abs(blk), 2.0**(e - 10))
                assert np.all(np.abs(got - blk) <= tol), "quantisation error beyond the E4M3 bound"
                if s_again[z, h, m] == sy[z, h, m]:
                    assert np.array_equal(again[z, r0:r1, h], cy[z, r0:r1, h]), "representable values moved"
                else:  # the tile's amax rounded up to 256 * 2^E, one binade higher
                    assert s_again[z, h, m] == sy[z, h, m] + 1 and np.max(np.abs(got)) * 2.0**-e == 256
    assert not cy[1, 70:].any(), "padded rows have non-zero codes"
    # scaling one tile by 2^5 moves only its byte
    y2 = y.copy()
    y2[1, 0:64, 1] *= 32.0
    c2, s2 = f8a.quantize(y2, n)
    assert np.array_equal(c2, cy) and s2[1, 1, 0] == sy[1, 1, 0] + 5
    s2[1, 1, 0] -= 5
    assert np.array_equal(s2, sy)


def _fp8_inputs(V, nq, nk, Z, L, H, D, q=None, k=None):
    q = np.zeros((Z, L, H, D)) if q is None else q
    k = np.zeros((Z, L, H, D)) if k is None else k
    q8, sq = f8a.quantize(q, nq)
    k8, sk = f8a.quantize(k, nk)
    v8, sv = f8a.quantize(V, nk)
    return q8, k8, v8, sq, sk, sv


def pin_fp8_forward_closed_forms():
    """Q = 0 gives P = sigma(b) on every valid key. sigma(ln 3) = 3/4 = 192 * 2^-8
    is on the E4M3 grid, so P is exact; sigma(ln 7/3) = 0.7: 0.7 * 2^8 = 179.2
    lies between 176 and 192 (step 16 in [128, 256)), so P becomes 176/256 =
    11/16. V holds values of at most two significant bits, exactly
    representable at every power-of-two scale, so O is 11/16 (or 3/4) times the
    column sums of V over the valid keys."""
    Z, L, H, D = 2, 150, 1, 4
    nq, nk = [150, 40], [130, 150]
    rng = np.random.default_rng(81)
    V = rng.choice([-2.0, -1.5, -1.0, -0.75, -0.5, 0.0, 0.5, 0.75, 1.0, 1.5, 2.0], (Z, L, H, D))
    q8, k8, v8, sq, sk, sv = _fp8_inputs(V, nq, nk, Z, L, H, D)
    for b, pw in ((math.log(3.0), 0.75), (math.log(7.0 / 3.0), 11.0 / 16.0)):
        o = f8a.forward(q8, k8, v8, sq, sk, sv, nq, nk, 0.3, b)
        for z in range(Z):
            want = pw * V[z, : nk[z]].sum(axis=0)
            _close(o[z, : nq[z]], np.broadcast_to(want, (nq[z], H, D)), rtol=0, atol=1e-12, what=f"fp8 O, P={pw}")
            assert not o[z, nq[z]:].any(), "fp8 padded rows not 0"


def pin_fp8_p_tiles():
    """P is scaled per query row and per tile of 64 keys. With q = e_0, keys
    0-31 at k = 0 and keys 32-99 at k = -13 e_0 (on the E4M3 grid, as is q),
    alpha = 1 and b = ln 3, keys 0-31 weigh 3/4 and the others
    p = 1 / (1 + e^13 / 3), about 6.8e-6. Tile 0's scale comes from 3/4
    (2^-8): p 2^8 is subnormal in E4M3 (below 2^-6) and within half a step of
    one step 2^-9, so p becomes 2^-17. Tile 1 (keys 64-99) holds p only, with
    its own scale 2^(floor(log2 p) - 7) = 2^-25: p 2^25 = 227.5 lies between
    224 and 240 (step 16), nearer 224, so p becomes 224 * 2^-25."""
    Z, L, H, D = 1, 100, 1, 2
    alpha, b = 1.0, math.log(3.0)
    q = np.zeros((Z, L, H, D))
    q[0, :, 0, 0] = 1.0
    k = np.zeros((Z, L, H, D))
    k[0, 32:, 0, 0] = -13.0
    V = np.zeros((Z, L, H, D))
    V[0, :, 0, 0] = 1.0
    V[0, :, 0, 1] = np.arange(L) % 5 - 2.0
    n = [L]
    p = 1.0 / (1.0 + math.exp(13.0) / 3.0)
    assert 0.5 < p * 2.0**17 < 1.5 and math.floor(math.log2(p)) == -18 and 224 < p * 2.0**25 < 232, "assumptions"
    q8, k8, v8, sq, sk, sv = _fp8_inputs(V, n, n, Z, L, H, D, q, k)
    _close(f8a.dequantize(k8, sk), k, rtol=0, atol=0, what="k on the grid")
    o = f8a.forward(q8, k8, v8, sq, sk, sv, n, n, alpha, b)
    w = np.where(np.arange(L) < 32, 0.75, np.where(np.arange(L) < 64, 2.0**-17, 224 * 2.0**-25))
    want = (w[:, None] * V[0, :, 0]).sum(axis=0)
    _close(o[0, 3, 0], want, rtol=0, atol=1e-15, what="fp8 per-tile P scales")


def pin_fp8_scaling_and_bound():
    """Exact laws of the power-of-two scales (V's bytes + 1 doubles O; Q's bytes
    + 2 with K's - 2 leave O alone), rows equal the whole, and the P
    quantisation error stays within 2^-4 sum_j P_j |V_j| (E4M3 relative bound;
    the weights come from the sigmoid oracle on the dequantised inputs) plus
    the subnormal tail 2^-17 max_j P_j sum_j |V_j|."""
    Z, L, H, D = 2, 200, 2, 16
    nq, nk = [200, 90], [150, 200]
    rng = np.random.default_rng(82)
    q, k, v = (rng.standard_normal((Z, L, H, D)) for _ in range(3))
    q8, k8, v8, sq, sk, sv = _fp8_inputs(v, nq, nk, Z, L, H, D, q, k)
    alpha, b = 0.25, -1.5
    o = f8a.forward(q8, k8, v8, sq, sk, sv, nq, nk, alpha, b)
    _close(f8a.forward(q8, k8, v8, sq, sk, sv + 1, nq, nk, alpha, b), 2 * o, rtol=0, atol=0, what="V scale law")
    _close(f8a.forward(q8, k8, v8, sq + 2, sk - 2, sv, nq, nk, alpha, b), o, rtol=0, atol=0, what="Q/K scale law")
    rows = np.array([0, 1, 63, 64, 89, 90, 199])
    _close(f8a.forward_rows(q8, k8, v8, sq, sk, sv, nq, nk, alpha, b, 1, 1, rows), o[1, rows, 1], rtol=0, atol=0,
           what="fp8 rows")
    Q, K, V = (f8a.dequantize(c, s) for c, s in ((q8, sq), (k8, sk), (v8, sv)))
    exact = osa.forward(Q, K, V, nq, nk, alpha, b)
    spv = osa.forward(Q, K, np.abs(V), nq, nk, alpha, b)            # sum_j P_j |V_j|
    pmax = osa.forward(Q, K, np.ones_like(V), nq, nk, alpha, b)     # >= max_j P_j
    sv_abs = np.stack([np.abs(V[z, : nk[z]]).sum(axis=0) for z in range(Z)])[:, None]
    bound = 2.0**-4 * spv + 2.0**-17 * pmax * sv_abs
    assert np.all(np.abs(o - exact) <= bound + 1e-15), "P quantisation beyond the E4M3 bound"
    assert np.max(np.abs(o - exact)) > 0, "P was not quantised at all"


ALL_PINS = [
    pin_sigmoid_closed_forms,
    pin_derivative_bound,
    pin_lipschitz_quarter,
    pin_q_zero_closed_form,
    pin_k_zero_closed_form,
    pin_single_key,
    pin_worked_example,
    pin_finite_differences,
    pin_torch_autograd,
    pin_gradient_identities,
    pin_padding_semantics,
    pin_symmetries,
    pin_large_scores,
    pin_row_sampling,
    pin_tile_plan,
    pin_default_scalars,
    pin_per_sample_bias_closed_form,
    pin_varlen_matches_padded,
    pin_pack_roundtrip,
    pin_softmax_q_zero_closed_form,
    pin_softmax_torch,
    pin_softmax_small_blocks,
    pin_softmax_invariants,
    pin_softmax_finite_differences,
    pin_e4m3_format,
    pin_fp8_quantize,
    pin_fp8_forward_closed_forms,
    pin_fp8_p_tiles,
    pin_fp8_scaling_and_bound,
]
