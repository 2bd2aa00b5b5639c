"""FLOP and byte accounting for the bench and the roofline.

FLOP rule (paperlayer.ai summary of arXiv:2604.27124, section A.2, "Kernel
benchmarking"): TFLOPS come from theoretical FLOPs, counted over valid
(non-padded) tokens, with the backward charged 2.5x the forward. The forward
of non-causal attention is two contractions of 2*D FLOP per score pair. So:
    fwd = 4 * D * H * sum_z n_q[z] * n_k[z]     (valid count)
    fwd = 4 * D * H * Z * L * L                 (padded count)
    bwd = 2.5 * fwd,   fwd+bwd = 3.5 * fwd.
sigma and the other elementwise work are not counted.

Bytes: per valid token and head, the forward moves 8*D bytes in bf16 (read Q,
K, V, write O) and the backward 14*D bytes (read Q, K, V, dO, write dQ, dK, dV).
"""

from __future__ import annotations

import numpy as np


def attention_flops(Z, L, H, D, seqlens_q=None, seqlens_k=None):
    """Returns a dict of fwd/bwd/total FLOPs, padded and valid."""
    padded = 4.0 * D * H * Z * L * L
    if seqlens_q is None:
        valid = padded
    else:
        nq = np.clip(np.asarray(seqlens_q, dtype=np.int64), 0, L)
        nk = np.clip(np.asarray(seqlens_k if seqlens_k is not None else seqlens_q, dtype=np.int64), 0, L)
        valid = 4.0 * D * H * float(np.sum(nq * nk))
    return {
        "fwd_padded": padded, "fwd_valid": valid,
        "bwd_padded": 2.5 * padded, "bwd_valid": 2.5 * valid,
        "total_padded": 3.5 * padded, "total_valid": 3.5 * valid,
    }


def executed_mfma_flops(H, D, seqlens_q, seqlens_k, L, fwd_tiles, dq_tiles, dkdv_tiles):
    """FLOPs the MFMA pipes actually execute, counting whole tiles (padding inside partial
    tiles included). Each *_tiles is (block_q, block_k). The forward runs 4*D per
    pair, the dQ kernel 6*D and the dK/dV kernel 8*D."""
    nq = np.clip(np.asarray(seqlens_q, dtype=np.int64), 0, L)
    nk = np.clip(np.asarray(seqlens_k, dtype=np.int64), 0, L)

    def pairs(bq, bk):
        return float(np.sum(-(-nq // bq) * bq * (-(-nk // bk)) * bk)) * H

    return {
        "fwd": 4.0 * D * pairs(*fwd_tiles),
        "dq": 6.0 * D * pairs(*dq_tiles),
        "dkdv": 8.0 * D * pairs(*dkdv_tiles),
    }


def hbm_bytes(Z, L, H, D, seqlens_q, seqlens_k, elem_bytes=2):
    """Algorithmic HBM bytes: valid rows read once, every output row written once."""
    nq = np.clip(np.asarray(seqlens_q, dtype=np.int64), 0, L)
    nk = np.clip(np.asarray(seqlens_k, dtype=np.int64), 0, L)
    row = H * D * elem_bytes
    full = Z * L * row
    fwd = float(np.sum(nq) + 2 * np.sum(nk)) * row + full
    bwd = float(2 * np.sum(nq) + 2 * np.sum(nk)) * row + 3 * full
    return {"fwd": fwd, "bwd": bwd}
