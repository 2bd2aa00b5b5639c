"""Seeded synthetic workloads for sigmoid attention (inputs only, no attention math).

This module is shared by the tests, the bench and the smoke check. It
generates inputs and nothing else. It holds none of the method's arithmetic,
and neither the CPU oracle nor the GPU library imports it.

Shapes and length mixes follow the pages' workloads:

* "tiny": Z=2, H=2, L=256, D=64 in fp32, with lengths [256, 160].
* "nopad16k": L=16384, D=128 with no padding, the kernel benchmark in the
  paperlayer.ai summary, section 4, and in the rainbus.top results table.
* "pad25_16k": the same shape with 25% of the batch's tokens as padding
  (rainbus.top results table; zhengruan.com article, part 3).
* "cellbatch8k": a batch of cells whose gene counts follow the length CDF in
  the rainbus.top figure notes (57.7/82.0/96.6/100% of cells at or below
  2048/4096/8192/16384 genes). They are padded to L=8192 with D=64, the head
  size of the 160M model (768 hidden / 12 heads, rainbus.top reproduction
  notes).
* "nopad8k_d64": the cell batch's shape (Z=16, H=12, L=8192, D=64) with no
  padding, the rate its kernels reach when every tile is full.
* "stress8k": L=8192, D=64 with Q and K scaled up to produce large scores,
  standing in for the 8K no-clipping stress test (paperlayer.ai summary,
  section 5).

The pages measure on no public suite. CellxGene cells are stood in for only
through this length model.

Generation:
* Lengths use numpy's default_rng(seed).
* Tensors use a CPU torch.Generator seeded with the same seed and are drawn in
  the order q, k, v, do.
* They are drawn as N(0, 1) in fp32 and rounded to bf16 (RNE) where the
  workload is bf16.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    Z: int
    H: int
    L: int
    D: int
    dtype: str  # "bf16" or "fp32"
    length_model: str
    qk_scales: tuple = (1.0,)
    description: str = ""
    fixed_lengths: tuple = field(default=())

    @property
    def alpha(self) -> float:
        """Score scale 1/sqrt(D)."""
        return 1.0 / math.sqrt(self.D)

    @property
    def bias(self) -> float:
        """Score bias -log(L): the padded length, natural log."""
        return -math.log(self.L)


WORKLOADS = {
    "tiny": Workload("tiny", 2, 2, 256, 64, "fp32", "fixed", fixed_lengths=(256, 160),
                     description="tiny oracle case, second sample 37.5% padded"),
    "nopad16k": Workload("nopad16k", 1, 16, 16384, 128, "bf16", "full",
                         description="kernel bench, L=16K, D=128, no padding"),
    "pad25_16k": Workload("pad25_16k", 4, 16, 16384, 128, "bf16", "simplex25",
                          description="kernel bench, L=16K, D=128, 25% of tokens padding"),
    "cellbatch8k": Workload("cellbatch8k", 16, 12, 8192, 64, "bf16", "lognormal_cells",
                            description="cell batch, log-normal gene counts clipped to 8192"),
    "nopad8k_d64": Workload("nopad8k_d64", 16, 12, 8192, 64, "bf16", "full",
                            description="the cell batch's shape with every sample at L: its kernels' rate "
                                        "without padding"),
    "stress8k": Workload("stress8k", 8, 12, 8192, 64, "bf16", "uniform_1k_8k", qk_scales=(1.0, 4.0, 16.0),
                         description="long-context stress, Q,K ~ N(0, s^2)"),
}

# Log-normal fitted to the page's gene-count CDF (57.7% <= 2048, 82.0% <= 4096,
# 96.6% <= 8192). Draws outside [200, 17000] are rejected, then clipped to L.
CELL_LOGNORMAL_MU = 7.4595
CELL_LOGNORMAL_SIGMA = 0.8501
CELL_MIN, CELL_MAX = 200, 17000


def lengths(w: Workload | str, seed: int = 0) -> np.ndarray:
    """Per-sample true lengths (int32[Z]); n_q = n_k = these in every workload."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = np.random.default_rng(seed)
    if w.length_model == "fixed":
        n = np.array(w.fixed_lengths, dtype=np.int64)
    elif w.length_model == "full":
        n = np.full(w.Z, w.L, dtype=np.int64)
    elif w.length_model == "simplex25":
        # Padding totals exactly 25% of Z*L. It is split over the samples at
        # uniformly drawn cut points, so the per-sample pads are uniform on the simplex.
        total = (w.Z * w.L) // 4
        cuts = np.sort(rng.integers(0, total + 1, w.Z - 1))
        pads = np.diff(np.concatenate([[0], cuts, [total]]))
        n = w.L - pads
    elif w.length_model == "lognormal_cells":
        out = []
        while len(out) < w.Z:
            x = rng.lognormal(CELL_LOGNORMAL_MU, CELL_LOGNORMAL_SIGMA)
            if CELL_MIN <= x <= CELL_MAX:
                out.append(int(np.rint(x)))
        n = np.minimum(np.array(out, dtype=np.int64), w.L)
    elif w.length_model == "uniform_1k_8k":
        n = rng.integers(1024, w.L, size=w.Z, endpoint=True)
    else:
        raise ValueError(w.length_model)
    return n.astype(np.int32)


def make_tensors(Z, L, H, D, dtype="bf16", seed=0, qk_scale=1.0):
    """q, k, v, do as CPU torch tensors [Z, L, H, D].

    They are drawn as N(0,1) fp32, with q and k then scaled by qk_scale. They
    are rounded to bf16 when dtype == "bf16".
    """
    import torch

    g = torch.Generator().manual_seed(int(seed))
    shape = (Z, L, H, D)
    out = []
    for i in range(4):
        t = torch.randn(shape, generator=g, dtype=torch.float32)
        if i < 2 and qk_scale != 1.0:
            t.mul_(qk_scale)
        if dtype == "bf16":
            t = t.to(torch.bfloat16)
        elif dtype != "fp32":
            raise ValueError(dtype)
        out.append(t)
    return tuple(out)


def make_inputs(name: str, seed: int = 0, qk_scale: float | None = None):
    """Everything one run of a named workload needs, as CPU tensors/arrays."""
    w = WORKLOADS[name]
    n = lengths(w, seed)
    s = w.qk_scales[0] if qk_scale is None else qk_scale
    q, k, v, do = make_tensors(w.Z, w.L, w.H, w.D, w.dtype, seed, s)
    return {"workload": w, "q": q, "k": k, "v": v, "do": do, "seqlens_q": n.copy(), "seqlens_k": n.copy(),
            "alpha": w.alpha, "bias": w.bias, "qk_scale": s}


def to_f64(t):
    """A CPU torch tensor as a float64 numpy array (exact for bf16 and fp32)."""
    return t.float().numpy().astype(np.float64)
