"""Helpers for the GPU parity tests: move seeded inputs to the device, compare with the oracle."""

from __future__ import annotations

import sys

import numpy as np
import torch

import workloads


def note(msg: str) -> None:
    """Name the case before a GPU step, so a failure can be traced from the log."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def device_inputs(q, k, v, do, nq, nk, dev="cuda:0"):
    to = lambda t: t.to(dev).contiguous()  # noqa: E731
    return (to(q), to(k), to(v), to(do), torch.as_tensor(np.asarray(nq), dtype=torch.int32).to(dev),
            torch.as_tensor(np.asarray(nk), dtype=torch.int32).to(dev))


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max|gpu - ref| / max|ref|; exact equality is required when ref is all zero."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    m = float(np.max(np.abs(ref))) if ref.size else 0.0
    d = float(np.max(np.abs(gpu - ref))) if ref.size else 0.0
    if m == 0.0:
        return 0.0 if d == 0.0 else float("inf")
    return d / m


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def f64(t: torch.Tensor) -> np.ndarray:
    return workloads.to_f64(t)


def assert_padding_zero(name, out: np.ndarray, n) -> None:
    for z, nz in enumerate(np.asarray(n)):
        pad = out[z, int(nz):]
        assert np.all(pad == 0.0), f"{name}: padded rows of sample {z} are not exactly 0"
