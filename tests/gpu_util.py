"""Helpers shared by the GPU tests: device uploads and parity statistics."""
from __future__ import annotations

import numpy as np


def torch():
    import torch as t
    return t


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float values to bf16 (ties to even) and return them as float32.
    Input preparation only (makes operands exactly representable)."""
    import workloads as wl
    return wl.round_to_bf16_(np.ascontiguousarray(a, dtype=np.float32).copy())


def to_dev_bf16(a: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a, np.float32)).cuda().to(t.bfloat16).contiguous()


def to_dev(a: np.ndarray, dtype=None):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a)).cuda() if dtype is None else \
        t.from_numpy(np.ascontiguousarray(a)).cuda().to(dtype)


def logit_stats(gpu: np.ndarray, ref: np.ndarray) -> dict:
    """max |diff|, error std, top-1 agreement, and whether every top-1
    disagreement is explained by an oracle top-2 margin below twice the
    largest error (several answers are then correct)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = gpu - ref
    g1 = np.argmax(gpu, axis=-1)
    r1 = np.argmax(ref, axis=-1)
    agree = g1 == r1
    part = np.partition(ref, -2, axis=-1)
    margin = part[..., -1] - part[..., -2]
    maxd = float(np.max(np.abs(diff)))
    explained = bool(np.all(margin[~agree] < 2 * maxd)) if (~agree).any() else True
    return {"max_abs": maxd, "std": float(np.std(diff)), "top1": float(np.mean(agree)),
            "n_rows": int(agree.size), "disagree": int((~agree).sum()),
            "disagree_explained": explained}
