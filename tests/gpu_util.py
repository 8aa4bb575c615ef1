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


LITERAL_MAX_ABS = 3e-2   # bf16 bar on the logits
LITERAL_TOP1 = 0.999     # bf16 bar on the next-token choice


def logit_stats(gpu: np.ndarray, ref: np.ndarray, chosen=None) -> dict:
    """Parity of GPU logits against the oracle's, row by row.

    max |diff|, error std, top-1 agreement of the GPU's choice (``chosen``,
    else the argmax of its own logits) with the oracle's argmax, and whether
    every disagreement is explained by that row's own errors: the oracle
    logit at the GPU's choice lies within |diff| at the choice plus |diff|
    at the oracle's argmax of the oracle's maximum (for a choice that is the
    argmax of the GPU's row this holds exactly when the choice is consistent
    with the row's logits).  Also whether the literal bars hold."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    V = gpu.shape[-1]
    gpu2, ref2 = gpu.reshape(-1, V), ref.reshape(-1, V)
    diff = gpu2 - ref2
    g1 = np.argmax(gpu2, axis=-1) if chosen is None else np.asarray(chosen).reshape(-1)
    r1 = np.argmax(ref2, axis=-1)
    agree = g1 == r1
    rows = np.arange(len(g1))
    gap = ref2[rows, r1] - ref2[rows, g1]
    own = np.abs(diff[rows, g1]) + np.abs(diff[rows, r1])
    explained = bool(np.all(gap[~agree] <= own[~agree] + 1e-12))
    maxd = float(np.max(np.abs(diff)))
    top1 = float(np.mean(agree))
    return {"max_abs": maxd, "std": float(np.std(diff)), "top1": top1,
            "n_rows": int(agree.size), "disagree": int((~agree).sum()),
            "rows_explained": explained,
            "literal_max_met": maxd <= LITERAL_MAX_ABS, "literal_top1_met": top1 >= LITERAL_TOP1}
