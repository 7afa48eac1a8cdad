"""Checking and repairing the row layout of the down (W2) expert weights.

The gfx90a paper ("DeepSeek-V4-Flash on AMD gfx90a: Correctness Recovery and
Inference Performance Engineering", abstract) reports that its routed-expert
W2 weights were laid out differently from what the kernels assumed, that the
resulting output permutation was identified, and that the layout was repaired
at load time. In this library the repair is ``moe_prepack``'s row_perm
argument; this module holds the host-side identification step.

If the stored W2 rows are a permutation pi of the canonical rows (stored row r
holds canonical row pi[r], codes and scales together), every output column of
the layer is permuted the same way: out_bad[:, n] == out_ref[:, pi[n]] bit for
bit, because each output column is an independent dot product over the
intermediate activation. ``recover_row_permutation`` finds pi from a
reference output and the suspect output by exact column matching, and refuses
anything that is not a bijection of columns (codes moved without their scales,
for instance, change the values and match no reference column). Passing
``inverse_permutation(pi)`` as row_perm to ``moe_prepack`` then repairs the
layout.
"""
from __future__ import annotations

import numpy as np


class LayoutError(ValueError):
    """The suspect output is not a column permutation of the reference."""


def inverse_permutation(perm) -> np.ndarray:
    perm = np.asarray(perm, dtype=np.int64)
    n = perm.shape[0]
    if np.any(perm < 0) or np.any(perm >= n) or np.unique(perm).size != n:
        raise LayoutError("not a permutation")
    inv = np.empty(n, dtype=np.int32)
    inv[perm] = np.arange(n, dtype=np.int32)
    return inv


def _column_keys(a: np.ndarray) -> list:
    a = np.ascontiguousarray(np.asarray(a).T)  # one row per column of a
    return [a[i].tobytes() for i in range(a.shape[0])]


def recover_row_permutation(out_ref, out_bad) -> np.ndarray:
    """pi (int32 [N]) with out_bad[:, n] == out_ref[:, pi[n]] bit for bit.

    out_ref, out_bad: [T, N] arrays of the same dtype and shape. Raises
    LayoutError when a column of out_bad matches no column of out_ref, when two
    columns map to the same reference column, or when out_ref has repeated
    columns (the permutation would not be identifiable).
    """
    out_ref = np.asarray(out_ref)
    out_bad = np.asarray(out_bad)
    if out_ref.shape != out_bad.shape or out_ref.dtype != out_bad.dtype or out_ref.ndim != 2:
        raise LayoutError("outputs must be 2-D arrays of one shape and dtype")
    ref = {}
    for i, k in enumerate(_column_keys(out_ref)):
        if k in ref:
            raise LayoutError(f"reference columns {ref[k]} and {i} are identical")
        ref[k] = i
    pi = np.empty(out_ref.shape[1], dtype=np.int32)
    for n, k in enumerate(_column_keys(out_bad)):
        m = ref.get(k)
        if m is None:
            raise LayoutError(f"output column {n} matches no reference column: not a row permutation")
        pi[n] = m
    if np.unique(pi).size != pi.size:
        raise LayoutError("two output columns match the same reference column")
    return pi


def interleave_permutation(n: int, group: int) -> np.ndarray:
    """pi[r] = (r % group) * (n // group) + r // group: rows of a [group][n/group]
    blocked order read as [n/group][group], the kind of transposed storage a
    layout mismatch produces."""
    if n % group:
        raise ValueError("n must be a multiple of group")
    r = np.arange(n)
    return ((r % group) * (n // group) + r // group).astype(np.int32)
