"""Shared helpers for the GPU parity tests: oracle-side expectations and error measures.

Expected values come only from oracle/ on the same seeded inputs; nothing here reads a
result of the HIP path except to compare it.
"""
from __future__ import annotations

import sys

import numpy as np

from oracle import mbq_oracle as O

# Per-token output bar: max_n |y - yref| / max_n |yref| <= 1e-2 (bf16 I/O, fp32 accumulate).
TOL = 1e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def oracle_blob(W: np.ndarray, group: int, slices: int) -> np.ndarray:
    p = O.pack(W, group, slices)
    return O.to_blob_fast(p["codes"], p["scale"], p["zero"], group), p


def oracle_linear_rows(W: np.ndarray, X: np.ndarray, budget: np.ndarray, group: int,
                       slices: int, rows: np.ndarray | None = None) -> np.ndarray:
    """float64 y for all tokens and the given rows (pack is row-independent)."""
    Wr = W if rows is None else W[rows]
    p = O.pack(Wr, group, slices)
    deq = O.dequant_slices(p["codes"], p["scale"], p["zero"], group)
    return O.linear(X, deq, budget)


def budget_from_perm(perm: np.ndarray, offsets: np.ndarray) -> np.ndarray:
    T = perm.shape[0]
    b = np.zeros(T, np.int32)
    for j in range(1, offsets.shape[0]):
        b[perm[offsets[j - 1]:offsets[j]]] = j
    return b


def token_errors(y: np.ndarray, yref: np.ndarray) -> np.ndarray:
    """Per token: max abs error over outputs / max abs reference output."""
    y = np.asarray(y, np.float64)
    yref = np.asarray(yref, np.float64)
    num = np.abs(y - yref).max(axis=1)
    den = np.maximum(np.abs(yref).max(axis=1), 1e-30)
    return num / den
