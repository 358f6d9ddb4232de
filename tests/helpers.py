"""Shared checks for the parity tests.

Tolerance metric (per row): max_i |got_i - ref_i| / max_i |ref_i| over finite
entries; masked entries must be -inf on both sides.  Top-k acceptance with a tie
band: with tau the k_eff-th largest oracle score of the row and
delta = 1e-3 |tau| + 1e-6 max|scores|, the device set must hold k_eff distinct
positions, contain every s scoring above tau + delta and none scoring below
tau - delta.
"""
from __future__ import annotations

import os
import sys

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 5e-2}
TIE_REL = 1e-3
TIE_ABS = 1e-6


def announce(msg: str):
    """Name the case on the real stderr before a GPU step (survives a lost box)."""
    sys.__stderr__.write(f"[case] {msg}\n")
    sys.__stderr__.flush()


def rel_rowmax(got, ref, axis=-1):
    """Per-row max |got - ref| / max |ref| over the finite reference entries.  Every
    reference entry must be finite or -inf; got must be finite exactly where ref is
    and -inf exactly where ref is -inf (NaN or +inf in got fails)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    fin = np.isfinite(ref)
    masked = ref == -np.inf
    assert np.all(fin | masked), "reference holds NaN or +inf"
    assert np.array_equal(fin, np.isfinite(got)), "masked (-inf) pattern differs"
    assert np.all(got[masked] == -np.inf), "masked entries are not -inf"
    g = np.where(fin, got, 0.0)
    r = np.where(fin, ref, 0.0)
    d = np.abs(g - r).max(axis=axis)
    m = np.abs(r).max(axis=axis)
    return np.where(m > 0, d / np.where(m > 0, m, 1.0), d)


def topk_valid(idx_row, score_row, p: int, K: int):
    """Return None if the device selection is valid under the tie band, else a message."""
    keff = max(0, min(K, p + 1))
    sel = [int(x) for x in idx_row if x >= 0]
    if len(sel) != keff:
        return f"selected {len(sel)} != k_eff {keff}"
    if len(set(sel)) != keff:
        return "duplicate positions"
    if any(s > p for s in sel):
        return "position beyond the query"
    if np.any(np.asarray(idx_row)[keff:] != -1):
        return "padding is not -1"
    if keff == 0:
        return None
    sc = np.asarray(score_row[: p + 1], dtype=np.float64)
    tau = np.sort(sc)[::-1][keff - 1]
    delta = TIE_REL * abs(tau) + TIE_ABS * np.abs(sc).max()
    must = set(np.nonzero(sc > tau + delta)[0].tolist())
    banned = set(np.nonzero(sc < tau - delta)[0].tolist())
    sset = set(sel)
    if not must <= sset:
        return f"missing {len(must - sset)} positions above the band"
    if sset & banned:
        return f"{len(sset & banned)} positions below the band"
    return None


def gpu_lib_ready():
    import torch
    here = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    return torch.cuda.is_available() and os.path.exists(os.path.join(here, "sparse_attention_09_amd", "libdsa.so"))
