"""Comparison rules between the GPU path and the CPU oracle.

Index sets: for each query the GPU row must hold exactly k_t = min(K, n_t)
distinct slots of that query's visible positions, followed by K - k_t entries
of -1.  Against the oracle's Top-K set, the symmetric difference must consist
of near-ties only: with G = GPU-only and O = oracle-only positions,
    max_{j in O} S_j - min_{i in G} S_i <= 1e-3 * max(|S_i|, |S_j|)
or the gap is at most 1e-6 * max_p |S_p| (absolute floor for near-zero scores),
where S are the oracle's fp64 scores.  Order of the valid entries is free.

Attention outputs: max |delta| <= 2e-2 and ||delta||_2 / ||ref||_2 <= 1e-2 over
the compared outputs (bf16 output, fp32 accumulation).
"""
from __future__ import annotations

import numpy as np

from oracle import dsa_oracle as O

REL_GAP = 1e-3
ABS_FLOOR = 1e-6
MAX_ABS = 2e-2
REL_L2 = 1e-2


def check_index_row(row, S, slots, K, rel=REL_GAP, abs_floor=ABS_FLOOR):
    """Return (ok, message) for one query's GPU index row.  S: oracle scores of
    positions 0..n-1; slots: their physical slots."""
    row = np.asarray(row, dtype=np.int64)
    n = S.shape[0]
    k = min(K, n)
    if row.shape[0] != K:
        return False, f"row length {row.shape[0]} != K={K}"
    if (row[:k] < 0).any():
        return False, f"fewer than k_t={k} valid entries"
    if (row[k:] != -1).any():
        return False, "entries after the first k_t are not -1"
    pos_of = {int(s): p for p, s in enumerate(np.asarray(slots, dtype=np.int64))}
    try:
        gpos = np.array([pos_of[int(s)] for s in row[:k]], dtype=np.int64)
    except KeyError as e:
        return False, f"slot {e} is not a visible position of this query"
    if np.unique(gpos).shape[0] != k:
        return False, "duplicate slots"
    opos = O.topk_positions(S, K)
    G = np.setdiff1d(gpos, opos)
    Om = np.setdiff1d(opos, gpos)
    if G.shape[0] == 0:
        return True, "exact"
    i = G[np.argmin(S[G])]
    j = Om[np.argmax(S[Om])]
    gap = S[j] - S[i]
    bound = max(rel * max(abs(S[i]), abs(S[j])), abs_floor * float(np.abs(S).max()))
    if gap <= bound:
        return True, f"{G.shape[0]} near-tie swaps (gap {gap:.3g} <= {bound:.3g})"
    return False, f"{G.shape[0]} swaps, worst gap {gap:.4g} > {bound:.4g} (S_i={S[i]:.6g}, S_j={S[j]:.6g})"


def check_outputs(got, ref, max_abs=MAX_ABS, rel_l2=REL_L2):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = got - ref
    mad = float(np.abs(d).max()) if d.size else 0.0
    nrm = float(np.linalg.norm(ref))
    rl2 = float(np.linalg.norm(d)) / nrm if nrm > 0 else float(np.linalg.norm(d))
    ok = mad <= max_abs and rl2 <= rel_l2
    return ok, f"max|d|={mad:.3g} relL2={rl2:.3g}"
