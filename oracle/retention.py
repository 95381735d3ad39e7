"""Plain fp64 oracle of attention-guided retention: the attention mass of every
prefix key and the choice of the rows to keep.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: aitopics tag page "kv state", Sparse-dLLM abstract: the cache keeps
the critical tokens and evicts the others, guided by attention. The pages do
not print the score; the plainest reading, used here, is the attention
probability a key receives summed over the queries that read it:

    mass[b, h, j] = sum over q-heads g of kv head h and block queries i of
                    exp(s[b, g, i, j] - LSE[b, g, i]),   s = scale * <q, k_j>,

with LSE each row's log-sum-exp over all keys it attends ([prefix; block]), so
one row's probabilities over all keys sum to 1. The kept set is the n_keep
keys of largest mass; ties go to the lower row index; the set is listed in
ascending row order (the index layout the gathered attention reads).
"""

from __future__ import annotations

import numpy as np

from .attention import _scale64, widen


def prefix_mass(q, k_pre, lse, scale: float) -> np.ndarray:
    """mass [B, Hkv, P] in float64 from q [B, Hq, Bq, d], k_pre [B, Hkv, P, d]
    (float32 or bf16 bits) and lse [B, Hq, Bq] (any float array)."""
    B, Hq, Bq, _ = q.shape
    Hkv, P = k_pre.shape[1], k_pre.shape[2]
    G = Hq // Hkv
    s64 = _scale64(scale)
    lse64 = np.asarray(lse, dtype=np.float64)
    out = np.zeros((B, Hkv, P), dtype=np.float64)
    for b in range(B):
        for h in range(Hkv):
            kk = widen(k_pre[b, h])                          # [P, d]
            for g in range(G):
                hq = h * G + g
                s = s64 * (widen(q[b, hq]) @ kk.T)           # [Bq, P]
                out[b, h] += np.exp(s - lse64[b, hq][:, None]).sum(axis=0)
    return out


def select_retained(mass: np.ndarray, n_keep: int) -> np.ndarray:
    """int32 [B, Hkv, n_keep]: per (b, h) the n_keep rows of largest mass,
    ties towards the lower row, in ascending row order."""
    B, Hkv, P = mass.shape
    out = np.zeros((B, Hkv, n_keep), dtype=np.int32)
    rows = np.arange(P)
    for b in range(B):
        for h in range(Hkv):
            order = np.lexsort((rows, -np.asarray(mass[b, h], dtype=np.float64)))  # mass desc, row asc
            out[b, h] = np.sort(order[:n_keep])
    return out
