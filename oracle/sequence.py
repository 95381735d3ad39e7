"""Plain fp64 oracle of the full-sequence FACache step: first-layer attention
of every token while one block of the sequence is being denoised.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "LaCache: Exact Caching and Precision-Adaptive Inference for Diffusion
Large Language Models", section 3.3.1 (the block C and the unchanged rows U:
prompt, earlier blocks and the masked suffix), section 3.3.3 FACache (the
online-softmax state of the U queries over the U keys is cached; later steps
start from it and stream only the key tiles that overlap C) and the Appendix J
pseudocode (cache populated at the block's first step, reused afterwards;
output O = O~/l, L = m + log l).

Two functions:
  sequence_full  the plain definition: softmax attention of every query row of
                 the sequence over every key row (no mask);
  facache_step   the method's procedure in the pages' order: build or take the
                 cache, continue it over the block's keys for the U queries,
                 and attend all keys for the block queries.
While the U rows keep the values the cache was built from, the two agree to
rounding (the cache is exact); the tests pin that.
"""

from __future__ import annotations

from typing import Iterable, Optional, Tuple

import numpy as np

from .attention import attention_rows, online_state, state_from_partial, widen, finalize, partial


def sequence_full(q, k, v, scale: float, heads: Optional[Iterable[Tuple[int, int]]] = None):
    """o [B, Hq, N, d], lse [B, Hq, N]: every query row attends every key row.

    q [B, Hq, N, d]; k, v [B, Hkv, N, d] (float32 or bf16 bits). Query head h
    reads kv head h // (Hq / Hkv). NaN outside `heads` when a sample is asked.
    """
    B, Hq, N, d = q.shape
    G = Hq // k.shape[1]
    o = np.full((B, Hq, N, v.shape[3]), np.nan)
    lse = np.full((B, Hq, N), np.nan)
    todo = sorted(set(heads)) if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in todo:
        o[b, h], lse[b, h] = attention_rows(widen(q[b, h]), widen(k[b, h // G]), widen(v[b, h // G]), scale)
    return o, lse


def split_rows(n: int, block_start: int, block_len: int):
    """Row indices of U (every row outside the block, in order) and of C."""
    rows = np.arange(n)
    in_block = (rows >= block_start) & (rows < block_start + block_len)
    return rows[~in_block], rows[in_block]


def facache_step(q, k, v, block_start: int, block_len: int, scale: float, cache=None, tile: int = 64):
    """One denoising step of the block at rows [block_start, block_start + block_len).

    With cache None (the block's first step) the cache is first built: the
    partial state (o, m, l) of the U queries over the U keys (the tiles the
    pseudocode marks as neither overlapping the block), stored per sequence row
    with the block rows left NaN. Then, as at every later step, the U queries'
    running state starts from the cache and streams only the block's keys
    (eqs. 2-6 over the overlapping tiles); the block queries attend every key.
    Returns (o [B, Hq, N, d], lse [B, Hq, N], cache) in float64.
    """
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    u, c = split_rows(N, block_start, block_len)
    if cache is None:
        po, pm, pl = partial(np.take(q, u, axis=2), np.take(k, u, axis=2), np.take(v, u, axis=2), scale)
        cache = (np.full((B, Hq, N, v.shape[3]), np.nan), np.full((B, Hq, N), np.nan),
                 np.full((B, Hq, N), np.nan))
        cache[0][:, :, u], cache[1][:, :, u], cache[2][:, :, u] = po, pm, pl
    co, cm, cl = (np.asarray(x, dtype=np.float64) for x in cache)
    o = np.full((B, Hq, N, v.shape[3]), np.nan)
    lse = np.full((B, Hq, N), np.nan)
    for b in range(B):
        for h in range(Hq):
            kk, vv = widen(k[b, h // G]), widen(v[b, h // G])
            qq = widen(q[b, h])
            if len(u):
                st = state_from_partial(co[b, h, u], cm[b, h, u], cl[b, h, u])
                m, l, ot = online_state(qq[u], kk[c], vv[c], scale, tile, state=st)
                o[b, h, u] = ot / l[:, None]
                lse[b, h, u] = finalize(m, l)
            o[b, h, c], lse[b, h, c] = attention_rows(qq[c], kk, vv, scale)
    return o, lse, cache
