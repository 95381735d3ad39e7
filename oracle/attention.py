"""Plain fp64 oracle: what block-diffusion attention over a cached prefix computes.

TEST INFRASTRUCTURE ONLY (see the package docstring): used by the tests, the
smoke check and the benchmark's CPU-baseline leg, never by the product path.

Sources (the pages this follows):
  [LaCache]    "LaCache: Exact Caching and Precision-Adaptive Inference for
               Diffusion Large Language Models": section 3.3.1 (notation: the
               current block C and the unchanged region U), section 3.3.3 FACache
               (eqs. 2-6, the online-softmax state (m, l, O~) and its caching),
               Appendix B.2 (eq. 9, tiled scores), Appendix J (pseudocode of
               FACache: state initialisation, output O = O~/l and L = m + log l).
  [FlashBlock] "FlashBlock: Attention Caching for Efficient Long-Context Block
               Diffusion", abstract: block-external attention output is cached
               and reused, block-internal attention is recomputed.
  [Fixed]      "Fixed State, Long Reach: What a Constant-Size Cache Buys Block
               Diffusion at Scale", abstract: the denoiser is bidirectional inside
               the block (no causal mask).
  [kv state]   aitopics tag page "kv state", Sparse-dLLM abstract: retained
               critical tokens, evicted others (attention over a kept subset).

Readings where the pages leave a step open:
  * scores carry an explicit scale: s = scale * <q, k> (the pages print QK^T;
    the scale is a float argument, 1/sqrt(d) in every workload), and the oracle
    uses that float32 value exactly;
  * L is the natural-log log-sum-exp of the scaled scores;
  * no mask: every block query attends to every prefix key and every block key;
  * GQA: query head h reads kv head h // (Hq/Hkv);
  * a partial stores normalised o = O~/l with m and l (O~ = l*o);
  * an empty key set has the partial (o=0, m=-inf, l=0); merging with it
    returns the other side; two empty sides give o=0, lse=-inf.

Storage: inputs are float32 arrays or bfloat16 bit patterns in uint16 arrays;
both widen exactly to float64.
"""

from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

NEG_INF = -math.inf


def widen(x: np.ndarray) -> np.ndarray:
    """Exact float64 value of a float32 array or of bfloat16 bits (uint16)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if x.dtype in (np.float32, np.float64):
        return x.astype(np.float64)
    raise TypeError(f"unsupported storage dtype {x.dtype}")


def _scale64(scale: float) -> float:
    """The kernel receives the scale as float32; the oracle uses that value."""
    return float(np.float32(scale))


# ---------------------------------------------------------------------------
# the definition
# ---------------------------------------------------------------------------

def attention_rows(q: np.ndarray, keys: np.ndarray, values: np.ndarray,
                   scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """softmax(scale * q K^T) V and the log-sum-exp, row by row.

    q [n, d], keys [N, d], values [N, d] (float64). This is the result the
    FACache recurrence reaches exactly ([LaCache] section 3.3.3: caching the
    online-softmax state leaves the output unchanged; eqs. 2-6 telescope to the
    plain softmax). Returns o [n, d] and lse [n].
    """
    n, d = q.shape
    if keys.shape[0] == 0:
        return np.zeros((n, values.shape[1])), np.full(n, NEG_INF)
    s = _scale64(scale) * (q @ keys.T)                 # scores, [n, N]
    mx = s.max(axis=1, keepdims=True)
    lse = mx[:, 0] + np.log(np.exp(s - mx).sum(axis=1))  # ln sum_j e^{s_j}
    p = np.exp(s - lse[:, None])                       # softmax weights
    return p @ values, lse


def _keys_of(k_pre, v_pre, idx, k_blk, v_blk, b: int, hkv: int):
    """Key/value rows one (batch, kv-head) attends: [prefix (gathered); block]."""
    kp, vp = k_pre[b, hkv], v_pre[b, hkv]
    if idx is not None:
        rows = np.asarray(idx[b, hkv], dtype=np.int64)
        kp, vp = kp[rows], vp[rows]
    ks, vs = [widen(kp)], [widen(vp)]
    if k_blk is not None:
        ks.append(widen(k_blk[b, hkv]))
        vs.append(widen(v_blk[b, hkv]))
    return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)


def full(q, k_pre, v_pre, k_blk, v_blk, scale: float, idx=None,
         heads: Optional[Iterable[Tuple[int, int]]] = None):
    """Block attention over [prefix; block] for every (batch, q-head).

    Every block query attends to all prefix rows (or the rows idx keeps, in
    order) and to all block rows, with no mask ([Fixed]: bidirectional denoiser;
    [LaCache] section 3.3.1: U holds the prefix, C the current block;
    [kv state]: attention over the retained rows).
    q [B, Hq, Bq, d]; k_pre/v_pre [B, Hkv, P, d]; k_blk/v_blk [B, Hkv, Bq, d]
    (None for no block keys); idx int32 [B, Hkv, n_keep] or None.
    Returns o [B, Hq, Bq, d] and lse [B, Hq, Bq] in float64 (NaN where `heads`
    restricts the evaluation to a sample of (batch, q-head) pairs).
    """
    B, Hq, Bq, d = q.shape
    Hkv = k_pre.shape[1]
    G = Hq // Hkv
    o = np.full((B, Hq, Bq, v_pre.shape[3]), np.nan)
    lse = np.full((B, Hq, Bq), np.nan)
    todo = sorted(set(heads)) if heads is not None else [
        (b, h) for b in range(B) for h in range(Hq)]
    by_group = {}
    for b, h in todo:
        by_group.setdefault((b, h // G), []).append(h)
    for (b, hkv), hs in by_group.items():
        keys, values = _keys_of(k_pre, v_pre, idx, k_blk, v_blk, b, hkv)
        for h in hs:
            o[b, h], lse[b, h] = attention_rows(widen(q[b, h]), keys, values, scale)
    return o, lse


# ---------------------------------------------------------------------------
# the cached state: partials and their merge
# ---------------------------------------------------------------------------

def partial(q, k, v, scale: float, idx=None):
    """Online-softmax state of the block queries over one key set.

    For keys J: m = max_j s_j, l = sum_j e^{s_j - m}, o = sum_j e^{s_j - m} v_j / l,
    i.e. the (m, l, O~) of [LaCache] section 3.3.3 after streaming over J, with
    o = O~/l stored normalised. An empty J gives (o=0, m=-inf, l=0), the initial
    state of the Appendix J pseudocode.
    q [B, Hq, n, d]; k, v [B, Hkv, N, d]; idx selects rows of k/v per
    (batch, kv-head) when given. Returns (o [B,Hq,n,d], m [B,Hq,n], l [B,Hq,n]).
    """
    B, Hq, n, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    o = np.zeros((B, Hq, n, v.shape[3]))
    m = np.full((B, Hq, n), NEG_INF)
    l = np.zeros((B, Hq, n))
    for b in range(B):
        for hkv in range(Hkv):
            keys, values = _keys_of(k, v, idx, None, None, b, hkv)
            if keys.shape[0] == 0:
                continue
            for h in range(hkv * G, (hkv + 1) * G):
                s = _scale64(scale) * (widen(q[b, h]) @ keys.T)
                mm = s.max(axis=1)
                e = np.exp(s - mm[:, None])
                ll = e.sum(axis=1)
                m[b, h], l[b, h] = mm, ll
                o[b, h] = (e @ values) / ll[:, None]
    return o, m, l


def finalize(m, l):
    """L = m + ln l ([LaCache] Appendix J); -inf for an empty state."""
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    with np.errstate(divide="ignore"):
        return np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), NEG_INF)


def merge(a, b):
    """Combine two partial states over disjoint key sets.

    M = max(m_a, m_b); w_x = l_x e^{m_x - M}; l = w_a + w_b;
    o = (w_a o_a + w_b o_b) / l; m = M; lse = M + ln l.
    Starting the recurrence of [LaCache] eqs. 2-6 from a cached state and
    streaming the remaining key tiles (section 3.3.3, and the Appendix J
    pseudocode's initialisation from the cache at later steps) produces exactly
    this. Returns (o, m, l, lse); both sides empty -> (0, -inf, 0, -inf).
    """
    oa, ma, la = (np.asarray(x, dtype=np.float64) for x in a)
    ob, mb, lb = (np.asarray(x, dtype=np.float64) for x in b)
    M = np.maximum(ma, mb)
    live = np.isfinite(M)
    Ms = np.where(live, M, 0.0)
    with np.errstate(invalid="ignore"):
        wa = np.where(np.isfinite(ma), la * np.exp(np.where(np.isfinite(ma), ma, 0.0) - Ms), 0.0)
        wb = np.where(np.isfinite(mb), lb * np.exp(np.where(np.isfinite(mb), mb, 0.0) - Ms), 0.0)
    l = wa + wb
    safe = np.where(l > 0, l, 1.0)
    o = (wa[..., None] * oa + wb[..., None] * ob) / safe[..., None]
    o = np.where((l > 0)[..., None], o, 0.0)
    m = np.where(live, M, NEG_INF)
    return o, m, l, finalize(m, l)


def gather(x_full: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Retained rows: out[b, h, r] = x_full[b, h, idx[b, h, r]] (a bit copy).

    [kv state] Sparse-dLLM keeps the critical tokens and evicts the rest; the
    kept rows are named by per-(batch, kv-head) indices.
    """
    B, H, n = idx.shape
    out = np.empty((B, H, n) + x_full.shape[3:], dtype=x_full.dtype)
    for b in range(B):
        for h in range(H):
            for r in range(n):
                out[b, h, r] = x_full[b, h, int(idx[b, h, r])]
    return out


# ---------------------------------------------------------------------------
# the pages' recurrence, step by step
# ---------------------------------------------------------------------------

def state_from_partial(o, m, l):
    """(m, l, O~) with O~ = l * o: the unnormalised state the pages cache."""
    o = np.asarray(o, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    return np.asarray(m, dtype=np.float64).copy(), l.copy(), o * l[..., None]


def online_state(q: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float,
                 tile: int, state: Optional[Sequence[np.ndarray]] = None):
    """Stream key/value tiles through eqs. 2-6 of [LaCache] section 3.3.3.

    q [n, d]; keys, values [N, d] (float64); tiles of `tile` rows in order.
    For each tile j: S = scale q K_j^T (eq. 9 of Appendix B.2, with the scale);
    m_j = max(m_{j-1}, rowmax S) (eq. 2); alpha = exp(m_{j-1} - m_j) (eq. 3);
    P~ = exp(S - m_j) (eq. 4); l_j = alpha l_{j-1} + rowsum P~ (eq. 5);
    O~_j = alpha O~_{j-1} + P~ V_j (eq. 6).
    `state` = (m, l, O~) to continue from (the cached state); default is the
    Appendix J initialisation m = -inf, l = 0, O~ = 0.
    Returns (m, l, O~); O = O~ / l and L = m + ln l finish it.
    """
    n = q.shape[0]
    if state is None:
        m = np.full(n, NEG_INF)
        l = np.zeros(n)
        ot = np.zeros((n, values.shape[1]))
    else:
        m, l, ot = (np.array(x, dtype=np.float64) for x in state)
    sc = _scale64(scale)
    for j0 in range(0, keys.shape[0], tile):
        kj, vj = keys[j0:j0 + tile], values[j0:j0 + tile]
        s = sc * (q @ kj.T)
        m_new = np.maximum(m, s.max(axis=1))
        with np.errstate(invalid="ignore"):
            alpha = np.where(np.isfinite(m), np.exp(m - m_new), 0.0)
        pt = np.exp(s - m_new[:, None])
        l = alpha * l + pt.sum(axis=1)
        ot = alpha[:, None] * ot + pt @ vj
        m = m_new
    return m, l, ot
