"""Pins of the full-sequence FACache oracle (oracle/sequence.py).

sequence_full is the plain definition; it is pinned to a pure-Python
per-element evaluation, closed forms and the absence of any mask.
facache_step follows the method's procedure (cache of the unchanged rows'
queries over the unchanged keys, continued over the block's keys); LaCache
section 3.3.3 says the cache is exact, so it must reproduce sequence_full at
every step while the rows outside the block keep their values, and must stop
doing so once a cached row changes (the cache is really what it reads).
"""

import math

import numpy as np
import pytest

import datagen
import oracle
from tests.test_oracle_pins import brute_row


def rnd(seed, *shape, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def test_definition_against_per_element_evaluation():
    q, k, v = rnd(1, 1, 4, 6, 3), rnd(2, 1, 2, 6, 3), rnd(3, 1, 2, 6, 3)   # GQA 4 q-heads / 2 kv-heads
    o, lse = oracle.sequence_full(q, k, v, 0.7)
    sc = float(np.float32(0.7))
    for h in range(4):
        for i in range(6):
            oo, ll = brute_row(q[0, h, i], k[0, h // 2], v[0, h // 2], sc)
            assert np.allclose(o[0, h, i], oo, atol=1e-13) and abs(lse[0, h, i] - ll) < 1e-13


def test_zero_queries_average_every_row():
    q = np.zeros((1, 2, 9, 4))
    k, v = rnd(4, 1, 2, 9, 4), rnd(5, 1, 2, 9, 4)
    o, lse = oracle.sequence_full(q, k, v, 0.5)
    assert np.allclose(o[0, 1], v[0, 1].mean(axis=0), atol=1e-14)
    assert np.allclose(lse, math.log(9), atol=1e-14)


def test_first_row_sees_the_last_key():
    """Row 0 (before the block) weights the last row (in the masked suffix)
    exactly as the closed form says: no causal or block mask anywhere."""
    N, d = 7, 4
    q = np.zeros((1, 1, N, d))
    q[0, 0, 0, 0] = 2.0
    k = np.zeros((1, 1, N, d))
    k[0, 0, N - 1, 0] = 1.5
    v = rnd(6, 1, 1, N, d)
    o, lse = oracle.sequence_full(q, k, v, 1.0)
    t = 3.0
    want = (math.exp(t) * v[0, 0, N - 1] + v[0, 0, :N - 1].sum(axis=0)) / (math.exp(t) + N - 1)
    assert np.allclose(o[0, 0, 0], want, atol=1e-14)
    assert abs(lse[0, 0, 0] - math.log(math.exp(t) + N - 1)) < 1e-14
    # the same with the block in the middle of the sequence, through the cached path
    of, lf, _ = oracle.facache_step(q, k, v, 2, 3, 1.0)
    assert np.allclose(of[0, 0, 0], want, atol=1e-13)


@pytest.mark.parametrize("c0,Bq,tile", [(0, 4, 64), (5, 4, 64), (16, 4, 3), (9, 1, 2), (0, 20, 64)])
def test_first_step_equals_the_definition(c0, Bq, tile):
    N = 20
    q, k, v = rnd(7, 2, 4, N, 8), rnd(8, 2, 2, N, 8), rnd(9, 2, 2, N, 8)
    o, lse, cache = oracle.facache_step(q, k, v, c0, Bq, 0.35, tile=tile)
    ro, rl = oracle.sequence_full(q, k, v, 0.35)
    assert np.abs(o - ro).max() < 1e-12 and np.abs(lse - rl).max() < 1e-12
    u, c = oracle.split_rows(N, c0, Bq)
    co, cm, cl = cache
    assert np.isnan(cm[:, :, c]).all()              # the block's rows hold no cached state
    if len(u):
        lcache = oracle.finalize(cm[:, :, u], cl[:, :, u])
        assert np.all(cl[:, :, u] >= 1 - 1e-12) and np.all(cl[:, :, u] <= len(u) + 1e-12)
        assert np.all(lcache >= cm[:, :, u] - 1e-12) and np.all(lcache <= cm[:, :, u] + math.log(len(u)) + 1e-12)


def test_reuse_is_exact_while_the_other_rows_are_fixed():
    N, c0, Bq = 23, 11, 5
    q, k, v = rnd(10, 1, 3, N, 6), rnd(11, 1, 3, N, 6), rnd(12, 1, 3, N, 6)
    _, _, cache = oracle.facache_step(q, k, v, c0, Bq, 0.4)
    for t in range(1, 4):
        q2, k2, v2 = q.copy(), k.copy(), v.copy()
        q2[:, :, c0:c0 + Bq] = rnd(100 + t, 1, 3, Bq, 6)
        k2[:, :, c0:c0 + Bq] = rnd(200 + t, 1, 3, Bq, 6)
        v2[:, :, c0:c0 + Bq] = rnd(300 + t, 1, 3, Bq, 6)
        o, lse, _ = oracle.facache_step(q2, k2, v2, c0, Bq, 0.4, cache=cache)
        ro, rl = oracle.sequence_full(q2, k2, v2, 0.4)
        assert np.abs(o - ro).max() < 1e-12 and np.abs(lse - rl).max() < 1e-12


def test_a_stale_cache_is_visible():
    """Changing a row outside the block without rebuilding the cache changes the
    exact answer of the other rows' queries but not what the cached step gives
    them: the step reads the cache instead of the U x U tiles."""
    N, c0, Bq = 16, 4, 4
    q, k, v = rnd(13, 1, 1, N, 4), rnd(14, 1, 1, N, 4), rnd(15, 1, 1, N, 4)
    o0, _, cache = oracle.facache_step(q, k, v, c0, Bq, 0.5)
    k2 = k.copy()
    k2[0, 0, N - 1] += 3.0                           # a masked-suffix key changes
    o, _, _ = oracle.facache_step(q, k2, v, c0, Bq, 0.5, cache=cache)
    ro, _ = oracle.sequence_full(q, k2, v, 0.5)
    u, c = oracle.split_rows(N, c0, Bq)
    assert np.abs(o[:, :, u] - ro[:, :, u]).max() > 1e-3   # U rows: stale
    assert np.abs(o[:, :, u] - o0[:, :, u]).max() < 1e-12  # ... and unchanged
    assert np.abs(o[:, :, c] - ro[:, :, c]).max() < 1e-12  # block rows attend every key afresh


def test_sequence_inputs_recipe():
    sh = datagen.scaled_shape("llada_seq", q_heads=2, kv_heads=2, head_dim=64, prefix_len=300, block_start=100)
    q0, k0, v0 = datagen.sequence_inputs(sh, 0)
    q1, k1, v1 = datagen.sequence_inputs(sh, 1)
    assert q0.shape == (1, 2, 300, 64) and q0.dtype == np.uint16
    blk = slice(100, 132)
    for a, b in ((q0, q1), (k0, k1), (v0, v1)):
        assert np.array_equal(np.delete(a, np.s_[100:132], axis=2), np.delete(b, np.s_[100:132], axis=2))
        assert not np.array_equal(a[:, :, blk], b[:, :, blk])
