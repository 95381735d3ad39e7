"""Pins of the retention oracle (attention mass of prefix keys and the choice
of retained rows) to facts that do not depend on its own code: probability
conservation, a closed form, brute force, and hand-checked selections."""

import math

import numpy as np

import datagen
import oracle


def _inputs(**kw):
    sh = datagen.scaled_shape("dream_gqa", **kw)
    return sh, datagen.make_inputs(sh)


def test_mass_conserves_probability():
    # every query row spends probability 1 over [prefix; block]: the prefix
    # mass plus the block mass of a kv head is G * Bq
    sh, inp = _inputs(batch=2, q_heads=6, kv_heads=2, prefix_len=150, block_len=12)
    _, lse = oracle.full(inp.q, inp.k_pre, inp.v_pre, inp.k_blk, inp.v_blk, sh.scale)
    mp = oracle.prefix_mass(inp.q, inp.k_pre, lse, sh.scale)
    mb = oracle.prefix_mass(inp.q, inp.k_blk, lse, sh.scale)
    total = mp.sum(-1) + mb.sum(-1)
    assert np.allclose(total, 3 * 12, rtol=0, atol=1e-10)
    assert np.all(mp > 0)


def test_mass_of_zero_queries_is_uniform():
    # q = 0: every score is 0, LSE = ln N, each key receives G*Bq/N
    sh, inp = _inputs(batch=1, q_heads=4, kv_heads=2, prefix_len=70, block_len=8)
    q0 = np.zeros_like(inp.q)
    n = 70 + 8
    lse = np.full((1, 4, 8), math.log(n))
    mp = oracle.prefix_mass(q0, inp.k_pre, lse, sh.scale)
    assert np.allclose(mp, 2 * 8 / n, rtol=0, atol=1e-14)


def test_mass_brute_force():
    sh, inp = _inputs(batch=1, q_heads=2, kv_heads=1, prefix_len=5, block_len=3, head_dim=64)
    _, lse = oracle.full(inp.q, inp.k_pre, inp.v_pre, inp.k_blk, inp.v_blk, sh.scale)
    mp = oracle.prefix_mass(inp.q, inp.k_pre, lse, sh.scale)
    s32 = float(np.float32(sh.scale))
    q = oracle.widen(inp.q)
    k = oracle.widen(inp.k_pre)
    for j in range(5):
        want = 0.0
        for g in range(2):
            for i in range(3):
                dot = sum(q[0, g, i, t] * k[0, 0, j, t] for t in range(64))
                want += math.exp(s32 * dot - lse[0, g, i])
        assert abs(mp[0, 0, j] - want) <= 1e-12 * max(1.0, want)


def test_select_hand_cases():
    m = np.array([[[0.5, 0.9, 0.1, 0.9, 0.3, 0.9]]])
    # three tied maxima at rows 1, 3, 5; the two lowest rows win the tie
    assert oracle.select_retained(m, 2).tolist() == [[[1, 3]]]
    assert oracle.select_retained(m, 4).tolist() == [[[0, 1, 3, 5]]]
    assert oracle.select_retained(m, 6).tolist() == [[[0, 1, 2, 3, 4, 5]]]
    assert oracle.select_retained(m, 0).shape == (1, 1, 0)
    flat = np.zeros((1, 1, 7))
    assert oracle.select_retained(flat, 3).tolist() == [[[0, 1, 2]]]


def test_select_matches_sorted_brute_force():
    rng = np.random.default_rng(11)
    m = rng.integers(0, 20, size=(2, 3, 300)).astype(np.float64)  # many ties
    got = oracle.select_retained(m, 57)
    for b in range(2):
        for h in range(3):
            ranked = sorted(range(300), key=lambda j: (-m[b, h, j], j))[:57]
            assert got[b, h].tolist() == sorted(ranked)
