"""Pins of the fp64 oracle to facts it does not compute itself.

Each test ties an oracle function to something other than its own code: a
pure-Python per-element evaluation, a closed form, an invariant of softmax
attention, a special case that reduces to a simpler routine, or values derived
by hand (tests/golden/hand_cases.json). The mutation tests at the end plant
plausible mistakes in copies of the oracle and check that a pin catches each.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import attention as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(seed, *shape, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------------------
# independent evaluations
# ---------------------------------------------------------------------------

def brute_row(q, keys, values, scale):
    """Per-element softmax attention in pure Python (no max shift, no numpy)."""
    s = [scale * sum(float(a) * float(b) for a, b in zip(q, k)) for k in keys]
    e = [math.exp(x) for x in s]
    z = sum(e)
    o = [sum(e[j] * float(values[j][c]) for j in range(len(keys))) / z
         for c in range(len(values[0]))]
    return o, math.log(z)


def brute_full(q, k_pre, v_pre, k_blk, v_blk, scale, idx=None):
    """Per-element evaluation; the scale is the float32 value a kernel receives."""
    scale = float(np.float32(scale))
    B, Hq, Bq, d = q.shape
    Hkv = k_pre.shape[1]
    G = Hq // Hkv
    o = np.zeros(q.shape[:3] + (v_pre.shape[3],))
    lse = np.zeros(q.shape[:3])
    for b in range(B):
        for h in range(Hq):
            g = h // G
            rows = range(k_pre.shape[2]) if idx is None else [int(r) for r in idx[b, g]]
            keys = [k_pre[b, g, r] for r in rows] + [k_blk[b, g, r] for r in range(k_blk.shape[2])]
            vals = [v_pre[b, g, r] for r in rows] + [v_blk[b, g, r] for r in range(v_blk.shape[2])]
            for i in range(Bq):
                oo, ll = brute_row(q[b, h, i], keys, vals, scale)
                o[b, h, i], lse[b, h, i] = oo, ll
    return o, lse


def tiny_case(seed, B=1, Hq=2, Hkv=1, Bq=3, P=4, d=3, scale=0.7):
    g = np.random.default_rng(seed)
    f = lambda *s: g.standard_normal(s)  # noqa: E731
    return (f(B, Hq, Bq, d), f(B, Hkv, P, d), f(B, Hkv, P, d), f(B, Hkv, Bq, d),
            f(B, Hkv, Bq, d), scale)


# ---------------------------------------------------------------------------
# full attention
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_full_matches_brute_force(seed):
    q, kp, vp, kb, vb, sc = tiny_case(seed, B=2, Hq=4, Hkv=2, Bq=3, P=2, d=3)
    o, lse = oracle.full(q, kp, vp, kb, vb, sc)
    ob, lb = brute_full(q, kp, vp, kb, vb, sc)
    assert np.max(np.abs(o - ob)) < 1e-13
    assert np.max(np.abs(lse - lb)) < 1e-13


def test_two_keys_closed_form():
    # one query, one prefix key, one block key: weights are logistic sigmoids
    q = rnd(3, 1, 1, 1, 4)
    kp, vp, kb, vb = (rnd(4 + i, 1, 1, 1, 4) for i in range(4))
    sc = 0.5
    o, lse = oracle.full(q, kp, vp, kb, vb, sc)
    s1 = float(np.float32(sc)) * float(q[0, 0, 0] @ kp[0, 0, 0])
    s2 = float(np.float32(sc)) * float(q[0, 0, 0] @ kb[0, 0, 0])
    sig = lambda x: 1.0 / (1.0 + math.exp(-x))  # noqa: E731
    want = sig(s1 - s2) * vp[0, 0, 0] + sig(s2 - s1) * vb[0, 0, 0]
    assert np.max(np.abs(o[0, 0, 0] - want)) < 1e-14
    assert abs(lse[0, 0, 0] - math.log(math.exp(s1) + math.exp(s2))) < 1e-14


def test_zero_queries_give_column_mean():
    _, kp, vp, kb, vb, sc = tiny_case(5, B=1, Hq=2, Hkv=2, Bq=4, P=7, d=5)
    q = np.zeros((1, 2, 4, 5))
    o, lse = oracle.full(q, kp, vp, kb, vb, sc)
    for h in range(2):
        mean = np.concatenate([vp[0, h], vb[0, h]]).mean(axis=0)
        assert np.max(np.abs(o[0, h] - mean)) < 1e-14
    assert np.max(np.abs(lse - math.log(7 + 4))) < 1e-14


@pytest.mark.parametrize("jstar", ["last_block", "first_prefix", "mid_prefix"])
def test_one_hot_score(jstar):
    # every key is orthogonal to e1 except key j*, which is a*e1; the query
    # row i is c*e1 -> o_i = (e^t v_j* + sum_{j!=j*} v_j) / (e^t + N - 1)
    P, Bq, d, c, a, sc = 6, 3, 4, 1.5, 2.0, 0.8
    kp = np.zeros((1, 1, P, d)); kp[..., 1:] = rnd(7, 1, 1, P, d - 1)
    kb = np.zeros((1, 1, Bq, d)); kb[..., 1:] = rnd(8, 1, 1, Bq, d - 1)
    vp, vb = rnd(9, 1, 1, P, d), rnd(10, 1, 1, Bq, d)
    j = {"last_block": P + Bq - 1, "first_prefix": 0, "mid_prefix": 3}[jstar]
    keys = np.concatenate([kp, kb], axis=2)
    keys[0, 0, j] = 0.0
    keys[0, 0, j, 0] = a
    kp, kb = keys[:, :, :P], keys[:, :, P:]
    q = np.zeros((1, 1, Bq, d))
    q[0, 0, 0, 0] = c            # query 0 is one-hot; the others are zero
    o, lse = oracle.full(q, kp, vp, kb, vb, sc)
    vals = np.concatenate([vp, vb], axis=2)[0, 0]
    N = P + Bq
    t = c * a * float(np.float32(sc))
    want = (math.exp(t) * vals[j] + vals.sum(axis=0) - vals[j]) / (math.exp(t) + N - 1)
    assert np.max(np.abs(o[0, 0, 0] - want)) < 1e-14
    assert abs(lse[0, 0, 0] - math.log(math.exp(t) + N - 1)) < 1e-14
    # the other (zero) queries weight every key equally: no causal mask
    assert np.max(np.abs(o[0, 0, 1] - vals.mean(axis=0))) < 1e-14


def test_constant_values_and_linearity():
    q, kp, vp, kb, vb, sc = tiny_case(11, B=1, Hq=2, Hkv=1, Bq=3, P=5, d=4)
    o1, _ = oracle.full(q, kp, np.ones_like(vp), kb, np.ones_like(vb), sc)
    assert np.max(np.abs(o1 - 1.0)) < 1e-14
    vp2, vb2 = rnd(12, *vp.shape), rnd(13, *vb.shape)
    oa, _ = oracle.full(q, kp, vp, kb, vb, sc)
    ob, _ = oracle.full(q, kp, vp2, kb, vb2, sc)
    oc, _ = oracle.full(q, kp, 2.0 * vp - 3.0 * vp2, kb, 2.0 * vb - 3.0 * vb2, sc)
    assert np.max(np.abs(oc - (2.0 * oa - 3.0 * ob))) < 1e-13


def test_key_permutation_invariance():
    q, kp, vp, kb, vb, sc = tiny_case(14, B=1, Hq=1, Hkv=1, Bq=2, P=6, d=3)
    o, lse = oracle.full(q, kp, vp, kb, vb, sc)
    perm = np.random.default_rng(15).permutation(6)
    o2, lse2 = oracle.full(q, kp[:, :, perm], vp[:, :, perm], kb, vb, sc)
    assert np.max(np.abs(o - o2)) < 1e-14 and np.max(np.abs(lse - lse2)) < 1e-13


def test_shift_invariance():
    # adding the same vector u to every key leaves o unchanged, lse += scale q.u
    q, kp, vp, kb, vb, sc = tiny_case(16, B=1, Hq=2, Hkv=2, Bq=3, P=4, d=5)
    u = rnd(17, 5)
    o, lse = oracle.full(q, kp, vp, kb, vb, sc)
    o2, lse2 = oracle.full(q, kp + u, vp, kb + u, vb, sc)
    assert np.max(np.abs(o - o2)) < 1e-13
    assert np.max(np.abs(lse2 - lse - float(np.float32(sc)) * (q @ u))) < 1e-13


def test_gqa_equals_repeated_mha():
    q, kp, vp, kb, vb, sc = tiny_case(18, B=2, Hq=6, Hkv=2, Bq=2, P=5, d=3)
    o, lse = oracle.full(q, kp, vp, kb, vb, sc)
    rep = lambda x: np.repeat(x, 3, axis=1)  # noqa: E731  kv head g serves q heads 3g..3g+2
    o2, lse2 = oracle.full(q, rep(kp), rep(vp), rep(kb), rep(vb), sc)
    assert np.max(np.abs(o - o2)) < 1e-15 and np.max(np.abs(lse - lse2)) < 1e-15


def test_hand_derived_golden_cases():
    with open(os.path.join(GOLDEN, "hand_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q = np.array(c["q"], dtype=np.float64)[None, None, None, :]
        kp = np.array(c["k_prefix"], dtype=np.float64)[None, None]
        vp = np.array(c["v_prefix"], dtype=np.float64)[None, None]
        kb = np.array(c["k_block"], dtype=np.float64)[None, None]
        vb = np.array(c["v_block"], dtype=np.float64)[None, None]
        o, lse = oracle.full(q, kp, vp, kb, vb, c["scale"])
        assert np.max(np.abs(o[0, 0, 0] - np.array(c["o"]))) < 1e-12, c["name"]
        assert abs(lse[0, 0, 0] - c["lse"]) < 1e-12, c["name"]


def test_bf16_bits_widen_exactly():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F7F, 0x0001, 0x3EAB], dtype=np.uint16)
    want = [1.0, -2.0, 0.0, -0.0, 3.3895313892515355e38, 9.183549615799121e-41, 0.333984375]
    assert list(oracle.widen(bits)) == want


# ---------------------------------------------------------------------------
# partial states and their merge
# ---------------------------------------------------------------------------

def test_partial_bounds_and_max():
    q, kp, vp, _, _, sc = tiny_case(19, B=1, Hq=2, Hkv=1, Bq=4, P=9, d=3)
    o, m, l = oracle.partial(q, kp, vp, sc)
    lse = oracle.finalize(m, l)
    scf = float(np.float32(sc))
    for h in range(2):
        for i in range(4):
            s = [scf * sum(q[0, h, i, c] * kp[0, 0, j, c] for c in range(3)) for j in range(9)]
            assert abs(m[0, h, i] - max(s)) < 1e-14
    assert np.all(l >= 1.0 - 1e-15) and np.all(l <= 9 + 1e-12)
    assert np.all(lse >= m - 1e-15) and np.all(lse <= m + math.log(9) + 1e-12)
    ob, lb = brute_full(q, kp, vp, np.zeros((1, 1, 0, 3)), np.zeros((1, 1, 0, 3)), sc)
    assert np.max(np.abs(o - ob)) < 1e-13 and np.max(np.abs(lse - lb)) < 1e-13


def test_split_invariance_every_split_point():
    q, kp, vp, kb, vb, sc = tiny_case(20, B=1, Hq=2, Hkv=1, Bq=3, P=7, d=4)
    o_full, lse_full = oracle.full(q, kp, vp, kb, vb, sc)
    keys = np.concatenate([kp, kb], axis=2)
    vals = np.concatenate([vp, vb], axis=2)
    N = keys.shape[2]
    for k in range(N + 1):                       # includes both empty sides
        a = oracle.partial(q, keys[:, :, :k], vals[:, :, :k], sc)
        b = oracle.partial(q, keys[:, :, k:], vals[:, :, k:], sc)
        o, m, l, lse = oracle.merge(a, b)
        assert np.max(np.abs(o - o_full)) < 1e-13, k
        assert np.max(np.abs(lse - lse_full)) < 1e-12, k


def test_merge_commutative_associative_many_way():
    q, kp, vp, kb, vb, sc = tiny_case(21, B=1, Hq=1, Hkv=1, Bq=2, P=12, d=3)
    o_full, lse_full = oracle.full(q, kp, vp, kb, vb, sc)
    keys = np.concatenate([kp, kb], axis=2)
    vals = np.concatenate([vp, vb], axis=2)
    cuts = [0, 3, 4, 9, 14]
    parts = [oracle.partial(q, keys[:, :, a:b], vals[:, :, a:b], sc)
             for a, b in zip(cuts[:-1], cuts[1:])]
    left = parts[0]
    for p in parts[1:]:
        left = oracle.merge(left, p)[:3]
    right = parts[-1]
    for p in reversed(parts[:-1]):
        right = oracle.merge(p, right)[:3]
    tree = oracle.merge(oracle.merge(parts[2], parts[0])[:3], oracle.merge(parts[3], parts[1])[:3])[:3]
    for st in (left, right, tree):
        assert np.max(np.abs(st[0] - o_full)) < 1e-13
        assert np.max(np.abs(oracle.finalize(st[1], st[2]) - lse_full)) < 1e-12


def test_merge_with_empty_sides():
    q, kp, vp, _, _, sc = tiny_case(22, B=1, Hq=1, Hkv=1, Bq=2, P=5, d=3)
    a = oracle.partial(q, kp, vp, sc)
    e = oracle.partial(q, kp[:, :, :0], vp[:, :, :0], sc)
    assert np.all(e[0] == 0) and np.all(np.isneginf(e[1])) and np.all(e[2] == 0)
    for o, m, l, lse in (oracle.merge(a, e), oracle.merge(e, a)):
        assert np.max(np.abs(o - a[0])) < 1e-15
        assert np.max(np.abs(m - a[1])) == 0 and np.max(np.abs(l - a[2])) < 1e-15
    o, m, l, lse = oracle.merge(e, e)
    assert np.all(o == 0) and np.all(np.isneginf(m)) and np.all(l == 0) and np.all(np.isneginf(lse))
    assert not np.any(np.isnan(o))


def test_online_recurrence_equals_definition_any_tile():
    # eqs. 2-6 streamed over tiles of any size reach the plain softmax
    q = rnd(23, 5, 6)
    keys, vals = rnd(24, 37, 6, scale=2.0), rnd(25, 37, 6)
    o_def, lse_def = A.attention_rows(q, keys, vals, 0.4)
    for tile in (1, 2, 5, 16, 37, 64):
        m, l, ot = oracle.online_state(q, keys, vals, 0.4, tile)
        assert np.max(np.abs(ot / l[:, None] - o_def)) < 1e-13, tile
        assert np.max(np.abs(m + np.log(l) - lse_def)) < 1e-13, tile


def test_cached_state_continuation_equals_merge():
    # FACache: state over U tiles, cached, then later steps start from it and
    # stream only the block's tiles; equals merging the two partials.
    q = rnd(26, 4, 5)
    ku, vu = rnd(27, 20, 5), rnd(28, 20, 5)
    kc, vc = rnd(29, 6, 5), rnd(30, 6, 5)
    cached = oracle.online_state(q, ku, vu, 0.6, tile=8)
    m, l, ot = oracle.online_state(q, kc, vc, 0.6, tile=4, state=cached)
    Q = q[None, None]
    pa = oracle.partial(Q, ku[None, None], vu[None, None], 0.6)
    pb = oracle.partial(Q, kc[None, None], vc[None, None], 0.6)
    o, mm, ll, lse = oracle.merge(pa, pb)
    assert np.max(np.abs(ot / l[:, None] - o[0, 0])) < 1e-13
    assert np.max(np.abs(m + np.log(l) - lse[0, 0])) < 1e-13
    # and the state round-trips through the normalised partial form
    m2, l2, ot2 = oracle.state_from_partial(*[x[0, 0] for x in pa])
    assert np.max(np.abs(ot2 - cached[2])) < 1e-12


# ---------------------------------------------------------------------------
# retained-row gather
# ---------------------------------------------------------------------------

def test_gather_row_tags_and_bits():
    B, H, P, d, n = 2, 3, 50, 4, 17
    g = np.random.default_rng(31)
    x = g.integers(0, 65536, size=(B, H, P, d), dtype=np.uint16)
    x[..., 0] = np.arange(P, dtype=np.uint16)            # tag each row with its index
    x[..., 1] = (np.arange(B)[:, None, None] * 16 + np.arange(H)[None, :, None]).astype(np.uint16)
    idx = np.sort(np.stack([np.stack([g.choice(P, n, replace=False) for _ in range(H)])
                            for _ in range(B)]), axis=-1).astype(np.int32)
    out = oracle.gather(x, idx)
    assert out.dtype == np.uint16
    assert np.array_equal(out[..., 0].astype(np.int32), idx)
    assert np.array_equal(out[..., 1], np.broadcast_to(x[:, :, :1, 1], out[..., 1].shape))
    ident = np.broadcast_to(np.arange(P, dtype=np.int32), (B, H, P)).copy()
    assert np.array_equal(oracle.gather(x, ident), x)


def test_full_with_idx_equals_dense_on_kept_rows():
    q, kp, vp, kb, vb, sc = tiny_case(32, B=2, Hq=4, Hkv=2, Bq=2, P=9, d=3)
    idx = np.array([[[0, 2, 3, 8], [1, 4, 5, 7]], [[2, 3, 6, 8], [0, 1, 2, 3]]], dtype=np.int32)
    o, lse = oracle.full(q, kp, vp, kb, vb, sc, idx=idx)
    ob, lb = brute_full(q, kp, vp, kb, vb, sc, idx=idx)
    assert np.max(np.abs(o - ob)) < 1e-13 and np.max(np.abs(lse - lb)) < 1e-13
    ident = np.broadcast_to(np.arange(9, dtype=np.int32), (2, 2, 9)).copy()
    o2, l2 = oracle.full(q, kp, vp, kb, vb, sc, idx=ident)
    o3, l3 = oracle.full(q, kp, vp, kb, vb, sc)
    assert np.max(np.abs(o2 - o3)) == 0 and np.max(np.abs(l2 - l3)) == 0


def test_heads_sample_matches_full_evaluation():
    q, kp, vp, kb, vb, sc = tiny_case(33, B=2, Hq=4, Hkv=2, Bq=2, P=5, d=3)
    o, lse = oracle.full(q, kp, vp, kb, vb, sc)
    os_, ls_ = oracle.full(q, kp, vp, kb, vb, sc, heads=[(1, 3), (0, 1)])
    assert np.array_equal(os_[1, 3], o[1, 3]) and np.array_equal(ls_[0, 1], lse[0, 1])
    assert np.isnan(os_[0, 0]).all()


# ---------------------------------------------------------------------------
# planted mistakes: each mutant of the oracle must fail at least one pin
# ---------------------------------------------------------------------------

def _mutant_full(kind):
    def f(q, k_pre, v_pre, k_blk, v_blk, scale, idx=None, heads=None):
        if kind == "no_scale":
            return A.full(q, k_pre, v_pre, k_blk, v_blk, 1.0, idx)
        if kind == "gqa_modulo":
            Hq, Hkv = q.shape[1], k_pre.shape[1]
            perm = [h % Hkv for h in range(Hq)]
            o = np.zeros(q.shape[:3] + (v_pre.shape[3],)); lse = np.zeros(q.shape[:3])
            for h in range(Hq):
                oo, ll = A.full(q[:, h:h + 1], k_pre[:, perm[h]:perm[h] + 1],
                                v_pre[:, perm[h]:perm[h] + 1], k_blk[:, perm[h]:perm[h] + 1],
                                v_blk[:, perm[h]:perm[h] + 1], scale, None)
                o[:, h], lse[:, h] = oo[:, 0], ll[:, 0]
            return o, lse
        if kind == "causal_block":
            # block query i only sees block keys <= i
            B, Hq, Bq, _ = q.shape
            o = np.zeros(q.shape[:3] + (v_pre.shape[3],)); lse = np.zeros(q.shape[:3])
            for i in range(Bq):
                oo, ll = A.full(q[:, :, i:i + 1], k_pre, v_pre, k_blk[:, :, :i + 1],
                                v_blk[:, :, :i + 1], scale, idx)
                o[:, :, i], lse[:, :, i] = oo[:, :, 0], ll[:, :, 0]
            return o, lse
        if kind == "kt_transposed_values":
            return A.full(q, k_pre, k_pre, k_blk, k_blk, scale, idx)
        raise ValueError(kind)
    return f


@pytest.mark.parametrize("kind", ["no_scale", "gqa_modulo", "causal_block", "kt_transposed_values"])
def test_mutants_of_full_are_caught(kind):
    mut = _mutant_full(kind)
    q, kp, vp, kb, vb, sc = tiny_case(40, B=1, Hq=4, Hkv=2, Bq=3, P=3, d=3)
    o, lse = mut(q, kp, vp, kb, vb, sc)
    ob, lb = brute_full(q, kp, vp, kb, vb, sc)
    assert np.max(np.abs(o - ob)) > 1e-6 or np.max(np.abs(lse - lb)) > 1e-6


def _mutant_merge(kind):
    def f(a, b):
        oa, ma, la = a
        ob, mb, lb = b
        M = np.maximum(ma, mb)
        if kind == "wrong_sign":
            wa, wb = la * np.exp(M - ma), lb * np.exp(M - mb)
        elif kind == "drop_l":
            wa, wb = np.exp(ma - M), np.exp(mb - M)
        else:
            raise ValueError(kind)
        l = wa + wb
        o = (wa[..., None] * oa + wb[..., None] * ob) / l[..., None]
        return o, M, l, M + np.log(l)
    return f


@pytest.mark.parametrize("kind", ["wrong_sign", "drop_l"])
def test_mutants_of_merge_are_caught(kind):
    mut = _mutant_merge(kind)
    q, kp, vp, kb, vb, sc = tiny_case(41, B=1, Hq=1, Hkv=1, Bq=3, P=6, d=3)
    o_full, _ = oracle.full(q, kp, vp, kb, vb, sc)
    keys = np.concatenate([kp, kb], axis=2)
    vals = np.concatenate([vp, vb], axis=2)
    a = oracle.partial(q, keys[:, :, :2], vals[:, :, :2], sc)
    b = oracle.partial(q, keys[:, :, 2:], vals[:, :, 2:], sc)
    o, *_ = mut(a, b)
    assert np.max(np.abs(o - o_full)) > 1e-6
