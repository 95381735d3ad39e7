"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Tolerances (max abs error vs the oracle): fp32 workloads 1e-5 on O and LSE;
bf16 workloads 1.5e-2 on O (and partial o) and 1e-3 on LSE (partials: m + ln l);
the gather is compared bit for bit. Small cases span several 64-key tiles,
ragged key and query tails, every wave count of the GQA packing and forced
split counts; the full-size workloads run in the launch configuration the
benchmark times and are checked on sampled (batch, q-head) pairs.
"""

import numpy as np
import pytest

import datagen
import oracle
from tests.gpu_util import TOL, bits, down, lse_of, max_err, say, up, worst

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ba():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import cached_block_attention_amd as mod
    mod.library()   # fails loudly when the library is missing
    return mod


def shape(name="dream_gqa", **kw):
    return datagen.scaled_shape(name, **kw)


def upload(inp):
    d = {k: up(getattr(inp, k)) for k in ("q", "k_pre", "v_pre", "k_blk", "v_blk")}
    d["idx"] = up(inp.idx) if inp.idx is not None else None
    return d


def check_full(ba, sh, splits=0, heads=None, seed_base=None):
    say(f"case full {sh} splits={splits}")
    inp = datagen.make_inputs(sh, seed_base)
    t = upload(inp)
    o, lse = ba.attention(t["q"], t["k_pre"], t["v_pre"], t["k_blk"], t["v_blk"], idx=t["idx"],
                          splits=splits)
    import torch
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.full(inp.q, inp.k_pre, inp.v_pre, inp.k_blk, inp.v_blk, sh.scale,
                                 idx=inp.idx, heads=heads)
    mask = ~np.isnan(lse_ref)
    tol = TOL[sh.dtype]
    eo = max_err(down(o), o_ref, mask[..., None].repeat(o_ref.shape[-1], -1))
    el = max_err(down(lse), lse_ref, mask)
    say(f"  max err O {eo:.3e} LSE {el:.3e}; worst O element {worst(down(o), o_ref, mask[..., None].repeat(o_ref.shape[-1], -1))}")
    assert eo <= tol["o"] and el <= tol["lse"], (eo, el)
    return o, lse


# ---------------------------------------------------------------------------
# blkattn_full on small shapes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("splits", [0, 1, 3])
def test_full_tiny_f32(ba, splits):
    check_full(ba, datagen.WORKLOADS["tiny_f32"], splits=splits)


@pytest.mark.parametrize("kw", [
    dict(batch=2, q_heads=8, kv_heads=2, prefix_len=1000, block_len=32),    # G=4, ragged P
    dict(batch=1, q_heads=4, kv_heads=4, prefix_len=777, block_len=32),     # G=1: one wave
    dict(batch=1, q_heads=14, kv_heads=2, prefix_len=500, block_len=64),    # 448 rows: 2 chunks
    dict(batch=2, q_heads=6, kv_heads=2, prefix_len=300, block_len=20),     # ragged rows
    dict(batch=1, q_heads=4, kv_heads=2, prefix_len=200, block_len=32, head_dim=64),
    dict(batch=1, q_heads=2, kv_heads=1, prefix_len=0, block_len=32),       # block only
    dict(batch=1, q_heads=1, kv_heads=1, prefix_len=70, block_len=1),       # one query
    dict(batch=1, q_heads=40, kv_heads=5, prefix_len=130, block_len=32),    # 8 waves
    dict(batch=1, q_heads=3, kv_heads=1, prefix_len=64, block_len=32),      # 3 waves, exact tiles
    dict(batch=1, q_heads=10, kv_heads=2, prefix_len=1000, block_len=32),   # 160 rows: waves 5, 6 idle
    dict(batch=2, q_heads=12, kv_heads=2, prefix_len=300, block_len=32),    # 192 rows: wave 6 idle
    dict(batch=1, q_heads=10, kv_heads=2, prefix_len=700, block_len=40),    # 200 rows: wave 6 part full
], ids=lambda kw: "-".join(f"{k}{v}" for k, v in kw.items()))
@pytest.mark.parametrize("splits", [0, 1, 2, 5])
def test_full_bf16_shapes(ba, kw, splits):
    check_full(ba, shape(**kw), splits=splits)


def test_full_f32_head_dim_128(ba):
    check_full(ba, datagen.scaled_shape("tiny_f32", head_dim=128, q_heads=4, kv_heads=2,
                                        prefix_len=100, block_len=40), splits=2)


def test_full_with_outliers(ba):
    sh = shape(batch=2, prefix_len=2048)
    assert sh.outlier_frac > 0
    check_full(ba, sh)


# Retained rows on the sequential kernel, where every row wave issues its share
# of each gathered tile: 64, 128 and 256 packed rows per workgroup (2, 4 and 8
# row waves). More than 8192 keys keep the plan from cutting the rows into
# one-wave chunks; ragged kept counts end the gathered rows inside a tile.
@pytest.mark.parametrize("kw", [
    dict(batch=2, q_heads=8, kv_heads=4, block_len=32, prefix_len=9000, n_keep=8213),   # 64 rows: 2 waves
    dict(batch=1, q_heads=16, kv_heads=4, block_len=32, prefix_len=9000, n_keep=8250),  # 128 rows: 4 waves
    dict(batch=1, q_heads=8, kv_heads=1, block_len=32, prefix_len=9000, n_keep=8301),   # 256 rows: 8 waves
], ids=["rows64", "rows128", "rows256"])
@pytest.mark.parametrize("splits", [0, 3])
def test_full_gathered_prefix_sequential_kernel(ba, kw, splits):
    check_full(ba, datagen.scaled_shape("sparse_gqa", **kw), splits=splits)


# One row wave and its DMA wave over splits of one to three 32-key tiles of
# retained rows (the block's keys after them): the first tiles are requested
# while the row wave's query loads are in flight.
@pytest.mark.parametrize("n_keep", [1, 40, 95])
@pytest.mark.parametrize("splits", [0, 2])
def test_full_few_retained_tiles_one_row_wave(ba, n_keep, splits):
    check_full(ba, datagen.scaled_shape("llada_bf16", q_heads=4, kv_heads=4, prefix_len=500, n_keep=n_keep),
               splits=splits)


# More partials than one chunk of the split merge, which folds them 16 at a
# time and carries the running max and sum from chunk to chunk (the last chunk
# ragged): forced split counts past 16 for each kernel family, for the final
# output and for a caller's partial.
@pytest.mark.parametrize("name,kw,splits", [
    ("dream_gqa", dict(batch=1, prefix_len=8192), 17),
    ("dream_gqa", dict(batch=1, prefix_len=8192), 40),
    ("llada_bf16", dict(q_heads=4, kv_heads=4, prefix_len=4096), 33),
    ("tiny_f32", dict(prefix_len=2048), 19),
])
def test_full_many_splits(ba, name, kw, splits):
    import torch
    sh = shape(name, **kw)
    q = torch.empty(sh.batch, sh.q_heads, sh.block_len, sh.head_dim, device="cuda",
                    dtype=torch.float32 if sh.dtype == datagen.F32 else torch.bfloat16)
    assert ba.plan_splits(ba.make_dims(q, sh.kv_heads, sh.prefix_len, splits=splits), ba.OP_FULL) == splits
    check_full(ba, sh, splits=splits)


def test_prefix_partial_many_splits(ba):
    import torch
    sh = shape(batch=1, prefix_len=8192)
    say(f"case prefix partial {sh} splits=24")
    inp = datagen.make_inputs(sh)
    t = upload(inp)
    pp = ba.prefix_partial(t["q"], t["k_pre"], t["v_pre"], splits=24)
    torch.cuda.synchronize()
    _check_partial(pp, _partial_ref(inp, sh, True), sh.dtype)


@pytest.mark.parametrize("splits", [0, 1, 4])
def test_full_gathered_prefix(ba, splits):
    check_full(ba, datagen.scaled_shape("sparse_gqa", prefix_len=3000, n_keep=700), splits=splits)


def test_zero_queries_give_column_mean(ba):
    import torch
    sh = shape(batch=1, q_heads=4, kv_heads=2, prefix_len=300, block_len=32)
    inp = datagen.make_inputs(sh)
    t = upload(inp)
    q = torch.zeros_like(t["q"])
    o, lse = ba.attention(q, t["k_pre"], t["v_pre"], t["k_blk"], t["v_blk"])
    for h in range(4):
        vals = np.concatenate([oracle.widen(inp.v_pre[0, h // 2]), oracle.widen(inp.v_blk[0, h // 2])])
        assert max_err(down(o)[0, h], np.broadcast_to(vals.mean(0), (32, 128))) <= TOL["bf16"]["o"]
    assert max_err(down(lse), np.log(332.0)) <= TOL["bf16"]["lse"]


def test_gqa_equals_repeated_mha(ba):
    import torch
    sh = shape(batch=1, q_heads=6, kv_heads=2, prefix_len=400, block_len=32)
    inp = datagen.make_inputs(sh)
    t = upload(inp)
    o1, l1 = ba.attention(t["q"], t["k_pre"], t["v_pre"], t["k_blk"], t["v_blk"], splits=2)
    rep = lambda x: x.repeat_interleave(3, dim=1).contiguous()  # noqa: E731
    o2, l2 = ba.attention(t["q"], rep(t["k_pre"]), rep(t["v_pre"]), rep(t["k_blk"]), rep(t["v_blk"]),
                          splits=2)
    torch.cuda.synchronize()
    assert max_err(down(o1), down(o2)) <= 1e-2 and max_err(down(l1), down(l2)) <= 1e-4


def test_strided_views(ba):
    # q and k/v given as non-contiguous views (head-major storage transposed)
    import torch
    sh = shape(batch=2, q_heads=4, kv_heads=2, prefix_len=333, block_len=32)
    inp = datagen.make_inputs(sh)
    t = upload(inp)
    tv = {k: t[k].transpose(1, 2).contiguous().transpose(1, 2) for k in ("q", "k_pre", "v_pre", "k_blk", "v_blk")}
    assert not tv["k_pre"].is_contiguous()
    o = torch.empty(2, 32, 4, 128, dtype=torch.bfloat16, device="cuda").transpose(1, 2)
    lse = torch.empty(2, 4, 32, dtype=torch.float32, device="cuda")
    ba.blkattn_full(tv["q"], tv["k_pre"], tv["v_pre"], tv["k_blk"], tv["v_blk"], o, lse)
    o_ref, lse_ref = oracle.full(inp.q, inp.k_pre, inp.v_pre, inp.k_blk, inp.v_blk, sh.scale)
    assert max_err(down(o), o_ref) <= TOL["bf16"]["o"] and max_err(down(lse), lse_ref) <= TOL["bf16"]["lse"]


def test_deterministic_bits(ba):
    import torch
    sh = shape(batch=2, prefix_len=3000)
    inp = datagen.make_inputs(sh)
    t = upload(inp)
    o1, l1 = ba.attention(t["q"], t["k_pre"], t["v_pre"], t["k_blk"], t["v_blk"])
    o2, l2 = ba.attention(t["q"], t["k_pre"], t["v_pre"], t["k_blk"], t["v_blk"])
    torch.cuda.synchronize()
    assert np.array_equal(bits(o1), bits(o2)) and np.array_equal(bits(l1), bits(l2))


# ---------------------------------------------------------------------------
# partials, merge (the cached-prefix path) and gather
# ---------------------------------------------------------------------------

def _partial_ref(inp, sh, prefix=True):
    if prefix:
        return oracle.partial(inp.q, inp.k_pre, inp.v_pre, sh.scale, idx=inp.idx)
    return oracle.partial(inp.q, inp.k_blk, inp.v_blk, sh.scale)


def _check_partial(got, ref, dtype):
    o, m, l = (down(x) for x in got)
    ro, rm, rl = ref
    eo = max_err(o, ro)
    el = max_err(lse_of(m, l), lse_of(rm, rl))
    say(f"  partial err o {eo:.3e} lse {el:.3e}")
    assert eo <= TOL[dtype]["o"] and el <= TOL[dtype]["lse"], (eo, el)
    assert np.all(l[np.isfinite(m)] >= 1.0 - 1e-4)        # the max term contributes 1


@pytest.mark.parametrize("name,kw", [
    ("tiny_f32", {}),
    ("dream_gqa", dict(batch=2, prefix_len=1500)),
    ("llada_bf16", dict(q_heads=4, kv_heads=4, prefix_len=900)),
    ("sparse_gqa", dict(prefix_len=2000, n_keep=333)),
])
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_prefix_block_partials_and_merge(ba, name, kw, splits):
    import torch
    sh = datagen.scaled_shape(name, **kw)
    say(f"case partials {sh} splits={splits}")
    inp = datagen.make_inputs(sh)
    t = upload(inp)
    pp = ba.prefix_partial(t["q"], t["k_pre"], t["v_pre"], idx=t["idx"], splits=splits)
    pb = ba.block_partial(t["q"], t["k_blk"], t["v_blk"])
    o, lse = ba.merge(pp, pb, dtype=t["q"].dtype)
    torch.cuda.synchronize()
    _check_partial(pp, _partial_ref(inp, sh, True), sh.dtype)
    _check_partial(pb, _partial_ref(inp, sh, False), sh.dtype)
    o_ref, lse_ref = oracle.full(inp.q, inp.k_pre, inp.v_pre, inp.k_blk, inp.v_blk, sh.scale, idx=inp.idx)
    assert max_err(down(o), o_ref) <= TOL[sh.dtype]["o"]
    assert max_err(down(lse), lse_ref) <= TOL[sh.dtype]["lse"]
    # in-place update of the cached state: ab aliases a
    ba.blkattn_merge(pp, pb, ab=pp)
    torch.cuda.synchronize()
    ro, rm, rl, rlse = oracle.merge(_partial_ref(inp, sh, True), _partial_ref(inp, sh, False))
    assert max_err(down(pp.o), ro) <= TOL[sh.dtype]["o"]
    assert max_err(lse_of(down(pp.m), down(pp.l)), rlse) <= TOL[sh.dtype]["lse"]


@pytest.mark.parametrize("name,kw", [
    ("tiny_f32", {}),
    ("dream_gqa", dict(batch=2, prefix_len=1500)),
    ("dream_gqa", dict(batch=1, q_heads=14, kv_heads=2, prefix_len=700, block_len=64)),
    ("llada_bf16", dict(q_heads=4, kv_heads=4, prefix_len=900)),
    ("sparse_gqa", dict(prefix_len=2000, n_keep=333)),
    ("dream_gqa", dict(batch=1, q_heads=6, kv_heads=2, prefix_len=300, block_len=20, head_dim=64)),
])
def test_block_step_continues_the_cached_state(ba, name, kw):
    # one launch: state initialised from the cached prefix partial, continued
    # over the block keys == full attention (same queries) == partial + merge
    import torch
    sh = datagen.scaled_shape(name, **kw)
    say(f"case block step {sh}")
    inp = datagen.make_inputs(sh)
    t = upload(inp)
    pp = ba.prefix_partial(t["q"], t["k_pre"], t["v_pre"], idx=t["idx"])
    o, lse = ba.block_step(t["q"], t["k_blk"], t["v_blk"], pp)
    pb = ba.block_partial(t["q"], t["k_blk"], t["v_blk"])
    o2, lse2 = ba.merge(pp, pb, dtype=t["q"].dtype)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.full(inp.q, inp.k_pre, inp.v_pre, inp.k_blk, inp.v_blk, sh.scale, idx=inp.idx)
    tol = TOL[sh.dtype]
    eo, el = max_err(down(o), o_ref), max_err(down(lse), lse_ref)
    say(f"  block step err O {eo:.3e} LSE {el:.3e}")
    assert eo <= tol["o"] and el <= tol["lse"], (eo, el)
    # two results each within tol of the oracle are within 2 tol of each other;
    # their bf16 roundings need not coincide (one ulp is 0.0156 for |O| in [2, 4))
    assert max_err(down(o), down(o2)) <= 2 * tol["o"] and max_err(down(lse), down(lse2)) <= 2 * tol["lse"]


def test_block_step_from_empty_and_from_other_queries(ba):
    import torch
    sh = shape(batch=1, q_heads=8, kv_heads=2, prefix_len=400, block_len=32)
    inp = datagen.make_inputs(sh)
    t = upload(inp)
    # an empty cached state gives block-only attention
    empty = ba.empty_partial(1, 8, 32, 128, "cuda")
    empty.o.zero_()
    empty.m.fill_(-float("inf"))
    empty.l.zero_()
    o, lse = ba.block_step(t["q"], t["k_blk"], t["v_blk"], empty)
    torch.cuda.synchronize()
    bo, bl = oracle.full(inp.q, inp.k_pre[:, :, :0], inp.v_pre[:, :, :0], inp.k_blk, inp.v_blk, sh.scale)
    assert max_err(down(o), bo) <= TOL["bf16"]["o"] and max_err(down(lse), bl) <= TOL["bf16"]["lse"]
    # a state cached from other (step-0) queries, continued with fresh block
    # queries: the composition merge(partial(Q_fix; prefix), partial(Q_t; block))
    q1_np, kb_np, vb_np = datagen.step_inputs(sh, 1)
    pp = ba.prefix_partial(t["q"], t["k_pre"], t["v_pre"])
    o, lse = ba.block_step(up(q1_np), up(kb_np), up(vb_np), pp)
    torch.cuda.synchronize()
    ro, rm, rl, rlse = oracle.merge(oracle.partial(inp.q, inp.k_pre, inp.v_pre, sh.scale),
                                    oracle.partial(q1_np, kb_np, vb_np, sh.scale))
    assert max_err(down(o), ro) <= TOL["bf16"]["o"] and max_err(down(lse), rlse) <= TOL["bf16"]["lse"]


def test_empty_prefix_partial_and_merges(ba):
    import torch
    sh = shape(batch=1, q_heads=4, kv_heads=2, prefix_len=0, block_len=32)
    inp = datagen.make_inputs(sh)
    t = upload(inp)
    pe = ba.prefix_partial(t["q"], t["k_pre"], t["v_pre"])
    torch.cuda.synchronize()
    assert np.all(down(pe.o) == 0) and np.all(np.isneginf(down(pe.m))) and np.all(down(pe.l) == 0)
    pb = ba.block_partial(t["q"], t["k_blk"], t["v_blk"])
    o, lse = ba.merge(pe, pb, dtype=torch.float32)
    o2, lse2 = ba.merge(pb, pe, dtype=torch.float32)
    torch.cuda.synchronize()
    # w*o/w in fp32: equal to the block partial up to rounding
    assert max_err(down(o), down(pb.o)) <= 1e-6 and max_err(down(o2), down(pb.o)) <= 1e-6
    assert max_err(down(lse), lse_of(down(pb.m), down(pb.l))) <= 1e-6
    oe, le = ba.merge(pe, pe, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert np.all(down(oe) == 0) and np.all(np.isneginf(down(le)))


def test_block_step_ignores_the_o_of_empty_cached_rows(ba):
    # rows whose cached state is empty (m = -inf, l = 0) start from nothing,
    # whatever their cached o holds (NaN here): block-only attention for those
    # rows, the cached state continued for the others
    import torch
    sh = shape(batch=2, q_heads=8, kv_heads=2, prefix_len=600, block_len=32)
    say(f"case block step over partly empty cached rows {sh}")
    inp = datagen.make_inputs(sh)
    t = upload(inp)
    pp = ba.prefix_partial(t["q"], t["k_pre"], t["v_pre"])
    dead = np.random.default_rng(7).random(tuple(pp.m.shape)) < 0.3
    dt = torch.from_numpy(dead).cuda()
    pp.m[dt] = -float("inf")
    pp.l[dt] = 0.0
    pp.o[dt] = float("nan")
    o, lse = ba.block_step(t["q"], t["k_blk"], t["v_blk"], pp)
    torch.cuda.synchronize()
    ro, rm, rl = oracle.partial(inp.q, inp.k_pre, inp.v_pre, sh.scale)
    ro[dead], rm[dead], rl[dead] = 0.0, -np.inf, 0.0
    want_o, _, _, want_lse = oracle.merge((ro, rm, rl), oracle.partial(inp.q, inp.k_blk, inp.v_blk, sh.scale))
    got_o, got_lse = down(o), down(lse)
    assert not np.isnan(got_o).any() and not np.isnan(got_lse).any()
    eo, el = max_err(got_o, want_o), max_err(got_lse, want_lse)
    say(f"  max err O {eo:.3e} LSE {el:.3e} ({int(dead.sum())} of {dead.size} rows empty)")
    assert eo <= TOL["bf16"]["o"] and el <= TOL["bf16"]["lse"], (eo, el)


@pytest.mark.parametrize("kw", [dict(batch=2, q_heads=4, kv_heads=2, prefix_len=63, block_len=1),
                                dict(batch=1, q_heads=28, kv_heads=4, prefix_len=700, block_len=32)],
                         ids=["B2-G2x2-P63-Bq1", "B1-G7x4-P700-Bq32"])
def test_empty_retained_set_is_an_empty_prefix(ba, kw):
    # n_keep = 0 beside a dense prefix: the keys are the block's alone (an
    # empty index tensor has no device address; it must not read as "dense")
    import torch
    sh = datagen.scaled_shape("sparse_gqa", n_keep=0, **kw)
    say(f"case empty retained set {sh}")
    inp = datagen.make_inputs(sh)
    assert inp.idx is not None and inp.idx.shape[-1] == 0
    t = upload(inp)
    o, lse = ba.attention(t["q"], t["k_pre"], t["v_pre"], t["k_blk"], t["v_blk"], idx=t["idx"])
    pp = ba.prefix_partial(t["q"], t["k_pre"], t["v_pre"], idx=t["idx"])
    ko = torch.empty(sh.batch, sh.kv_heads, 0, sh.head_dim, dtype=t["k_pre"].dtype, device="cuda")
    ba.blkattn_gather_prefix(t["k_pre"], t["v_pre"], t["idx"], ko, ko.clone())
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.full(inp.q, inp.k_pre, inp.v_pre, inp.k_blk, inp.v_blk, sh.scale, idx=inp.idx)
    eo, el = max_err(down(o), o_ref), max_err(down(lse), lse_ref)
    say(f"  max err O {eo:.3e} LSE {el:.3e}")
    assert eo <= TOL[sh.dtype]["o"] and el <= TOL[sh.dtype]["lse"], (eo, el)
    assert np.all(down(pp.o) == 0) and np.all(np.isneginf(down(pp.m))) and np.all(down(pp.l) == 0)


@pytest.mark.parametrize("dtype_name,kw", [("bf16", dict(prefix_len=3000, n_keep=700)),
                                           ("f32", dict(prefix_len=500, n_keep=77))])
def test_gather_bit_exact(ba, dtype_name, kw):
    base = "sparse_gqa" if dtype_name == "bf16" else "tiny_f32"
    sh = datagen.scaled_shape(base, **kw)
    if dtype_name == "f32":
        import dataclasses
        sh = dataclasses.replace(sh, n_keep=kw["n_keep"])
    inp = datagen.make_inputs(sh)
    if inp.idx is None:
        inp.idx = datagen.retained_indices(sh.batch, sh.kv_heads, sh.prefix_len, kw["n_keep"], 77)
    t = upload(inp)
    idx = up(inp.idx)
    ko, vo = ba.gather_prefix(t["k_pre"], t["v_pre"], idx)
    assert np.array_equal(bits(ko), oracle.gather(inp.k_pre, inp.idx))
    assert np.array_equal(bits(vo), oracle.gather(inp.v_pre, inp.idx))


def test_gather_then_dense_matches_fused(ba):
    import torch
    sh = datagen.scaled_shape("sparse_gqa", prefix_len=5000, n_keep=1000)
    inp = datagen.make_inputs(sh)
    t = upload(inp)
    ko, vo = ba.gather_prefix(t["k_pre"], t["v_pre"], t["idx"])
    o1, l1 = ba.attention(t["q"], ko, vo, t["k_blk"], t["v_blk"], splits=4)
    o2, l2 = ba.attention(t["q"], t["k_pre"], t["v_pre"], t["k_blk"], t["v_blk"], idx=t["idx"], splits=4)
    torch.cuda.synchronize()
    # same keys in the same tile order: identical bits
    assert np.array_equal(bits(o1), bits(o2)) and np.array_equal(bits(l1), bits(l2))


def test_identity_indices_equal_dense(ba):
    import torch
    sh = shape(batch=1, q_heads=7, kv_heads=1, prefix_len=600, block_len=32)
    inp = datagen.make_inputs(sh)
    t = upload(inp)
    ident = torch.arange(600, dtype=torch.int32, device="cuda").view(1, 1, 600).contiguous()
    o1, l1 = ba.attention(t["q"], t["k_pre"], t["v_pre"], t["k_blk"], t["v_blk"], idx=ident, splits=3)
    o2, l2 = ba.attention(t["q"], t["k_pre"], t["v_pre"], t["k_blk"], t["v_blk"], splits=3)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o1), bits(o2)) and np.array_equal(bits(l1), bits(l2))
