"""GPU parity where the online-softmax reference moves: the row maximum arrives
late (in the last tile of the last key split, in the block's own tile, or in a
retained row of a gathered prefix), scores span far more than the kernels'
lazy-rescale window (2^8 in exp2 units), and scores ramp up tile after tile.
These are the rescale steps of eqs. 3-6 in section 3.3.3 of "LaCache: Exact
Caching and Precision-Adaptive Inference for Diffusion Large Language Models"
(running max, alpha = e^{m_old - m_new} applied to l and O~).

Every case compares blkattn_full (through the C ABI) with the fp64 oracle
element by element, at the stated bf16 tolerance (O 1.5e-2, LSE 1e-3); the
oracle's own one-hot closed form is pinned in test_oracle_pins.py.
"""

import numpy as np
import pytest

import datagen
import oracle
from tests.gpu_util import TOL, down, max_err, say, up

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ba():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import cached_block_attention_amd as mod
    mod.library()
    return mod


def bf(x):
    return datagen.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def one_hot_inputs(sh, where: str):
    """Queries point along head dimension 0 with row-dependent strength;
    every key has component 0 equal to zero except one special key per
    (batch, kv-head), so a row's scores are 0 except at that key, where they
    are far above the lazy-rescale window (up to scale*64*16 = 90 natural-log
    units)."""
    inp = datagen.make_inputs(sh)
    B, Hq, Bq, d = inp.q.shape
    strengths = np.array([8.0, 16.0, 32.0, 64.0], dtype=np.float32)
    q = np.zeros((B, Hq, Bq, d), dtype=np.float32)
    q[..., 0] = strengths[np.arange(Bq) % 4][None, None, :]
    inp.q = bf(q)
    inp.k_pre[..., 0] = 0
    inp.k_blk[..., 0] = 0
    a = bf(16.0)
    if where == "last_prefix":
        inp.k_pre[:, :, -1, 0] = a
    elif where == "last_block":
        inp.k_blk[:, :, -1, 0] = a
    elif where == "first_prefix":
        inp.k_pre[:, :, 0, 0] = a
    elif where == "last_kept":
        for b in range(B):
            for h in range(inp.k_pre.shape[1]):
                inp.k_pre[b, h, inp.idx[b, h, -1], 0] = a
    else:
        raise ValueError(where)
    return inp


def ramp_inputs(sh, total: float):
    """Scores that grow along the keys: key j's component 0 is
    total * j / (N_k - 1) (prefix then block), queries e_0 * 8: the running max
    rises at every tile, by about total * 64 / N_k per 64-key tile."""
    inp = datagen.make_inputs(sh)
    B, Hq, Bq, d = inp.q.shape
    q = np.zeros((B, Hq, Bq, d), dtype=np.float32)
    q[..., 0] = 8.0
    inp.q = bf(q)
    P = inp.k_pre.shape[2]
    nk = P + Bq
    ramp = total * np.arange(nk, dtype=np.float32) / max(1, nk - 1)
    inp.k_pre[..., 0] = bf(ramp[:P])[None, None, :]
    inp.k_blk[..., 0] = bf(ramp[P:])[None, None, :]
    return inp


def hdr_inputs(sh, q_scale: float):
    """Random queries scaled up: scores ~ N(0, q_scale^2) natural-log units."""
    inp = datagen.make_inputs(sh)
    inp.q = bf(datagen.bf16_bits_to_f32(inp.q) * np.float32(q_scale))
    return inp


def row_scaled_inputs(sh):
    """Random queries whose scale depends on the row's place in its 32-row
    block (0.25 * 2^(r % 32 / 4), up to about 54): every row of a block has its
    own dynamic range, so the per-row sums of the weights all differ, and a
    sum that reached the wrong row of its block would show."""
    inp = datagen.make_inputs(sh)
    B, Hq, Bq, d = inp.q.shape
    q = datagen.bf16_bits_to_f32(inp.q)
    G = sh.q_heads // sh.kv_heads
    packed = (np.arange(Hq) % G)[:, None] * Bq + np.arange(Bq)[None, :]  # packed row of (q-head, query)
    scale = (0.25 * 2.0 ** ((packed % 32) / 4.0)).astype(np.float32)
    inp.q = bf(q * scale[None, :, :, None])
    return inp


def run_and_compare(ba, sh, inp, splits):
    import torch
    t = {k: up(getattr(inp, k)) for k in ("q", "k_pre", "v_pre", "k_blk", "v_blk")}
    idx = up(inp.idx) if inp.idx is not None else None
    o, lse = ba.attention(t["q"], t["k_pre"], t["v_pre"], t["k_blk"], t["v_blk"], idx=idx, splits=splits)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.full(inp.q, inp.k_pre, inp.v_pre, inp.k_blk, inp.v_blk, sh.scale, idx=inp.idx)
    eo, el = max_err(down(o), o_ref), max_err(down(lse), lse_ref)
    say(f"  max err O {eo:.3e} LSE {el:.3e} (LSE range {np.nanmin(lse_ref):.1f} .. {np.nanmax(lse_ref):.1f})")
    assert eo <= TOL["bf16"]["o"] and el <= TOL["bf16"]["lse"], (eo, el)
    # the prefix partial alone, where the special key is in the prefix
    return o, lse


SHAPES = [
    dict(batch=2, q_heads=8, kv_heads=2, prefix_len=1000, block_len=32),     # 128 rows, 4 waves
    dict(batch=1, q_heads=28, kv_heads=4, prefix_len=4000, block_len=32),    # 224 rows: ping-pong kernel
    dict(batch=1, q_heads=4, kv_heads=4, prefix_len=777, block_len=32),      # MHA: one row wave + DMA wave
    dict(batch=1, q_heads=10, kv_heads=2, prefix_len=700, block_len=40),     # ragged rows, 200 per kv-head
]


@pytest.mark.parametrize("kw", SHAPES, ids=lambda kw: "-".join(f"{k}{v}" for k, v in kw.items()))
@pytest.mark.parametrize("where", ["last_prefix", "last_block", "first_prefix"])
@pytest.mark.parametrize("splits", [0, 1, 5])
def test_one_hot_maximum_arrives_late(ba, kw, where, splits):
    sh = datagen.scaled_shape("dream_gqa", outlier_frac=0.0, **kw)
    say(f"case one-hot {where} {sh} splits={splits}")
    run_and_compare(ba, sh, one_hot_inputs(sh, where), splits)


@pytest.mark.parametrize("kw", [SHAPES[1], dict(batch=1, q_heads=4, kv_heads=4, prefix_len=2500, block_len=32)],
                         ids=["pingpong", "mha"])
def test_one_hot_maximum_in_a_late_merge_chunk(ba, kw):
    # the winning key in the last of 20 splits: in the second chunk of 16
    # partials that the split merge folds
    sh = datagen.scaled_shape("dream_gqa", outlier_frac=0.0, **kw)
    say(f"case one-hot last_prefix {sh} splits=20")
    run_and_compare(ba, sh, one_hot_inputs(sh, "last_prefix"), 20)


@pytest.mark.parametrize("splits", [0, 1, 3])
def test_one_hot_maximum_in_a_retained_row(ba, splits):
    sh = datagen.scaled_shape("sparse_gqa", prefix_len=6000, n_keep=1500)
    say(f"case one-hot last kept row {sh} splits={splits}")
    run_and_compare(ba, sh, one_hot_inputs(sh, "last_kept"), splits)


@pytest.mark.parametrize("kw", SHAPES[:3], ids=lambda kw: "-".join(f"{k}{v}" for k, v in kw.items()))
@pytest.mark.parametrize("total", [40.0, 90.0, 400.0])
def test_scores_ramp_up_every_tile(ba, kw, total):
    sh = datagen.scaled_shape("dream_gqa", outlier_frac=0.0, **kw)
    say(f"case ramp total {total} {sh}")
    run_and_compare(ba, sh, ramp_inputs(sh, total), 0)


@pytest.mark.parametrize("q_scale", [6.0, 16.0])
@pytest.mark.parametrize("kw", SHAPES, ids=lambda kw: "-".join(f"{k}{v}" for k, v in kw.items()))
def test_high_dynamic_range_scores(ba, kw, q_scale):
    sh = datagen.scaled_shape("dream_gqa", **kw)
    say(f"case hdr q x{q_scale} {sh}")
    run_and_compare(ba, sh, hdr_inputs(sh, q_scale), 3)


@pytest.mark.parametrize("kw", SHAPES, ids=lambda kw: "-".join(f"{k}{v}" for k, v in kw.items()))
@pytest.mark.parametrize("splits", [0, 3])
def test_row_dependent_score_scale(ba, kw, splits):
    sh = datagen.scaled_shape("dream_gqa", **kw)
    say(f"case row-scaled q {sh} splits={splits}")
    run_and_compare(ba, sh, row_scaled_inputs(sh), splits)


def test_one_hot_full_size_metric_workload_sampled(ba):
    """The metric workload's launch configuration (16 key splits, ping-pong
    kernel) with the special key at the last prefix row."""
    import torch
    sh = datagen.WORKLOADS["dream_gqa"]
    inp = one_hot_inputs(sh, "last_prefix")
    t = {k: up(getattr(inp, k)) for k in ("q", "k_pre", "v_pre", "k_blk", "v_blk")}
    o, lse = ba.attention(t["q"], t["k_pre"], t["v_pre"], t["k_blk"], t["v_blk"])
    torch.cuda.synchronize()
    heads = [(0, 0), (1, 13), (3, 27)]
    o_ref, lse_ref = oracle.full(inp.q, inp.k_pre, inp.v_pre, inp.k_blk, inp.v_blk, sh.scale, heads=heads)
    mask = ~np.isnan(lse_ref)
    eo = max_err(down(o), o_ref, mask[..., None].repeat(o_ref.shape[-1], -1))
    el = max_err(down(lse), lse_ref, mask)
    say(f"  full-size one-hot: max err O {eo:.3e} LSE {el:.3e}")
    assert eo <= TOL["bf16"]["o"] and el <= TOL["bf16"]["lse"]


@pytest.mark.parametrize("kw", SHAPES + [dict(batch=1, q_heads=14, kv_heads=2, prefix_len=900, block_len=32,
                                              head_dim=64),
                                         # 2048 query rows: the merge's eight-values-per-thread form, d 64 and 128
                                         dict(batch=2, q_heads=32, kv_heads=4, prefix_len=600, block_len=32,
                                              head_dim=64),
                                         dict(batch=2, q_heads=32, kv_heads=4, prefix_len=600, block_len=32)],
                         ids=lambda kw: "-".join(f"{k}{v}" for k, v in kw.items()))
@pytest.mark.parametrize("v_scale", [2.0 ** 20, 2.0 ** -30])
@pytest.mark.parametrize("splits", [0, 3])
def test_value_magnitudes_outside_fp16(ba, kw, v_scale, splits):
    """V far beyond fp16's range (|V| up to ~2^23) and far below its normal
    range (~2^-30): the bf16 kernels keep split partials of o in fp16 scaled by
    a power of two per row, so O must still match the oracle to the bf16
    tolerance relative to the size of V (O scales with V, LSE does not)."""
    import torch
    sh = datagen.scaled_shape("dream_gqa", **kw)
    say(f"case value scale 2^{np.log2(v_scale):.0f} {sh} splits={splits}")
    inp = datagen.make_inputs(sh)
    inp.v_pre = bf(datagen.bf16_bits_to_f32(inp.v_pre) * np.float32(v_scale))
    inp.v_blk = bf(datagen.bf16_bits_to_f32(inp.v_blk) * np.float32(v_scale))
    t = {k: up(getattr(inp, k)) for k in ("q", "k_pre", "v_pre", "k_blk", "v_blk")}
    o, lse = ba.attention(t["q"], t["k_pre"], t["v_pre"], t["k_blk"], t["v_blk"], splits=splits)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.full(inp.q, inp.k_pre, inp.v_pre, inp.k_blk, inp.v_blk, sh.scale)
    eo = max_err(down(o) / v_scale, o_ref / v_scale)
    el = max_err(down(lse), lse_ref)
    say(f"  max err O/scale {eo:.3e} LSE {el:.3e}")
    assert np.all(np.isfinite(down(o)))
    assert eo <= TOL["bf16"]["o"] and el <= TOL["bf16"]["lse"], (eo, el)
