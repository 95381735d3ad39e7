"""Large blocks (FlashBlock abstract: block diffusion also generates video,
with blocks of hundreds of tokens): the block partial becomes a square,
bidirectional tile and the packed (q-head, query) rows of one kv head span
several workgroups. Parity with the fp64 oracle at the tolerances of
test_parity_gpu.py, including ragged row and key tails."""

import numpy as np
import pytest

import datagen
import oracle
from tests.gpu_util import TOL, down, lse_of, max_err, say, up

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ba():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import cached_block_attention_amd as mod
    mod.library()
    return mod


@pytest.mark.parametrize("kw", [
    dict(q_heads=4, kv_heads=4, block_len=256),
    dict(q_heads=8, kv_heads=2, block_len=300),                  # 1200 packed rows per kv head
    dict(q_heads=2, kv_heads=1, head_dim=64, block_len=1000),
    dict(batch=2, q_heads=2, kv_heads=2, block_len=1024),
    # 32 heads: enough 224-row chunks for the ping-pong kernel (five per head,
    # the last one with 128 or 104 rows and idle row waves)
    dict(q_heads=32, kv_heads=32, block_len=1024),
    dict(q_heads=32, kv_heads=32, block_len=1000),
])
def test_block_partial_large(ba, kw):
    import torch
    sh = datagen.scaled_shape("llada_bf16", prefix_len=0, batch=kw.pop("batch", 1), **kw)
    say(f"case large block partial {sh}")
    inp = datagen.make_inputs(sh)
    q, kb, vb = up(inp.q), up(inp.k_blk), up(inp.v_blk)
    pb = ba.block_partial(q, kb, vb)
    torch.cuda.synchronize()
    o, m, l = oracle.partial(inp.q, inp.k_blk, inp.v_blk, sh.scale)
    tol = TOL["bf16"]
    eo = max_err(down(pb.o), o)
    el = max_err(lse_of(down(pb.m), down(pb.l)), lse_of(m, l))
    say(f"  max err o {eo:.3e} lse {el:.3e}")
    assert eo <= tol["o"] and el <= tol["lse"]


@pytest.mark.parametrize("kw,splits", [
    (dict(q_heads=4, kv_heads=4, block_len=512, prefix_len=1000), 0),
    (dict(q_heads=14, kv_heads=2, block_len=200, prefix_len=777), 3),
    (dict(dtype=datagen.F32, head_dim=64, q_heads=2, kv_heads=2, block_len=300, prefix_len=250), 2),
    # 7 q-heads x 256 queries = 1792 packed rows per kv head over 4256 keys: eight 224-row
    # ping-pong chunks x 8 key splits (256 workgroups), merged from fp16 partials
    (dict(q_heads=28, kv_heads=4, block_len=256, prefix_len=4000), 0),
])
def test_full_with_large_block(ba, kw, splits):
    import torch
    sh = datagen.scaled_shape("llada_bf16", **kw)
    say(f"case large block full {sh} splits={splits}")
    inp = datagen.make_inputs(sh)
    o, lse = ba.attention(up(inp.q), up(inp.k_pre), up(inp.v_pre), up(inp.k_blk), up(inp.v_blk), splits=splits)
    torch.cuda.synchronize()
    ro, rl = oracle.full(inp.q, inp.k_pre, inp.v_pre, inp.k_blk, inp.v_blk, sh.scale)
    tol = TOL[sh.dtype]
    eo, el = max_err(down(o), ro), max_err(down(lse), rl)
    say(f"  max err O {eo:.3e} LSE {el:.3e}")
    assert eo <= tol["o"] and el <= tol["lse"]
