"""blkattn_full_noalloc (the entry point for callers that cannot allocate):
through the C ABI, two calls in a row on one stream, the second smaller, each
bit-identical to blkattn_full with a caller workspace (the same kernels and
split plan) and within the bf16 tolerance of the fp64 oracle; a call whose
scratch need exceeds the static array is refused with a clear error."""

import numpy as np
import pytest

import datagen
import oracle
from tests.gpu_util import TOL, bits, down, max_err, say, up

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ba():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import cached_block_attention_amd as mod
    mod.library()
    return mod


def _run_pair(ba, sh, splits=0):
    import torch
    inp = datagen.make_inputs(sh)
    t = {k: up(getattr(inp, k)) for k in ("q", "k_pre", "v_pre", "k_blk", "v_blk")}
    idx = up(inp.idx) if inp.idx is not None else None
    B, Hq, Bq, d = inp.q.shape
    o1 = torch.empty_like(t["q"])
    l1 = torch.empty(B, Hq, Bq, dtype=torch.float32, device="cuda")
    o2 = torch.empty_like(t["q"])
    l2 = torch.empty_like(l1)
    ba.blkattn_full_noalloc(t["q"], t["k_pre"], t["v_pre"], t["k_blk"], t["v_blk"], o1, l1, idx=idx, splits=splits)
    ba.blkattn_full(t["q"], t["k_pre"], t["v_pre"], t["k_blk"], t["v_blk"], o2, l2, idx=idx, splits=splits)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o1), bits(o2)) and np.array_equal(bits(l1), bits(l2))
    o_ref, lse_ref = oracle.full(inp.q, inp.k_pre, inp.v_pre, inp.k_blk, inp.v_blk, sh.scale, idx=inp.idx)
    eo, el = max_err(down(o1), o_ref), max_err(down(l1), lse_ref)
    say(f"  noalloc {sh.name} B{sh.batch} Hq{sh.q_heads} P{sh.prefix_len}: err O {eo:.3e} LSE {el:.3e}")
    assert eo <= TOL[sh.dtype]["o"] and el <= TOL[sh.dtype]["lse"]


def test_two_calls_second_smaller(ba):
    _run_pair(ba, datagen.scaled_shape("dream_gqa", batch=2, prefix_len=6000), splits=0)
    _run_pair(ba, datagen.scaled_shape("dream_gqa", batch=1, q_heads=8, kv_heads=2, prefix_len=700), splits=3)


def test_metric_workload_then_a_small_one(ba):
    _run_pair(ba, datagen.WORKLOADS["dream_gqa"])     # 16 key splits: 30 MB of scratch
    _run_pair(ba, datagen.scaled_shape("sparse_gqa", prefix_len=3000, n_keep=500), splits=2)


def test_too_large_is_refused(ba):
    import torch
    sh = datagen.scaled_shape("dream_gqa", batch=1, q_heads=28, kv_heads=4, prefix_len=4096, block_len=512)
    q = torch.zeros(1, 28, 512, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 4, 4096, 128, dtype=torch.bfloat16, device="cuda")
    kb = torch.zeros(1, 4, 512, 128, dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    dims = ba.make_dims(q, 4, 4096, 0, None, 60)
    need = ba.workspace_bytes(dims, ba.OP_FULL)
    assert need > 64 << 20, need
    with pytest.raises(ba.BlkAttnError, match="scratch"):
        ba.blkattn_full_noalloc(q, k, k, kb, kb, o, splits=60)
