"""Parity of blkattn_sequence_step (through the C ABI) with the fp64 oracle.

The step is LaCache's first-layer attention over the whole sequence with
FACache: at the block's first step the cache of the other rows' queries over
the other rows' keys is built, at later steps it is reused and only the
block's keys are streamed for those queries. Since only the block's rows change
between steps, every step must equal plain attention over the current sequence
(oracle.sequence_full); the cache itself is checked against the oracle's
procedure (oracle.facache_step). Same tolerances as test_parity_gpu.py.
"""

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


def sentinel_cache(ba, B, Hq, N, d):
    c = ba.empty_partial(B, Hq, N, d, "cuda")
    for x in c:
        x.fill_(7.0)
    return c


def run_steps(ba, sh, steps, splits=0, heads=None):
    import torch
    B, Hq, N, d = sh.batch, sh.q_heads, sh.prefix_len, sh.head_dim
    c0, Bq = sh.block_start, sh.block_len
    u, c = oracle.split_rows(N, c0, Bq)
    tol = TOL[sh.dtype]
    cache = sentinel_cache(ba, B, Hq, N, d)
    ref_cache = None
    for t in range(steps):
        say(f"case sequence {sh.name} N={N} block=[{c0},{c0 + Bq}) Hq={Hq}/{sh.kv_heads} d={d} "
            f"{sh.dtype} splits={splits} step {t}")
        q, k, v = datagen.sequence_inputs(sh, t)
        tq, tk, tv = up(q), up(k), up(v)
        o = torch.empty_like(tq)
        lse = torch.full((B, Hq, N), float("nan"), dtype=torch.float32, device="cuda")
        ba.blkattn_sequence_step(tq, tk, tv, c0, Bq, cache, t == 0, o, lse, splits=splits)
        torch.cuda.synchronize()
        ro, rl = oracle.sequence_full(q, k, v, sh.scale, heads=heads)
        mask = ~np.isnan(rl)
        eo = max_err(down(o), ro, np.repeat(mask[..., None], d, -1))
        el = max_err(down(lse), rl, mask)
        say(f"  step {t}: max err O {eo:.3e} LSE {el:.3e}")
        assert eo <= tol["o"] and el <= tol["lse"], (t, eo, el)
        if t == 0:
            # the cache: U rows hold the oracle's partial of U queries over U keys,
            # the block rows are left as they were
            if heads is None and len(u):
                _, _, ref_cache = oracle.facache_step(q, k, v, c0, Bq, sh.scale)
                co, cm, cl = (down(x) for x in cache)
                assert max_err(co[:, :, u], ref_cache[0][:, :, u]) <= tol["o"]
                assert max_err(lse_of(cm[:, :, u], cl[:, :, u]),
                               lse_of(ref_cache[1][:, :, u], ref_cache[2][:, :, u])) <= tol["lse"]
            co = down(cache.o)
            assert np.all(co[:, :, c] == 7.0) and np.all(down(cache.m)[:, :, c] == 7.0)


CASES = [
    dict(dtype=datagen.F32, head_dim=64, q_heads=4, kv_heads=4, prefix_len=300, block_start=100),
    dict(q_heads=8, kv_heads=2, prefix_len=517, block_start=0),                    # block first, GQA
    dict(batch=2, q_heads=8, kv_heads=2, prefix_len=517, block_start=517 - 32),    # block last
    dict(q_heads=4, kv_heads=4, head_dim=64, prefix_len=700, block_start=333, block_len=20),
    dict(q_heads=14, kv_heads=2, prefix_len=1100, block_start=640, block_len=64),  # G*rows > 256
    dict(q_heads=2, kv_heads=2, prefix_len=64, block_start=0, block_len=64),       # no rows outside
]


@pytest.mark.parametrize("kw", CASES)
@pytest.mark.parametrize("splits", [0, 3])
def test_sequence_steps_equal_full_attention(ba, kw, splits):
    sh = datagen.scaled_shape("llada_seq", batch=kw.pop("batch", 1), **kw)
    run_steps(ba, sh, 3, splits=splits)


def test_sequence_rejects_bad_blocks(ba):
    import torch
    sh = datagen.scaled_shape("llada_seq", q_heads=2, kv_heads=2, prefix_len=100, block_start=10)
    q = torch.zeros(1, 2, 100, 128, dtype=torch.bfloat16, device="cuda")
    cache = ba.empty_partial(1, 2, 100, 128, "cuda")
    o = torch.empty_like(q)
    for c0, bq in ((-1, 32), (69, 32), (0, 101), (0, 0)):
        with pytest.raises(ba.BlkAttnError):
            ba.blkattn_sequence_step(q, q, q, c0, bq, cache, True, o)


@pytest.mark.slow
def test_llada_sequence_full_size_sampled(ba):
    """The 4096-row sequence of the workload in the benchmark's launch
    configuration, two steps, on sampled heads."""
    sh = datagen.WORKLOADS["llada_seq"]
    run_steps(ba, sh, 2, heads=[(0, 0), (0, 13), (0, 31)])
