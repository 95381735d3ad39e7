"""Parity at the workloads' full sizes, in the launch configuration the benchmark
times (automatic split plan), on sampled (batch, q-head) pairs the fp64 oracle
evaluates one by one. Same tolerances as test_parity_gpu.py."""

import numpy as np
import pytest

import datagen
import oracle
from tests.gpu_util import TOL, bits, down, lse_of, max_err, say, up

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module")
def ba():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import cached_block_attention_amd as mod
    mod.library()
    return mod


def sample_heads(sh, n, seed):
    g = np.random.default_rng(seed)
    pairs = {(int(g.integers(sh.batch)), int(g.integers(sh.q_heads))) for _ in range(n)}
    pairs.add((sh.batch - 1, sh.q_heads - 1))
    pairs.add((0, 0))
    return sorted(pairs)


def run_full(ba, name, nsample):
    import torch
    sh = datagen.WORKLOADS[name]
    say(f"case full-size {name}: generating inputs")
    inp = datagen.make_inputs(sh)
    q, kp, vp, kb, vb = (up(getattr(inp, k)) for k in ("q", "k_pre", "v_pre", "k_blk", "v_blk"))
    idx = up(inp.idx) if inp.idx is not None else None
    say(f"  launching {name}")
    o, lse = ba.attention(q, kp, vp, kb, vb, idx=idx)
    torch.cuda.synchronize()
    heads = sample_heads(sh, nsample, 9) if nsample else None
    o_ref, lse_ref = oracle.full(inp.q, inp.k_pre, inp.v_pre, inp.k_blk, inp.v_blk, sh.scale,
                                 idx=inp.idx, heads=heads)
    mask = ~np.isnan(lse_ref)
    eo = max_err(down(o), o_ref, np.repeat(mask[..., None], o_ref.shape[-1], -1))
    el = max_err(down(lse), lse_ref, mask)
    say(f"  {name}: max err O {eo:.3e} LSE {el:.3e} over {int(mask.sum())} rows")
    assert eo <= TOL[sh.dtype]["o"] and el <= TOL[sh.dtype]["lse"]
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    return inp, (q, kp, vp, kb, vb, idx), o, lse


def test_llada_full_all_heads(ba):
    run_full(ba, "llada_bf16", 0)


def test_dream_gqa_full_sampled(ba):
    run_full(ba, "dream_gqa", 6)


def test_tiny_f32_full(ba):
    run_full(ba, "tiny_f32", 0)


def test_sparse_gqa_full_and_gather(ba):
    import torch
    inp, (q, kp, vp, kb, vb, idx), o, lse = run_full(ba, "sparse_gqa", 4)
    ko, vo = ba.gather_prefix(kp, vp, idx)
    torch.cuda.synchronize()
    assert np.array_equal(bits(ko), oracle.gather(inp.k_pre, inp.idx))
    assert np.array_equal(bits(vo), oracle.gather(inp.v_pre, inp.idx))


def test_reuse_eight_steps_sampled(ba):
    """Prefix partial once from the step-0 queries, then per step a fresh block
    partial merged with it (the cached-prefix reuse), against the oracle's
    composition of the same three steps; at step 0 it is exact full attention."""
    import torch
    sh = datagen.WORKLOADS["reuse_bf16"]
    say("case full-size reuse_bf16: generating inputs")
    inp = datagen.make_inputs(sh)
    q0, kp, vp = up(inp.q), up(inp.k_pre), up(inp.v_pre)
    pp = ba.prefix_partial(q0, kp, vp)
    torch.cuda.synchronize()
    heads = sample_heads(sh, 3, 11)
    tol = TOL["bf16"]
    ref_pp = {}
    for b, h in heads:
        ref_pp[(b, h)] = oracle.partial(inp.q[b:b + 1, h:h + 1], inp.k_pre[b:b + 1, h:h + 1],
                                        inp.v_pre[b:b + 1, h:h + 1], sh.scale)
        o, m, l = ref_pp[(b, h)]
        assert max_err(down(pp.o[b, h]), o[0, 0]) <= tol["o"]
        assert max_err(lse_of(down(pp.m[b, h]), down(pp.l[b, h])), lse_of(m, l)[0, 0]) <= tol["lse"]
    for t in range(sh.steps):
        if t == 0:
            qt_np, kb_np, vb_np = inp.q, inp.k_blk, inp.v_blk
        else:
            qt_np, kb_np, vb_np = datagen.step_inputs(sh, t)
        qt, kb, vb = up(qt_np), up(kb_np), up(vb_np)
        pb = ba.block_partial(qt, kb, vb)
        o, lse = ba.merge(pp, pb, dtype=torch.bfloat16)
        so, slse = ba.block_step(qt, kb, vb, pp)   # the same step in one launch
        torch.cuda.synchronize()
        for b, h in heads:
            rb = oracle.partial(qt_np[b:b + 1, h:h + 1], kb_np[b:b + 1, h:h + 1], vb_np[b:b + 1, h:h + 1],
                                sh.scale)
            ro, rm, rl, rlse = oracle.merge(ref_pp[(b, h)], rb)
            assert max_err(down(o[b, h]), ro[0, 0]) <= tol["o"], (t, b, h)
            assert max_err(down(lse[b, h]), rlse[0, 0]) <= tol["lse"], (t, b, h)
            assert max_err(down(so[b, h]), ro[0, 0]) <= tol["o"], (t, b, h)
            assert max_err(down(slse[b, h]), rlse[0, 0]) <= tol["lse"], (t, b, h)
            if t == 0:
                fo, fl = oracle.full(inp.q[b:b + 1, h:h + 1], inp.k_pre[b:b + 1, h:h + 1],
                                     inp.v_pre[b:b + 1, h:h + 1], inp.k_blk[b:b + 1, h:h + 1],
                                     inp.v_blk[b:b + 1, h:h + 1], sh.scale)
                assert max_err(down(o[b, h]), fo[0, 0]) <= tol["o"]
                assert max_err(down(lse[b, h]), fl[0, 0]) <= tol["lse"]
        say(f"  reuse step {t} ok")


def test_sparse_gqa_retention_from_attention_mass(ba):
    """The step that produces the retained rows at the sparse workload's full
    size: dense attention over all 131072 prefix rows and the block gives each
    row's LSE, the attention mass of every prefix row follows, and the 8192
    rows of largest mass are kept. Mass checked on sampled kv heads against the
    oracle; selection bit-exact against the oracle's rule on the same masses."""
    import torch
    sh = datagen.WORKLOADS["sparse_gqa"]
    say("case full-size sparse_gqa retention: generating inputs")
    inp = datagen.make_inputs(sh)
    q, kp, vp, kb, vb = (up(getattr(inp, k)) for k in ("q", "k_pre", "v_pre", "k_blk", "v_blk"))
    _, lse = ba.attention(q, kp, vp, kb, vb)
    mass = ba.prefix_mass(q, kp, lse)
    idx = ba.select_retained(mass, sh.n_keep)
    torch.cuda.synchronize()
    got = down(mass)
    gi = idx.cpu().numpy()
    assert np.array_equal(gi, oracle.select_retained(got, sh.n_keep))
    G = sh.q_heads // sh.kv_heads
    rows = G * sh.block_len
    for b, h in ((0, 0), (sh.batch - 1, sh.kv_heads - 1)):
        heads = [(b, h * G + g) for g in range(G)]
        _, lse_ref = oracle.full(inp.q, inp.k_pre, inp.v_pre, inp.k_blk, inp.v_blk, sh.scale, heads=heads)
        ref = oracle.prefix_mass(inp.q[b:b + 1, h * G:(h + 1) * G], inp.k_pre[b:b + 1, h:h + 1],
                                 lse_ref[b:b + 1, h * G:(h + 1) * G], sh.scale)[0, 0]
        err = np.abs(got[b, h] - ref)
        say(f"  mass (b={b}, kv head {h}): max err {err.max():.3e}, max mass {ref.max():.3e}")
        assert np.all(err <= 1e-4 * np.maximum(1.0, ref) + 1e-7 * rows)
        cut = np.sort(ref)[::-1][sh.n_keep - 1]
        assert np.all(ref[gi[b, h]] >= cut - 2 * (1e-4 * max(1.0, cut) + 1e-7 * rows))
