"""Guard canaries: every output of every entry point is a window into a larger
buffer whose other bytes hold a sentinel bit pattern (a NaN payload for
floats), and strided outputs are given padded rows. After each call the
sentinels must be bit-for-bit intact, so a write outside the output (from the
row map, the packed-row chunks, the key-split workspace layout or a ragged
tail) fails the test. The results inside the windows are checked against the
fp64 oracle as in the parity tests.
"""

import numpy as np
import pytest

import datagen
import oracle
from tests.gpu_util import TOL, bits, down, lse_of, max_err, say, up

pytestmark = pytest.mark.gpu

BORDER = 4096  # sentinel elements before and after every window
SENTINEL = {"float32": 0x7FC0DEAD, "bfloat16": 0x7FC1, "int32": 0x5A5A5A5A}


@pytest.fixture(scope="module")
def ba():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import cached_block_attention_amd as mod
    mod.library()
    return mod


class Guarded:
    """A contiguous window of `shape` inside a sentinel-filled buffer, or (pad)
    a strided [..., T, d] window whose rows are padded by `pad` elements."""

    def __init__(self, shape, dtype, pad=0):
        import torch
        self.torch = torch
        self.dtype = dtype
        name = str(dtype).replace("torch.", "")
        self.name = name
        inner = list(shape)
        if pad:
            inner[-1] += pad
        n = int(np.prod(inner))
        ibits = {"float32": torch.int32, "bfloat16": torch.int16, "int32": torch.int32}[name]
        self.buf = torch.empty(n + 2 * BORDER, dtype=dtype, device="cuda")
        s = SENTINEL[name]
        if ibits == torch.int16:
            s = s - 0x10000 if s >= 0x8000 else s
        else:
            s = s - 0x100000000 if s >= 0x80000000 else s
        self.buf.view(ibits).fill_(s)
        self.ibits = ibits
        self.sentinel = s
        self.inner = inner
        win = self.buf[BORDER:BORDER + n].view(*inner)
        self.t = win[..., :shape[-1]] if pad else win
        self.pad = pad

    def check(self, what):
        self.torch.cuda.synchronize()
        v = self.buf.view(self.ibits)
        n = int(np.prod(self.inner))
        ok = bool((v[:BORDER] == self.sentinel).all()) and bool((v[BORDER + n:] == self.sentinel).all())
        if self.pad:
            gaps = v[BORDER:BORDER + n].view(*self.inner)[..., self.inner[-1] - self.pad:]
            ok = ok and bool((gaps == self.sentinel).all())
        assert ok, f"{what}: a write landed outside the output"


def g_partial(B, Hq, rows, d):
    import torch
    import cached_block_attention_amd as mod
    go, gm, gl = Guarded((B, Hq, rows, d), torch.float32), Guarded((B, Hq, rows), torch.float32), \
        Guarded((B, Hq, rows), torch.float32)
    return (go, gm, gl), mod.Partial(go.t, gm.t, gl.t)


def check_all(gs, what):
    for g in gs:
        g.check(what)


CASES = [
    ("dream_gqa", dict(batch=2, q_heads=28, kv_heads=4, prefix_len=1100, block_len=32), 0),   # ping-pong, splits
    ("dream_gqa", dict(batch=1, q_heads=10, kv_heads=2, prefix_len=700, block_len=40), 3),    # ragged 200 rows
    ("llada_bf16", dict(q_heads=3, kv_heads=3, prefix_len=900), 0),                           # MHA + DMA wave
    ("dream_gqa", dict(batch=1, q_heads=14, kv_heads=2, prefix_len=500, block_len=64), 2),    # 448 rows: 2 chunks
    ("dream_gqa", dict(batch=1, q_heads=6, kv_heads=2, prefix_len=333, block_len=20, head_dim=64), 0),
    ("tiny_f32", {}, 2),
    ("sparse_gqa", dict(prefix_len=3000, n_keep=700), 0),
]


@pytest.mark.parametrize("name,kw,splits", CASES, ids=lambda x: str(x))
def test_attention_outputs_stay_in_bounds(ba, name, kw, splits):
    import torch
    sh = datagen.scaled_shape(name, **kw)
    say(f"case guards {sh} splits={splits}")
    inp = datagen.make_inputs(sh)
    t = {k: up(getattr(inp, k)) for k in ("q", "k_pre", "v_pre", "k_blk", "v_blk")}
    idx = up(inp.idx) if inp.idx is not None else None
    B, Hq, Bq, d = inp.q.shape
    dt = t["q"].dtype
    tol = TOL[sh.dtype]
    o_ref, lse_ref = oracle.full(inp.q, inp.k_pre, inp.v_pre, inp.k_blk, inp.v_blk, sh.scale, idx=inp.idx)

    # full: padded O rows, bordered LSE
    go, gl = Guarded((B, Hq, Bq, d), dt, pad=16), Guarded((B, Hq, Bq), torch.float32)
    ba.blkattn_full(t["q"], t["k_pre"], t["v_pre"], t["k_blk"], t["v_blk"], go.t, gl.t, idx=idx, splits=splits)
    check_all((go, gl), "blkattn_full")
    assert max_err(down(go.t), o_ref) <= tol["o"] and max_err(down(gl.t), lse_ref) <= tol["lse"]

    # prefix partial and block partial
    gpp, pp = g_partial(B, Hq, Bq, d)
    ba.blkattn_prefix_partial(t["q"], t["k_pre"], t["v_pre"], pp, idx=idx, splits=splits)
    check_all(gpp, "blkattn_prefix_partial")
    gpb, pb = g_partial(B, Hq, Bq, d)
    ba.blkattn_block_partial(t["q"], t["k_blk"], t["v_blk"], pb)
    check_all(gpb, "blkattn_block_partial")
    ro, rm, rl = oracle.partial(inp.q, inp.k_pre, inp.v_pre, sh.scale, idx=inp.idx)
    assert max_err(down(pp.o), ro) <= tol["o"]
    assert max_err(lse_of(down(pp.m), down(pp.l)), lse_of(rm, rl)) <= tol["lse"]

    # merge into padded O, bordered LSE and a bordered merged partial
    go2, gl2 = Guarded((B, Hq, Bq, d), dt, pad=8), Guarded((B, Hq, Bq), torch.float32)
    gab, ab = g_partial(B, Hq, Bq, d)
    ba.blkattn_merge(pp, pb, o=go2.t, lse=gl2.t, ab=ab)
    check_all((go2, gl2, *gab), "blkattn_merge")
    assert max_err(down(go2.t), o_ref) <= tol["o"] and max_err(down(gl2.t), lse_ref) <= tol["lse"]

    # block step into padded O
    go3, gl3 = Guarded((B, Hq, Bq, d), dt, pad=8), Guarded((B, Hq, Bq), torch.float32)
    ba.blkattn_block_step(t["q"], t["k_blk"], t["v_blk"], pp, go3.t, gl3.t)
    check_all((go3, gl3), "blkattn_block_step")
    assert max_err(down(go3.t), o_ref) <= tol["o"] and max_err(down(gl3.t), lse_ref) <= tol["lse"]

    if idx is not None:
        nk = inp.idx.shape[-1]
        gk, gv = Guarded((B, sh.kv_heads, nk, d), dt, pad=8), Guarded((B, sh.kv_heads, nk, d), dt)
        ba.blkattn_gather_prefix(t["k_pre"], t["v_pre"], idx, gk.t, gv.t)
        check_all((gk, gv), "blkattn_gather_prefix")
        assert np.array_equal(bits(gk.t.contiguous()), oracle.gather(inp.k_pre, inp.idx))
        assert np.array_equal(bits(gv.t), oracle.gather(inp.v_pre, inp.idx))


def test_sequence_step_outputs_stay_in_bounds(ba):
    import torch
    sh = datagen.scaled_shape("llada_seq", q_heads=4, kv_heads=2, prefix_len=700, block_len=32, block_start=300)
    q_np, k_np, v_np = datagen.sequence_inputs(sh, 0)
    q, k, v = up(q_np), up(k_np), up(v_np)
    B, Hq, N, d = q_np.shape
    gcache, cache = g_partial(B, Hq, N, d)
    go, gl = Guarded((B, Hq, N, d), torch.bfloat16, pad=8), Guarded((B, Hq, N), torch.float32)
    for gen in (True, False):
        ba.blkattn_sequence_step(q, k, v, sh.block_start, sh.block_len, cache, gen, go.t, gl.t, splits=3)
        check_all((go, gl), f"blkattn_sequence_step gen={gen}")
    # the cache's block rows are never written: still the sentinel
    c0, c1 = sh.block_start, sh.block_start + sh.block_len
    cm = gcache[1].buf.view(torch.int32)[BORDER:BORDER + B * Hq * N].view(B, Hq, N)
    assert bool((cm[:, :, c0:c1] == gcache[1].sentinel).all())
    check_all(gcache, "sequence cache")
    o_ref, lse_ref = oracle.sequence_full(q_np, k_np, v_np, sh.scale)
    assert max_err(down(go.t), o_ref) <= TOL["bf16"]["o"] and max_err(down(gl.t), lse_ref) <= TOL["bf16"]["lse"]


@pytest.mark.parametrize("kw", [dict(batch=2, prefix_len=1000), dict(batch=1, q_heads=16, kv_heads=2,
                                                                     prefix_len=300, block_len=75)])
def test_mass_and_selection_stay_in_bounds(ba, kw):
    import torch
    sh = datagen.scaled_shape("dream_gqa", **kw)
    inp = datagen.make_inputs(sh)
    t = {k: up(getattr(inp, k)) for k in ("q", "k_pre", "v_pre", "k_blk", "v_blk")}
    _, lse = ba.attention(t["q"], t["k_pre"], t["v_pre"], t["k_blk"], t["v_blk"])
    gm = Guarded((sh.batch, sh.kv_heads, sh.prefix_len), torch.float32)
    ba.blkattn_prefix_mass(t["q"], t["k_pre"], lse, gm.t)
    gm.check("blkattn_prefix_mass")
    n_keep = sh.prefix_len // 5
    gi = Guarded((sh.batch, sh.kv_heads, n_keep), torch.int32)
    ba.blkattn_select_retained(gm.t, gi.t)
    gi.check("blkattn_select_retained")
    assert np.array_equal(gi.t.cpu().numpy(), oracle.select_retained(down(gm.t), n_keep))
