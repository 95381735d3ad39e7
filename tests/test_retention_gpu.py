"""Parity of attention-guided retention on the GPU (blkattn_prefix_mass and
blkattn_select_retained, through the C ABI) with the fp64 oracle.

Mass tolerance, derived from the arithmetic of one term exp(s - LSE) and the
fp32 sum of R of them (R = q-heads per kv-head x block queries):
  * the score s is a fp32 sum of d products (exact for bf16 inputs), off by at
    most d * 2^-24 * scale * sum_i |q_i k_i| (natural-log units), which is
    the relative error it gives the term;
  * the exp2 argument (|x| < 64) is rounded once and exp2 is faithful: 2e-6;
  * the fp32 sum of R positive terms: R * 2^-24 relative.
The kernel is compared against the oracle's mass at the kernel's own LSE (the
input it was given), and against the oracle's mass at the oracle's LSE with the
measured LSE difference added (a factor e^{dLSE} on every term).
Selection: bit-exact against the oracle's rule applied to the same fp32 masses;
against the oracle's own masses the kept set must equal the oracle's, except
for rows whose oracle mass lies within that tolerance band of the cut (such
rows may trade places)."""

import numpy as np
import pytest

import datagen
import oracle
from tests.gpu_util import down, say, up

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ba():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import cached_block_attention_amd as mod
    mod.library()
    return mod


def upload(inp):
    return {k: up(getattr(inp, k)) for k in ("q", "k_pre", "v_pre", "k_blk", "v_blk")}


def mass_rel_tol(inp, sh, rows):
    """Relative error bound of one mass (see the module docstring)."""
    import oracle as _o
    q = _o.widen(inp.q)
    k = _o.widen(inp.k_pre)
    G = sh.q_heads // sh.kv_heads
    smax = 0.0
    for b in range(sh.batch):
        for h in range(sh.q_heads):
            smax = max(smax, float(np.max(np.abs(q[b, h]) @ np.abs(k[b, h // G]).T)))
    return sh.head_dim * 2.0 ** -24 * sh.scale * smax + 2e-6 + rows * 2.0 ** -24


CASES = [
    ("tiny_f32", {}),
    ("dream_gqa", dict(batch=2, prefix_len=1000)),                                   # 224 rows
    ("sparse_gqa", dict(prefix_len=1500, n_keep=None)),                             # 448 rows
    ("llada_bf16", dict(q_heads=3, kv_heads=3, prefix_len=700)),                    # 32 rows
    ("dream_gqa", dict(batch=1, q_heads=6, kv_heads=2, prefix_len=333, block_len=20, head_dim=64)),
    ("dream_gqa", dict(batch=1, q_heads=16, kv_heads=1, prefix_len=200, block_len=64)),  # 1024 rows
    ("dream_gqa", dict(batch=1, q_heads=8, kv_heads=1, prefix_len=300, block_len=75)),   # 600 rows: 2 passes
    ("dream_gqa", dict(batch=1, q_heads=16, kv_heads=2, prefix_len=130, block_len=200)),  # 1600 rows: 4 passes
]


@pytest.mark.parametrize("name,kw", CASES, ids=lambda x: str(x))
def test_mass_and_selection(ba, name, kw):
    import torch
    sh = datagen.scaled_shape(name, **kw)
    say(f"case retention {sh}")
    inp = datagen.make_inputs(sh)
    t = upload(inp)
    _, lse = ba.attention(t["q"], t["k_pre"], t["v_pre"], t["k_blk"], t["v_blk"])
    mass = ba.prefix_mass(t["q"], t["k_pre"], lse)
    torch.cuda.synchronize()
    _, lse_ref = oracle.full(inp.q, inp.k_pre, inp.v_pre, inp.k_blk, inp.v_blk, sh.scale)
    lse_gpu = down(lse)
    ref_at_gpu_lse = oracle.prefix_mass(inp.q, inp.k_pre, lse_gpu, sh.scale)
    ref = oracle.prefix_mass(inp.q, inp.k_pre, lse_ref, sh.scale)
    got = down(mass)
    rows = sh.q_heads // sh.kv_heads * sh.block_len
    rel = mass_rel_tol(inp, sh, rows)
    floor = 1e-30   # terms below 2^-126 may flush to zero
    err = np.abs(got - ref_at_gpu_lse)
    rerr = float(np.max(err / np.maximum(ref_at_gpu_lse, 1e-300)))
    say(f"  mass max abs err {err.max():.3e}, max rel err {rerr:.3e} (bound {rel:.3e}; max mass {ref.max():.3e})")
    assert np.all(err <= rel * ref_at_gpu_lse + floor)
    dl = float(np.max(np.abs(lse_gpu - lse_ref)))
    rel_o = rel + 2.0 * dl          # e^{dl} - 1 <= 2 dl for dl < 1
    assert np.all(np.abs(got - ref) <= rel_o * ref + floor)
    n_keep = max(1, sh.prefix_len // 7)
    idx = ba.select_retained(mass, n_keep)
    torch.cuda.synchronize()
    gi = idx.cpu().numpy()
    assert np.array_equal(gi, oracle.select_retained(got, n_keep))
    # against the oracle's own masses: the kept set is the oracle's, except for
    # rows inside the tolerance band of the cut
    ki = oracle.select_retained(ref, n_keep)
    for b in range(sh.batch):
        for h in range(sh.kv_heads):
            cut = np.sort(ref[b, h])[::-1][n_keep - 1]
            band = 2.0 * rel_o * cut + floor
            diff = np.setxor1d(gi[b, h], ki[b, h])
            assert np.all(np.abs(ref[b, h, diff] - cut) <= band), (b, h, diff[:8])
    # the kept rows feed the gathered attention
    o, lse2 = ba.attention(t["q"], t["k_pre"], t["v_pre"], t["k_blk"], t["v_blk"], idx=idx)
    torch.cuda.synchronize()
    o_ref, lse2_ref = oracle.full(inp.q, inp.k_pre, inp.v_pre, inp.k_blk, inp.v_blk, sh.scale, idx=gi)
    from tests.gpu_util import TOL, max_err
    assert max_err(down(o), o_ref) <= TOL[sh.dtype]["o"] and max_err(down(lse2), lse2_ref) <= TOL[sh.dtype]["lse"]


def test_selection_ties_and_edges(ba):
    import torch
    rng = np.random.default_rng(5)
    P = 5000
    m = rng.integers(0, 40, size=(2, 3, P)).astype(np.float32)   # heavy ties
    m[1, 2] = 0.25                                                # all equal
    m[0, 1, ::2] = 1e-30                                          # tiny values
    m[1, 0, 7::11] = -0.0                                         # -0 ranks as 0
    m[1, 0, 3::13] = 0.0
    mt = torch.from_numpy(m).cuda()
    for k in (1, 2, 777, P - 1, P):
        idx = ba.select_retained(mt, k)
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), oracle.select_retained(m.astype(np.float64), k)), k
    # a large row count crossing many threads' chunks
    big = rng.random((1, 1, 131072)).astype(np.float32)
    big[0, 0, 1000:1100] = big[0, 0, 5]
    bt = torch.from_numpy(big).cuda()
    idx = ba.select_retained(bt, 8192)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), oracle.select_retained(big.astype(np.float64), 8192))


@pytest.mark.parametrize("groups,P,k", [(8, 131072, 8192), (3, 70001, 33333), (1, 1023, 500), (5, 300, 7),
                                         (2, 300007, 20000), (1, 262145, 65536)])
def test_selection_ties_across_chunks(ba, groups, P, k):
    """Rows equal to the k-th largest mass spread over every workgroup's chunk,
    so the lower-index tie rule is decided across chunk boundaries; the rows
    are not a multiple of the chunk or of a workgroup (the last two cases: more
    than 2^18 rows per group, 32 chunks of more than 8192 rows each)."""
    import torch
    rng = np.random.default_rng(groups * 1000 + k)
    m = np.full((1, groups, P), 0.5, dtype=np.float32)
    cols = rng.integers(0, P, size=P // 7)
    m[0][:, cols] = rng.random(P // 7).astype(np.float32)[None, :]
    m[0, 0, rng.integers(0, P, size=k // 3)] = 2.0                 # a set certainly above the ties
    mt = torch.from_numpy(m).cuda()
    dims = ba.Dims(1, groups, groups, 64, 1, k, P, ba.F32, 1.0, 0, 0)
    ws = torch.empty(ba.workspace_bytes(dims, ba.OP_SELECT), dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)                                                   # stale workspace contents are ignored
    idx = torch.empty(1, groups, k, dtype=torch.int32, device="cuda")
    ba.blkattn_select_retained(mt, idx, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), oracle.select_retained(m.astype(np.float64), k))


def test_mass_is_deterministic(ba):
    import torch
    sh = datagen.scaled_shape("dream_gqa", batch=1, prefix_len=3000)
    inp = datagen.make_inputs(sh)
    t = upload(inp)
    _, lse = ba.attention(t["q"], t["k_pre"], t["v_pre"], t["k_blk"], t["v_blk"])
    m1 = ba.prefix_mass(t["q"], t["k_pre"], lse)
    m2 = ba.prefix_mass(t["q"], t["k_pre"], lse)
    torch.cuda.synchronize()
    assert torch.equal(m1, m2)
