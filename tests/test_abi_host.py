"""Host-side checks of libblkattn.so: it loads, exports every symbol the
header declares, and rejects bad arguments before touching the GPU."""

import ctypes
import os
import re

import pytest

import cached_block_attention_amd as ba

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_symbols():
    txt = open(os.path.join(ROOT, "include", "blkattn.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(blkattn_[a-z_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ba.LIB_PATH):
        pytest.skip("libblkattn.so not built")
    return ba.library()


def test_exports_every_declared_symbol(lib):
    syms = header_symbols()
    assert len(syms) == 16, syms
    for s in syms:
        assert hasattr(lib, s), s


def test_version_and_strings(lib):
    assert lib.blkattn_abi_version() == 1
    assert lib.blkattn_strerror(ba.ERR_WORKSPACE) == b"workspace missing or too small"
    assert lib.blkattn_strerror(12345) == b"unknown status"


def dims(**kw):
    base = dict(batch=4, q_heads=28, kv_heads=4, head_dim=128, block_len=32, n_keep=0,
                prefix_len=32768, dtype=ba.BF16, scale=0.08838834764831845, splits=0, reserved=0)
    base.update(kw)
    return ba.Dims(**base)


def call_full(lib, d, **ptrs):
    t = ba.Tensor(ptrs.get("data", 4096), 128 * 32, 128 * 32, 128)
    tp = ba.Tensor(ptrs.get("data", 4096), 128 * 32768, 128 * 32768, 128)
    return lib.blkattn_full(ctypes.byref(d), ctypes.byref(t), ctypes.byref(tp), ctypes.byref(tp),
                            ptrs.get("idx"), ctypes.byref(t), ctypes.byref(t), ctypes.byref(t),
                            None, ptrs.get("ws"), ptrs.get("ws_bytes", 0), None)


@pytest.mark.parametrize("kw,status", [
    (dict(q_heads=28, kv_heads=5), ba.ERR_INVALID_ARG),
    (dict(kv_heads=0), ba.ERR_INVALID_ARG),
    (dict(batch=-1), ba.ERR_INVALID_ARG),
    (dict(head_dim=96), ba.ERR_UNSUPPORTED),
    (dict(dtype=7), ba.ERR_UNSUPPORTED),
    (dict(scale=0.0), ba.ERR_INVALID_ARG),
    (dict(scale=float("inf")), ba.ERR_INVALID_ARG),
    (dict(reserved=1), ba.ERR_INVALID_ARG),
    (dict(n_keep=5), ba.ERR_INVALID_ARG),      # n_keep set without indices
])
def test_bad_dims_rejected(lib, kw, status):
    assert call_full(lib, dims(**kw)) == status
    assert lib.blkattn_last_error() != b""


def test_workspace_and_alignment_rejected(lib):
    d = dims()
    need = lib.blkattn_workspace_bytes(ctypes.byref(d), ba.OP_FULL)
    assert need > 0
    assert call_full(lib, d) == ba.ERR_WORKSPACE                        # none given
    assert call_full(lib, d, ws=4096, ws_bytes=need - 1) == ba.ERR_WORKSPACE
    assert call_full(lib, d, data=4100, ws=4096, ws_bytes=need) == ba.ERR_MISALIGNED


def test_degenerate_sizes_are_noops(lib):
    for kw in (dict(batch=0), dict(q_heads=0), dict(block_len=0)):
        d = dims(**kw)
        assert lib.blkattn_full(ctypes.byref(d), None, None, None, None, None, None, None, None,
                                None, 0, None) == ba.OK


def test_block_step_rejects_before_launch(lib):
    d = dims()
    t = ba.Tensor(4096, 128 * 32, 128 * 32, 128)
    good = ba.PartialDesc(8192, 4096, 4096)

    def call(cached, o=t, lse=None, dd=d):
        return lib.blkattn_block_step(ctypes.byref(dd), ctypes.byref(t), ctypes.byref(t), ctypes.byref(t),
                                      None if cached is None else ctypes.byref(cached),
                                      None if o is None else ctypes.byref(o), lse, None)
    assert call(None) == ba.ERR_INVALID_ARG                                   # no cached partial
    assert call(ba.PartialDesc(8192, None, 4096)) == ba.ERR_INVALID_ARG        # cached.m missing
    assert call(ba.PartialDesc(8200, 4096, 4096)) == ba.ERR_MISALIGNED         # cached.o not 16 B aligned
    assert call(good, o=None) == ba.ERR_INVALID_ARG                          # no output
    assert call(good, lse=4098) == ba.ERR_MISALIGNED
    assert call(good, dd=dims(head_dim=80)) == ba.ERR_UNSUPPORTED
    assert call(None, o=None, dd=dims(block_len=0)) == ba.OK                   # empty block: no-op


def test_split_plan_is_a_function_of_dims(lib):
    # the metric workload: 16 (batch, kv-head) groups x 16 key splits = one
    # 8-wave workgroup per compute unit, ~32 tiles of 64 keys each
    d = dims()
    assert lib.blkattn_plan_splits(ctypes.byref(d), ba.OP_FULL) == 16
    rows = 4 * 28 * 32
    # bf16: fp16 o plus a 16-byte {m, l, inverse o scale} record per (split, row)
    assert lib.blkattn_workspace_bytes(ctypes.byref(d), ba.OP_FULL) >= 16 * rows * (128 * 2 + 16)
    d1 = dims(splits=1)
    assert lib.blkattn_plan_splits(ctypes.byref(d1), ba.OP_FULL) == 1
    assert lib.blkattn_workspace_bytes(ctypes.byref(d1), ba.OP_FULL) == 0
    # fp32: 4 (batch, q-head) workgroups per split, so its 32-key tiles are
    # spread one per split at this size ((256 + 32) / 32 = 9)
    tiny = dims(batch=1, q_heads=4, kv_heads=4, head_dim=64, prefix_len=256, dtype=ba.F32)
    assert lib.blkattn_plan_splits(ctypes.byref(tiny), ba.OP_FULL) == 9
    tiny1 = dims(batch=1, q_heads=4, kv_heads=4, head_dim=64, prefix_len=256, dtype=ba.F32, splits=2)
    assert lib.blkattn_plan_splits(ctypes.byref(tiny1), ba.OP_FULL) == 2
    huge = dims(splits=100000)
    assert lib.blkattn_plan_splits(ctypes.byref(huge), ba.OP_FULL) == (32768 + 32 + 63) // 64
    # more packed rows than one ping-pong workgroup over a long key range, in one round:
    # 1792 rows per kv head (7 x 256) go in eight 224-row chunks, and 8 key splits fill the
    # 256 compute units (256-row chunks of the sequential kernel would take 10 splits)
    big_block = dims(batch=1, block_len=256, prefix_len=4000)
    assert lib.blkattn_plan_splits(ctypes.byref(big_block), ba.OP_FULL) == 8
    # an indexed prefix stages at most 2048 indices per split
    sparse = dims(batch=2, prefix_len=131072, n_keep=100000, block_len=64, splits=1)
    assert lib.blkattn_plan_splits(ctypes.byref(sparse), ba.OP_FULL) >= (100000 + 64) // 2048


def test_select_plan_and_workspace(lib):
    d = dims(batch=2, kv_heads=4, q_heads=4, n_keep=8192, prefix_len=131072, dtype=ba.F32)
    chunks = lib.blkattn_plan_splits(ctypes.byref(d), ba.OP_SELECT)
    assert 1 <= chunks <= 32 and 8 * chunks >= 256          # the row is spread over the chip
    need = lib.blkattn_workspace_bytes(ctypes.byref(d), ba.OP_SELECT)
    assert need >= 8 * chunks * 4 * 256 * 4                   # per-chunk histograms of four passes
    small = dims(batch=1, kv_heads=1, q_heads=1, n_keep=3, prefix_len=100, dtype=ba.F32)
    assert lib.blkattn_plan_splits(ctypes.byref(small), ba.OP_SELECT) == 1

    def sel(dd, ws=None, nbytes=0):
        return lib.blkattn_select_retained(ctypes.byref(dd), 4096, 8192, ws, nbytes, None)
    assert sel(d) == ba.ERR_WORKSPACE
    assert sel(d, 4096, need - 1) == ba.ERR_WORKSPACE
    assert sel(d, 4104, need) == ba.ERR_MISALIGNED
    assert sel(dims(n_keep=10, prefix_len=9)) == ba.ERR_INVALID_ARG
    assert sel(dims(batch=0, n_keep=10)) == ba.OK


def test_sequence_step_rejects_before_launch(lib):
    d = dims(q_heads=4, kv_heads=4, prefix_len=1000, block_len=32)
    t = ba.Tensor(4096, 128 * 1000, 128 * 1000, 128)
    cache = ba.PartialDesc(8192, 4096, 4096)

    def call(c0, dd=d, gen=1, c=cache, ws=None, nbytes=0):
        return lib.blkattn_sequence_step(ctypes.byref(dd), c0, gen, ctypes.byref(t), ctypes.byref(t),
                                         ctypes.byref(t), None if c is None else ctypes.byref(c), ctypes.byref(t),
                                         None, ws, nbytes, None)
    assert call(-1) == ba.ERR_INVALID_ARG
    assert call(1000 - 31) == ba.ERR_INVALID_ARG                 # block past the end
    assert call(0, dd=dims(q_heads=4, kv_heads=4, prefix_len=1000, block_len=0)) == ba.ERR_INVALID_ARG
    assert call(0, dd=dims(q_heads=4, kv_heads=4, prefix_len=1000, n_keep=5)) == ba.ERR_INVALID_ARG
    assert call(0, c=None) == ba.ERR_INVALID_ARG                 # rows outside the block need a cache
    assert call(0, c=ba.PartialDesc(8200, 4096, 4096)) == ba.ERR_MISALIGNED
    need = lib.blkattn_workspace_bytes(ctypes.byref(d), ba.OP_SEQUENCE)
    if need:
        assert call(500) == ba.ERR_WORKSPACE
    assert call(0, dd=dims(batch=0, prefix_len=1000)) == ba.OK    # empty batch: no-op
    # the plan: the block's queries over all 1000 keys fill the chip with key splits
    assert lib.blkattn_plan_splits(ctypes.byref(d), ba.OP_SEQUENCE) >= 1
    assert lib.blkattn_plan_splits(ctypes.byref(dims(prefix_len=10, block_len=32)), ba.OP_SEQUENCE) < 0


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 1, 32, 64)
    with pytest.raises(ValueError):
        ba.attention(q, q, q, q, q)


def _cpu(*shape, dtype=None):
    torch = pytest.importorskip("torch")
    return torch.zeros(*shape, dtype=dtype or torch.bfloat16)


@pytest.mark.parametrize("bad,who", [
    (dict(o=("f32",)), "o"),                         # fp32 O for bf16 inputs: the kernel would write bf16 offsets
    (dict(k_blk=(1, 2, 16, 128)), "k_blk"),          # fewer block rows than queries
    (dict(v_pre=(1, 2, 300, 64)), "v_pre"),          # head_dim disagrees
    (dict(k_pre=(1, 3, 300, 128), v_pre=(1, 3, 300, 128)), "heads"),  # 8 q-heads over 3 kv-heads
    (dict(idx=("i64",)), "idx"),                     # int64 indices
    (dict(idx=("noncontig",)), "idx"),
    (dict(lse=(1, 8, 31)), "lse"),
])
def test_binding_rejects_mismatched_arguments(bad, who):
    """The C ABI takes pointers and one set of sizes; the binding checks every
    tensor against them before anything reaches the library."""
    torch = pytest.importorskip("torch")
    B, Hq, Hkv, Bq, P, d = 1, 8, 2, 32, 300, 128
    args = dict(q=_cpu(B, Hq, Bq, d), k_pre=_cpu(B, Hkv, P, d), v_pre=_cpu(B, Hkv, P, d),
                k_blk=_cpu(B, Hkv, Bq, d), v_blk=_cpu(B, Hkv, Bq, d), o=_cpu(B, Hq, Bq, d),
                lse=torch.zeros(B, Hq, Bq), idx=torch.zeros(B, Hkv, 50, dtype=torch.int32))
    for k, v in bad.items():
        if v == ("f32",):
            args[k] = torch.zeros(*args[k].shape)
        elif v == ("i64",):
            args[k] = torch.zeros(B, Hkv, 50, dtype=torch.int64)
        elif v == ("noncontig",):
            args[k] = torch.zeros(B, Hkv, 100, dtype=torch.int32)[:, :, ::2]
        elif k == "lse":
            args[k] = torch.zeros(*v)
        else:
            args[k] = _cpu(*v)
    with pytest.raises(ValueError, match=who):
        ba.blkattn_full(args["q"], args["k_pre"], args["v_pre"], args["k_blk"], args["v_blk"], args["o"],
                        args["lse"], idx=args["idx"])


def test_binding_checks_partials_and_other_entry_points():
    torch = pytest.importorskip("torch")
    B, Hq, Hkv, Bq, P, d = 1, 4, 2, 32, 100, 64
    q = _cpu(B, Hq, Bq, d)
    kb = _cpu(B, Hkv, Bq, d)
    good = ba.Partial(torch.zeros(B, Hq, Bq, d), torch.zeros(B, Hq, Bq), torch.zeros(B, Hq, Bq))
    short = ba.Partial(torch.zeros(B, Hq, Bq - 1, d), torch.zeros(B, Hq, Bq - 1), torch.zeros(B, Hq, Bq - 1))
    half = ba.Partial(good.o.to(torch.bfloat16), good.m, good.l)
    with pytest.raises(ValueError, match="out.o"):
        ba.blkattn_block_partial(q, kb, kb, short)
    with pytest.raises(ValueError, match="out.o"):
        ba.blkattn_prefix_partial(q, _cpu(B, Hkv, P, d), _cpu(B, Hkv, P, d), half)
    with pytest.raises(ValueError, match="cached"):
        ba.blkattn_block_step(q, kb, kb, short, _cpu(B, Hq, Bq, d))
    with pytest.raises(ValueError, match="b.m"):
        ba.blkattn_merge(good, ba.Partial(good.o, torch.zeros(B, Hq, Bq + 1), good.l), o=_cpu(B, Hq, Bq, d))
    with pytest.raises(ValueError, match="k_out"):
        ba.blkattn_gather_prefix(_cpu(B, Hkv, P, d), _cpu(B, Hkv, P, d), torch.zeros(B, Hkv, 10, dtype=torch.int32),
                                 _cpu(B, Hkv, 9, d), _cpu(B, Hkv, 10, d))
    with pytest.raises(ValueError, match="mass"):
        ba.blkattn_prefix_mass(q, _cpu(B, Hkv, P, d), torch.zeros(B, Hq, Bq), torch.zeros(B, Hkv, P - 1))
    with pytest.raises(ValueError, match="idx"):
        ba.blkattn_select_retained(torch.zeros(B, Hkv, P), torch.zeros(B, Hkv, P + 1, dtype=torch.int32))
    with pytest.raises(ValueError, match="cache"):
        ba.blkattn_sequence_step(_cpu(B, Hq, P, d), _cpu(B, Hkv, P, d), _cpu(B, Hkv, P, d), 10, 32, short, True,
                                 _cpu(B, Hq, P, d))
    # consistent CPU arguments pass every shape check and stop at the device check
    with pytest.raises(ValueError, match="GPU only"):
        ba.blkattn_block_partial(q, kb, kb, good)
