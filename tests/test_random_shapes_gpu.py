"""Parity of blkattn_full with the fp64 oracle over seeded random shapes.

The launch plan picks a kernel from the packed row count and the key range of
a split: the fp32 kernel; one row wave with or without a DMA wave; two or four
row waves; the eight-wave ping-pong kernel (129 to 224 rows, with one or two
idle row waves); the eight-wave sequential kernel (225 to 256 rows); several
row chunks above 256 rows. The cases below are drawn once from a fixed seed
over group sizes 1-9, block lengths 1-80, prefixes 0-2500 (dense, or gathered
through sorted indices), head dims 64 and 128, outlier rows and forced split
counts, so that together they cover every one of those paths with ragged key
and row tails. Tolerances as in test_parity_gpu.py.
"""

import numpy as np
import pytest

import datagen
from tests.test_parity_gpu import ba, check_full  # noqa: F401  (ba is a fixture)

pytestmark = pytest.mark.gpu


def _cases(n=32, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        f32 = rng.random() < 0.15
        g = int(rng.integers(1, 10))
        hkv = int(rng.integers(1, 3))
        bq = int(rng.choice([1, 7, 16, 20, 32, 32, 32, 40, 64, 80]))
        p = int(rng.choice([0, 33, 64, 300, 777, 1000, 1500, 2500]))
        d = int(rng.choice([64, 128]))
        kw = dict(dtype=datagen.F32 if f32 else datagen.BF16, batch=int(rng.integers(1, 3)), q_heads=g * hkv,
                  kv_heads=hkv, head_dim=d, prefix_len=p, block_len=bq, seed_base=50000 + 100 * i,
                  outlier_frac=0.0 if f32 or rng.random() < 0.5 else 0.01, n_keep=None)
        if not f32 and p > 0 and rng.random() < 0.3:
            kw["n_keep"] = int(rng.integers(0, p + 1))
        splits = int(rng.choice([0, 0, 1, 2, 3, 7]))
        out.append((kw, splits))
    return out


CASES = _cases()


def _id(case):
    kw, splits = case
    keep = f"k{kw['n_keep']}" if kw["n_keep"] is not None else ""
    return (f"{kw['dtype']}-B{kw['batch']}-G{kw['q_heads'] // kw['kv_heads']}x{kw['kv_heads']}-d{kw['head_dim']}"
            f"-P{kw['prefix_len']}{keep}-Bq{kw['block_len']}-s{splits}")


def test_cases_cover_every_kernel_path():
    rows = [c[0]["q_heads"] // c[0]["kv_heads"] * c[0]["block_len"] for c in CASES if c[0]["dtype"] == datagen.BF16]
    assert any(r <= 32 for r in rows)
    assert any(32 < r <= 128 for r in rows)
    assert any(128 < r <= 192 for r in rows)     # ping-pong with an idle row wave
    assert any(192 < r <= 224 for r in rows)     # ping-pong, all seven row waves
    assert any(224 < r <= 256 for r in rows)     # eight-wave sequential
    assert any(r > 256 for r in rows)            # several row chunks
    assert any(c[0]["dtype"] == datagen.F32 for c in CASES)
    assert any(c[0]["n_keep"] is not None for c in CASES)


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_full_random_shape(ba, case):  # noqa: F811
    kw, splits = case
    sh = datagen.scaled_shape("dream_gqa", **kw)
    check_full(ba, sh, splits=splits)
