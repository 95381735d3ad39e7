"""Host checks of the seeded input recipe (no attention arithmetic here)."""

import numpy as np

import datagen


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5, 3.0e38], dtype=np.float32)
    got = datagen.bf16_bits_to_f32(datagen.f32_to_bf16_bits(x))
    # spacing near 1 is 2^-7; halfway cases go to the even mantissa
    assert got[0] == 1.0 and got[1] == 1.0 and got[2] == np.float32(1.0 + 2**-6)
    assert got[3] == 1.0 and got[4] == -2.5
    assert np.isfinite(got[5])


def test_chunked_draws_are_one_stream():
    a = datagen._normal(7, (3, 5, 4), datagen.F32, chunk_axis0=False)
    b = datagen._normal(7, (3, 5, 4), datagen.F32, chunk_axis0=True)
    assert np.array_equal(a, b)


def test_outliers_and_indices_recipe():
    sh = datagen.scaled_shape("dream_gqa", batch=2, prefix_len=1000)
    inp = datagen.make_inputs(sh)
    assert inp.outlier_rows.shape == (2, 10)
    for b in range(2):
        r = inp.outlier_rows[b]
        assert len(set(r.tolist())) == 10
        base = datagen._normal(sh.seed_base + 2, inp.k_pre.shape, datagen.BF16)
        ratio = datagen.bf16_bits_to_f32(inp.k_pre[b][:, r]) / datagen.bf16_bits_to_f32(base[b][:, r])
        ok = np.isfinite(ratio)
        assert np.all(ratio[ok] == 4.0)
        other = np.setdiff1d(np.arange(1000), r)
        assert np.array_equal(inp.k_pre[b][:, other], base[b][:, other])
    sp = datagen.scaled_shape("sparse_gqa", prefix_len=5000, n_keep=300)
    inp = datagen.make_inputs(sp)
    assert inp.idx.dtype == np.int32 and inp.idx.shape == (2, 4, 300)
    for b in range(2):
        for h in range(4):
            row = inp.idx[b, h]
            assert np.all(np.diff(row) > 0) and row[0] >= 0 and row[-1] < 5000


def test_workload_table():
    w = datagen.WORKLOADS
    assert (w["dream_gqa"].group, w["dream_gqa"].prefix_len, w["dream_gqa"].block_len) == (7, 32768, 32)
    assert w["sparse_gqa"].prefix_keys == 8192 and w["tiny_f32"].dtype == datagen.F32
