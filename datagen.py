"""Seeded synthetic inputs for block-diffusion attention over a cached prefix.

This module is shared by the tests, the benchmark and the smoke check. It only
draws random numbers and rounds them to the storage type: it holds none of the
attention arithmetic, so both the fp64 oracle and the HIP path consume the same
host buffers without sharing any computation.

Workloads (the five shapes the method is exercised on):

  tiny_f32     fp32, B1, H4/4, d64, P256, Bq32
  llada_bf16   bf16, B1, H32/32, d128, P4096, Bq32          (LLaDA-8B-like layer)
  dream_gqa    bf16, B4, Hq28/Hkv4, d128, P32768, Bq32,     (Dream-7B-like GQA)
               1 % of the prefix key rows scaled by 4 (salient-token outliers)
  reuse_bf16   bf16, B8, H32/32, d128, P16384, Bq32, 8 denoising steps
  sparse_gqa   bf16, B2, Hq28/Hkv4, d128, P_full 131072, n_keep 8192, Bq64,
               per-(batch, kv-head) sorted distinct int32 row indices
  llada_seq    bf16, B1, H32/32, d128, a 4096-row sequence whose block is rows
               [2048, 2080), 8 denoising steps (full-sequence FACache step:
               prompt and earlier blocks before the block, masked suffix after)

Generator: numpy PCG64 ``standard_normal`` in float32, rounded to bfloat16 with
round-to-nearest-even (kept as uint16 bit patterns; numpy has no bf16 type) or
kept as float32 for the fp32 workload. Layout [B, H, rows, d], contiguous.

Seeds: workload c (1..6) uses base 1000*c; streams base+1 Q, +2 K_prefix,
+3 V_prefix, +4 K_block, +5 V_block, +6 outlier rows, +7 indices. Denoising
step t of the reuse workload draws Q_t, K_t, V_t from base + 100*(t+1) + {1,4,5}.
The sequence workload draws the whole sequence's Q, K, V from base + {1, 2, 3};
at step t >= 1 the block rows of each are redrawn from base + 100*(t+1) + {1, 2, 3}
and every other row keeps its value (LaCache: U token ids do not change).
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"


# ---------------------------------------------------------------------------
# storage-type rounding (input preparation only)
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(seed: int, shape, dtype: str, chunk_axis0: bool = True) -> np.ndarray:
    """N(0,1) of `shape` from PCG64(seed), stored as float32 or bf16 bits.

    Large tensors are drawn one slice of axis 0 at a time from the same
    generator, which yields exactly the same stream as a single draw.
    """
    g = np.random.default_rng(seed)
    out_dtype = np.float32 if dtype == F32 else np.uint16
    out = np.empty(shape, dtype=out_dtype)
    if not chunk_axis0 or len(shape) == 0 or shape[0] == 0:
        x = g.standard_normal(shape, dtype=np.float32)
        out[...] = x if dtype == F32 else f32_to_bf16_bits(x)
        return out
    for i in range(shape[0]):
        x = g.standard_normal(shape[1:], dtype=np.float32)
        out[i] = x if dtype == F32 else f32_to_bf16_bits(x)
    return out


# ---------------------------------------------------------------------------
# problem description
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Shape:
    name: str
    dtype: str
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    prefix_len: int          # P (dense) or P_full (when n_keep is set)
    block_len: int           # Bq: block queries == block keys
    n_keep: Optional[int] = None
    outlier_frac: float = 0.0
    outlier_scale: float = 4.0
    steps: int = 1
    seed_base: int = 0
    block_start: Optional[int] = None  # sequence workloads: the block's first row

    @property
    def group(self) -> int:
        return self.q_heads // self.kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def prefix_keys(self) -> int:
        """Prefix rows actually attended (n_keep when gathered, else P)."""
        return self.n_keep if self.n_keep is not None else self.prefix_len

    @property
    def elt_bytes(self) -> int:
        return 4 if self.dtype == F32 else 2


WORKLOADS = {
    "tiny_f32": Shape("tiny_f32", F32, 1, 4, 4, 64, 256, 32, seed_base=1000),
    "llada_bf16": Shape("llada_bf16", BF16, 1, 32, 32, 128, 4096, 32, seed_base=2000),
    "dream_gqa": Shape("dream_gqa", BF16, 4, 28, 4, 128, 32768, 32,
                       outlier_frac=0.01, seed_base=3000),
    "reuse_bf16": Shape("reuse_bf16", BF16, 8, 32, 32, 128, 16384, 32, steps=8,
                        seed_base=4000),
    "sparse_gqa": Shape("sparse_gqa", BF16, 2, 28, 4, 128, 131072, 64, n_keep=8192,
                        seed_base=5000),
    # prefix_len is the sequence length N here; the block is rows [block_start, +block_len)
    "llada_seq": Shape("llada_seq", BF16, 1, 32, 32, 128, 4096, 32, steps=8, seed_base=6000,
                       block_start=2048),
}


@dataclasses.dataclass
class Inputs:
    shape: Shape
    q: np.ndarray            # [B, Hq, Bq, d]
    k_pre: np.ndarray        # [B, Hkv, P(_full), d]
    v_pre: np.ndarray
    k_blk: np.ndarray        # [B, Hkv, Bq, d]
    v_blk: np.ndarray
    idx: Optional[np.ndarray] = None          # int32 [B, Hkv, n_keep], sorted
    outlier_rows: Optional[np.ndarray] = None  # int64 [B, n_outliers]


def outlier_rows(shape: Shape, seed: int) -> np.ndarray:
    """Per batch element, round(frac*P) distinct prefix positions (all kv-heads)."""
    n = int(round(shape.outlier_frac * shape.prefix_len))
    g = np.random.default_rng(seed)
    rows = np.empty((shape.batch, n), dtype=np.int64)
    for b in range(shape.batch):
        rows[b] = np.sort(g.choice(shape.prefix_len, size=n, replace=False))
    return rows


def retained_indices(batch: int, kv_heads: int, p_full: int, n_keep: int, seed: int) -> np.ndarray:
    """Independent per-(batch, kv-head) draws of n_keep distinct rows, sorted."""
    g = np.random.default_rng(seed)
    idx = np.empty((batch, kv_heads, n_keep), dtype=np.int32)
    for b in range(batch):
        for h in range(kv_heads):
            idx[b, h] = np.sort(g.choice(p_full, size=n_keep, replace=False)).astype(np.int32)
    return idx


def make_inputs(shape: Shape, seed_base: Optional[int] = None) -> Inputs:
    """Draw every input of `shape` from its seeded streams."""
    base = shape.seed_base if seed_base is None else seed_base
    B, Hq, Hkv, d = shape.batch, shape.q_heads, shape.kv_heads, shape.head_dim
    P, Bq, dt = shape.prefix_len, shape.block_len, shape.dtype
    q = _normal(base + 1, (B, Hq, Bq, d), dt)
    k_pre = _normal(base + 2, (B, Hkv, P, d), dt)
    v_pre = _normal(base + 3, (B, Hkv, P, d), dt)
    k_blk = _normal(base + 4, (B, Hkv, Bq, d), dt)
    v_blk = _normal(base + 5, (B, Hkv, Bq, d), dt)
    rows = None
    if shape.outlier_frac > 0.0 and P > 0:
        rows = outlier_rows(shape, base + 6)
        for b in range(B):
            # scaling by a power of two is exact in both storage types
            sel = k_pre[b][:, rows[b], :]
            if dt == F32:
                k_pre[b][:, rows[b], :] = sel * np.float32(shape.outlier_scale)
            else:
                k_pre[b][:, rows[b], :] = f32_to_bf16_bits(
                    bf16_bits_to_f32(sel) * np.float32(shape.outlier_scale))
    idx = None
    if shape.n_keep is not None:
        idx = retained_indices(B, Hkv, P, shape.n_keep, base + 7)
    return Inputs(shape, q, k_pre, v_pre, k_blk, v_blk, idx, rows)


def step_inputs(shape: Shape, t: int, seed_base: Optional[int] = None):
    """Fresh (Q_t, K_blk_t, V_blk_t) of denoising step t (reuse workload)."""
    base = (shape.seed_base if seed_base is None else seed_base) + 100 * (t + 1)
    B, Hq, Hkv, d, Bq, dt = (shape.batch, shape.q_heads, shape.kv_heads,
                             shape.head_dim, shape.block_len, shape.dtype)
    return (_normal(base + 1, (B, Hq, Bq, d), dt),
            _normal(base + 4, (B, Hkv, Bq, d), dt),
            _normal(base + 5, (B, Hkv, Bq, d), dt))


def scaled_shape(name: str, **overrides) -> Shape:
    """A workload with some sizes overridden (small parity cases)."""
    return dataclasses.replace(WORKLOADS[name], **overrides)


def sequence_inputs(shape: Shape, t: int = 0, seed_base: Optional[int] = None):
    """(q [B, Hq, N, d], k, v [B, Hkv, N, d]) of the whole sequence at denoising
    step t: step 0 draws every row; a later step redraws only the block's rows
    (rows [block_start, block_start + block_len)), the others keep step 0's values."""
    base = shape.seed_base if seed_base is None else seed_base
    B, Hq, Hkv, d, N, dt = (shape.batch, shape.q_heads, shape.kv_heads, shape.head_dim,
                            shape.prefix_len, shape.dtype)
    c0, Bq = shape.block_start, shape.block_len
    q = _normal(base + 1, (B, Hq, N, d), dt)
    k = _normal(base + 2, (B, Hkv, N, d), dt)
    v = _normal(base + 3, (B, Hkv, N, d), dt)
    if t > 0:
        sb = base + 100 * (t + 1)
        q[:, :, c0:c0 + Bq] = _normal(sb + 1, (B, Hq, Bq, d), dt)
        k[:, :, c0:c0 + Bq] = _normal(sb + 2, (B, Hkv, Bq, d), dt)
        v[:, :, c0:c0 + Bq] = _normal(sb + 3, (B, Hkv, Bq, d), dt)
    return q, k, v
