// Partial attention in fp32 (fp32 inputs, fp32 FMA accumulation) for gfx950.
//
// Same operation as the bf16 kernel - the online-softmax state of the block
// queries over one key split of [prefix (optionally gathered); block], eqs. 2-6
// of section 3.3.3 of "LaCache: Exact Caching and Precision-Adaptive Inference
// for Diffusion Large Language Models", finished as o = O~/l, L = m + ln l
// (Appendix J pseudocode) - for the fp32 workloads, where exactness matters
// more than speed (small sizes, errors near 1e-6). One workgroup per (key
// split, q-head, batch); each thread owns one query row, keeps q and O~ in
// registers, and streams 32-key K/V tiles staged in LDS (read as broadcasts).
#include "launch.h"

#include <math.h>

namespace blkattn {
namespace {

constexpr int kF32Tile = 32;

__device__ __forceinline__ const float* key_row_f32(const KeySeq& ks, int b, int hkv, int kv_heads,
                                                    int64_t j, bool want_v) {
  if (j < ks.n_pre) {
    int64_t row = j + (j >= ks.k_hole ? ks.k_hole_len : 0);
    if (ks.idx != nullptr) {
      int64_t r = ks.idx[((int64_t)b * kv_heads + hkv) * ks.n_pre + j];
      row = r < 0 ? 0 : (r >= ks.p_rows ? ks.p_rows - 1 : r);
    }
    return want_v ? (const float*)ks.v_pre + b * ks.vp_sb + hkv * ks.vp_sh + row * ks.vp_st
                  : (const float*)ks.k_pre + b * ks.kp_sb + hkv * ks.kp_sh + row * ks.kp_st;
  }
  const int64_t row = j - ks.n_pre;
  return want_v ? (const float*)ks.v_blk + b * ks.vb_sb + hkv * ks.vb_sh + row * ks.vb_st
                : (const float*)ks.k_blk + b * ks.kb_sb + hkv * ks.kb_sh + row * ks.kb_st;
}

template <int D>
__global__ __launch_bounds__(64) void attn_f32_kernel(const AttnParams p) {
  __shared__ __attribute__((aligned(16))) float ks[kF32Tile][D];
  __shared__ __attribute__((aligned(16))) float vs[kF32Tile][D];
  const int tid = threadIdx.x;
  const int split = blockIdx.x;
  const int hq = blockIdx.y;
  const int b = blockIdx.z;
  const int hkv = hq / p.group;
  const int64_t N = p.keys.n_pre + p.keys.n_blk;
  const int t0 = (int)((int64_t)split * p.tiles / p.splits);
  const int t1 = (int)((int64_t)(split + 1) * p.tiles / p.splits);
  const float scale = p.scale;

  for (int i0 = 0; i0 < p.block_len; i0 += 64) {
    const int qi = i0 + tid;
    const bool ok = qi < p.block_len;
    float q[D];
    float o[D];
    const int64_t srow = ok ? qi + (qi >= p.rows.q_hole ? p.rows.q_hole_len : 0) : 0;  // sequence row
    const int64_t mrow = ((int64_t)b * p.q_heads + hq) * p.rows.row_pitch + srow;      // per-row arrays
    const float* qrow = (const float*)p.q + b * p.q_sb + hq * p.q_sh + srow * p.q_st;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      q[d] = ok ? qrow[d] : 0.0f;
      o[d] = 0.0f;
    }
    float m = -INFINITY, l = 0.0f;
    if (p.init_m != nullptr && ok) {
      // initial state from a cached partial: O~ = l * o (LaCache Appendix J)
      const float mi = p.init_m[mrow];
      const float li = p.init_l[mrow];
      if (mi > -INFINITY && li > 0.0f) {
        m = mi;
        l = li;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] = p.init_o[mrow * D + d] * li;
      }
    }
    for (int t = t0; t < t1; ++t) {
      const int64_t key0 = (int64_t)t * kF32Tile;
      const int64_t rem = N - key0;
      const int nvalid = rem < kF32Tile ? (int)rem : kF32Tile;
      __syncthreads();
      for (int e = tid; e < kF32Tile * (D / 4); e += 64) {
        const int key = e / (D / 4), c = e - (e / (D / 4)) * (D / 4);
        float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
        if (key < nvalid) {
          kv = *(const float4*)(key_row_f32(p.keys, b, hkv, p.kv_heads, key0 + key, false) + 4 * c);
          vv = *(const float4*)(key_row_f32(p.keys, b, hkv, p.kv_heads, key0 + key, true) + 4 * c);
        }
        *(float4*)&ks[key][4 * c] = kv;
        *(float4*)&vs[key][4 * c] = vv;
      }
      __syncthreads();
      // scores: the head dimension outermost, so that the tile's keys are 32
      // independent FMA chains
      float s[kF32Tile];
#pragma unroll
      for (int j = 0; j < kF32Tile; ++j) s[j] = 0.0f;
#pragma unroll
      for (int d4 = 0; d4 < D / 4; ++d4)
#pragma unroll
        for (int j = 0; j < kF32Tile; ++j) {
          const float4 k4 = *(const float4*)&ks[j][4 * d4];
          s[j] = fmaf(q[4 * d4 + 0], k4.x, s[j]);
          s[j] = fmaf(q[4 * d4 + 1], k4.y, s[j]);
          s[j] = fmaf(q[4 * d4 + 2], k4.z, s[j]);
          s[j] = fmaf(q[4 * d4 + 3], k4.w, s[j]);
        }
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < kF32Tile; ++j) {
        s[j] = j < nvalid ? s[j] * scale : -INFINITY;
        mx = fmaxf(mx, s[j]);
      }
      const float mnew = fmaxf(m, mx);
      const float alpha = expf(m - mnew);
      l *= alpha;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] *= alpha;
#pragma unroll
      for (int j = 0; j < kF32Tile; ++j) {
        const float pj = expf(s[j] - mnew);
        l += pj;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] = fmaf(pj, vs[j][d], o[d]);
      }
      m = mnew;
    }
    if (!ok) continue;
    const bool live = l > 0.0f;
    const float inv = live ? 1.0f / l : 0.0f;
    if (p.out.mode == kOutFinal) {
      float* orow = (float*)p.out.o + b * p.out.o_sb + hq * p.out.o_sh + srow * p.out.o_st;
#pragma unroll
      for (int d = 0; d < D; d += 4)
        *(float4*)(orow + d) = make_float4(o[d] * inv, o[d + 1] * inv, o[d + 2] * inv, o[d + 3] * inv);
      if (p.out.lse != nullptr) p.out.lse[mrow] = live ? m + logf(l) : -INFINITY;
    } else {
      const int64_t base = p.out.mode == kOutSplit
                               ? (int64_t)split * p.out.split_rows + ((int64_t)b * p.q_heads + hq) * p.block_len + qi
                               : mrow;
      float* orow = p.out.po + base * D;
#pragma unroll
      for (int d = 0; d < D; d += 4)
        *(float4*)(orow + d) = make_float4(o[d] * inv, o[d + 1] * inv, o[d + 2] * inv, o[d + 3] * inv);
      p.out.pm[base] = live ? m : -INFINITY;
      p.out.pl[base] = l;
    }
  }
}

}  // namespace

hipError_t launch_attn_f32(const AttnParams& p, hipStream_t stream, KernelEvents ev) {
  dim3 grid(p.splits, p.q_heads, p.batch);
  if (p.head_dim == 64)
    hipExtLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(64), 0, stream, ev.start, ev.stop, 0, p);
  else if (p.head_dim == 128)
    hipExtLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(64), 0, stream, ev.start, ev.stop, 0, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace blkattn
