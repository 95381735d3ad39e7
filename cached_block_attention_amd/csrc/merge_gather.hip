// Log-sum-exp merge of partial attention states, the retained-row gather, and
// the empty-state fill, for gfx950. All three are HBM-bound streaming kernels.
//
// Merge: for partials (o_s, m_s, l_s) of the same query rows over disjoint key
// sets, M = max_s m_s, w_s = l_s e^{m_s - M}, l = sum_s w_s,
// o = sum_s w_s o_s / l, LSE = M + ln l. Continuing the online-softmax
// recurrence (eqs. 2-6 of section 3.3.3 of "LaCache: Exact Caching and
// Precision-Adaptive Inference for Diffusion Large Language Models") from a
// cached state over further key tiles gives exactly this; the same kernel
// reduces the key splits of one attention call (fixed order over s, so the
// result is bitwise reproducible).
//
// Gather: k_out[b, h, r] = k_full[b, h, idx[b, h, r]] (and v), a bit copy of the
// retained rows (aitopics "kv state" page, Sparse-dLLM abstract).
#include "launch.h"

#include <math.h>

namespace blkattn {
namespace {

// One thread merges 4 consecutive head-dim values of one row; D/4 threads of
// the same wave share a row, so a row's m and l are read by all of its lanes in
// the same instruction, before any lane writes them (safe in-place update).
// The partials are consumed in chunks of CH: all loads of a chunk are issued
// before any is used, then folded into a running (M, L, acc) with the merge
// formula, in fixed split order.
template <int D, int CH>
__global__ __launch_bounds__(256) void merge_kernel(const MergeParams p) {
  constexpr int TPR = D / 4;
  constexpr int RPB = 256 / TPR;
  const int64_t rows = (int64_t)p.batch * p.q_heads * p.block_len;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const int c4 = threadIdx.x % TPR;
  if (row >= rows) return;
  const int64_t hb = row / p.block_len;  // b * Hq + hq
  const int64_t qi = row - hb * p.block_len;
  const int64_t srow = qi + (qi >= p.rows.q_hole ? p.rows.q_hole_len : 0);  // sequence row
  const int64_t mrow = hb * p.rows.row_pitch + srow;                      // per-row arrays

  float M = -INFINITY;
  float L = 0.0f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < p.nsrc; s0 += CH) {
    float ms[CH], ls[CH];
    float4 os[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int s = s0 + i;
      ms[i] = -INFINITY;
      ls[i] = 0.0f;
      os[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (s < p.nsrc) {
        const float* po;
        if (p.strided) {
          const int64_t e = (int64_t)s * p.split_rows + row;
          ms[i] = p.src_m[0][e];
          ls[i] = p.src_l[0][e];
          po = p.src_o[0] + e * D;
        } else {
          const int si = s < 2 ? s : 1;  // two explicit sources
          ms[i] = p.src_m[si][mrow];
          ls[i] = p.src_l[si][mrow];
          po = p.src_o[si] + mrow * D;
        }
        os[i] = *(const float4*)(po + 4 * c4);
      }
    }
    float mc = M;
#pragma unroll
    for (int i = 0; i < CH; ++i) mc = fmaxf(mc, ms[i]);
    if (mc == -INFINITY) continue;  // every partial so far is empty
    if (M != -INFINITY) {
      const float sc = expf(M - mc);
      L *= sc;
      acc.x *= sc, acc.y *= sc, acc.z *= sc, acc.w *= sc;
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const float w = (ms[i] == -INFINITY) ? 0.0f : ls[i] * expf(ms[i] - mc);
      L += w;
      acc.x = fmaf(w, os[i].x, acc.x);
      acc.y = fmaf(w, os[i].y, acc.y);
      acc.z = fmaf(w, os[i].z, acc.z);
      acc.w = fmaf(w, os[i].w, acc.w);
    }
    M = mc;
  }
  const bool live = L > 0.0f;
  const float inv = live ? 1.0f / L : 0.0f;
  const float4 o = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  const float mo = live ? M : -INFINITY;

  if (p.o_final != nullptr) {
    const int64_t b = hb / p.q_heads, hq = hb - (hb / p.q_heads) * p.q_heads;
    const int64_t off = b * p.o_sb + hq * p.o_sh + srow * p.o_st + 4 * c4;
    if (p.out_dtype == 0) {
      *(float4*)((float*)p.o_final + off) = o;
    } else {
      const __bf16 v0 = (__bf16)o.x, v1 = (__bf16)o.y, v2 = (__bf16)o.z, v3 = (__bf16)o.w;
      uint2 w;
      w.x = (uint32_t)__builtin_bit_cast(uint16_t, v0) | ((uint32_t)__builtin_bit_cast(uint16_t, v1) << 16);
      w.y = (uint32_t)__builtin_bit_cast(uint16_t, v2) | ((uint32_t)__builtin_bit_cast(uint16_t, v3) << 16);
      *(uint2*)((uint16_t*)p.o_final + off) = w;
    }
  }
  if (p.lse != nullptr && c4 == 0) p.lse[mrow] = live ? M + logf(L) : -INFINITY;
  if (p.out_o != nullptr) {
    *(float4*)(p.out_o + mrow * D + 4 * c4) = o;
    if (c4 == 0) {
      p.out_m[mrow] = mo;
      p.out_l[mrow] = live ? L : 0.0f;
    }
  }
}

// One thread copies one 16-byte chunk of one retained row of K and of V.
__global__ __launch_bounds__(256) void gather_kernel(const GatherParams p) {
  const int cpr = p.head_dim * p.elt_bytes / 16;
  const int64_t total = (int64_t)p.batch * p.kv_heads * p.n_keep * cpr;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= total) return;
  const int64_t rowi = e / cpr;
  const int c = (int)(e - rowi * cpr);
  const int64_t bh = rowi / p.n_keep;
  const int64_t r = rowi - bh * p.n_keep;
  const int64_t b = bh / p.kv_heads, h = bh - (bh / p.kv_heads) * p.kv_heads;
  int64_t src = p.idx[rowi];
  src = src < 0 ? 0 : (src >= p.p_rows ? p.p_rows - 1 : src);
  const int64_t eb = p.elt_bytes;
  const char* ks = (const char*)p.k_full + (b * p.kf_sb + h * p.kf_sh + src * p.kf_st) * eb;
  const char* vs = (const char*)p.v_full + (b * p.vf_sb + h * p.vf_sh + src * p.vf_st) * eb;
  char* kd = (char*)p.k_out + (b * p.ko_sb + h * p.ko_sh + r * p.ko_st) * eb;
  char* vd = (char*)p.v_out + (b * p.vo_sb + h * p.vo_sh + r * p.vo_st) * eb;
  const uint4 kv = *(const uint4*)(ks + 16 * c);
  const uint4 vv = *(const uint4*)(vs + 16 * c);
  *(uint4*)(kd + 16 * c) = kv;
  *(uint4*)(vd + 16 * c) = vv;
}

// Empty key set: o = 0, m = -inf, l = 0.
__global__ __launch_bounds__(256) void fill_empty_kernel(float* o, float* m, float* l, int64_t rows,
                                                         int head_dim) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e < rows * head_dim) o[e] = 0.0f;
  if (e < rows) {
    m[e] = -INFINITY;
    l[e] = 0.0f;
  }
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.batch * p.q_heads * p.block_len;
  if (rows == 0) return hipSuccess;
  if (p.head_dim == 128) {
    const int64_t blocks = (rows + 7) / 8;
    hipLaunchKernelGGL((merge_kernel<128, 8>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
  } else if (p.head_dim == 64) {
    const int64_t blocks = (rows + 15) / 16;
    hipLaunchKernelGGL((merge_kernel<64, 8>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gather(const GatherParams& p, hipStream_t stream) {
  const int64_t total = (int64_t)p.batch * p.kv_heads * p.n_keep * (p.head_dim * p.elt_bytes / 16);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_fill_empty(float* o, float* m, float* l, int64_t rows, int head_dim,
                             hipStream_t stream) {
  const int64_t total = rows * head_dim;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_empty_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                     o, m, l, rows, head_dim);
  return hipGetLastError();
}

}  // namespace blkattn
