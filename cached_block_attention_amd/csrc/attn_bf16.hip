// Partial attention of packed block-query rows over one key split, bf16 in,
// fp32 accumulate, for gfx950 (CDNA4, wave64, MFMA 32x32x16 bf16).
//
// What it computes: for every (batch, kv-head) and every query row of the G
// q-heads sharing that kv-head, the online-softmax state (m, l, O~) over the
// keys of one split of the concatenated sequence [prefix (optionally gathered
// through retained-row indices); block], streamed tile by tile with the
// recurrence of eqs. 2-6 in section 3.3.3 of "LaCache: Exact Caching and
// Precision-Adaptive Inference for Diffusion Large Language Models" (running
// max m, rescale alpha = exp(m_old - m_new), P~ = exp(S - m), l and O~
// updates), finished as o = O~ / l (same page, Appendix J pseudocode). There is
// no mask: the block is bidirectional.
//
// How it maps to the hardware:
//  * One workgroup per (key split, kv-head, packed-row chunk, batch). The rows
//    of all G q-heads of a kv-head are packed (row = g * Bq + i), so every K/V
//    tile staged in LDS feeds all of them: K/V is read from HBM once per
//    kv-head and split (GQA packing).
//  * Each wave owns 32 packed rows. Scores are computed transposed,
//    S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: keys on the M side (LDS
//    operand), queries on the N side (Q stays in registers for the whole key
//    loop). A lane then holds one query row's scores for 16 keys per 32-key
//    block, so the row max and row sum are lane-local plus one exchange
//    between the two wave halves (v_permlane32_swap).
//  * The output is accumulated transposed too, O^T += V^T P^T: P^T comes
//    straight from the score registers (converted to bf16), V^T is read from
//    LDS, where V is stored key-contiguous per head-dim row with the keys
//    permuted so that each lane's 8 keys are one 16-byte read.
//  * K/V tiles move HBM -> registers (16-byte loads, one tile ahead) ->
//    LDS (two buffers, rows padded against bank conflicts), one barrier per
//    tile.
//  * Softmax runs in base 2: scores are scaled by scale*log2(e) inside one FMA
//    before v_exp_f32; m is exported in natural-log units.
#include "launch.h"

#include <math.h>

namespace blkattn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLn2 = 0.693147180559945309f;

// Position of tile key k inside a V^T row. Within each 16-key group the order
// is keys 0-3, 8-11, 4-7, 12-15, which is the order in which the score
// registers of the two wave halves hand keys to the PV product.
__device__ __forceinline__ int vt_pos(int k) {
  const int o = k & 15;
  return (k & ~15) | (((o >> 2) & 1) << 3) | ((o >> 3) << 2) | (o & 3);
}

__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Per-(batch, kv-head) view of the key sequence [prefix (gathered); block].
struct SeqView {
  const uint16_t* kpre;  // k_pre + b*sb + h*sh
  const uint16_t* vpre;
  const uint16_t* kblk;
  const uint16_t* vblk;
  const int32_t* idx;    // idx + (b*Hkv + h)*n_pre, or nullptr
  int64_t kp_st, vp_st, kb_st, vb_st;
  int64_t n_pre, p_rows;
};

// Element offset of key j's row and whether it lies in the prefix.
__device__ __forceinline__ int64_t seq_row(const SeqView& sv, int64_t j, bool& pre) {
  pre = j < sv.n_pre;
  int64_t r = pre ? j : j - sv.n_pre;
  if (sv.idx != nullptr && pre) {
    const int64_t x = sv.idx[j];
    r = x < 0 ? 0 : (x >= sv.p_rows ? sv.p_rows - 1 : x);
  }
  return r;
}

__device__ __forceinline__ const uint16_t* k_row(const SeqView& sv, int64_t j) {
  bool pre;
  const int64_t r = seq_row(sv, j, pre);
  return pre ? sv.kpre + r * sv.kp_st : sv.kblk + r * sv.kb_st;
}

__device__ __forceinline__ const uint16_t* v_row(const SeqView& sv, int64_t j) {
  bool pre;
  const int64_t r = seq_row(sv, j, pre);
  return pre ? sv.vpre + r * sv.vp_st : sv.vblk + r * sv.vb_st;
}

template <int D, int STAGE, int NW>
__global__ __launch_bounds__(64 * NW) void attn_bf16_kernel(const AttnParams p) {
  constexpr int NT = 64 * NW;
  constexpr int CPR = D / 8;               // 16-byte chunks per K row
  constexpr int KCH = STAGE * CPR;         // K chunks per tile
  constexpr int VUN = (STAGE / 2) * CPR;   // V units per tile (2 keys x 16 bytes)
  constexpr int KIT = (KCH + NT - 1) / NT;
  constexpr int VIT = (VUN + NT - 1) / NT;
  // LDS rows are padded by 16 bytes: 16 consecutive rows read at the same
  // column then fall on distinct banks, and every operand read of a lane is a
  // fixed immediate offset from one base address.
  constexpr int K_ROW = D * 2 + 16;        // bytes per K row
  constexpr int VT_ROW = STAGE * 2 + 16;   // bytes per V^T row (one head-dim index)
  constexpr int K_BYTES = STAGE * K_ROW;
  constexpr int BUF_BYTES = K_BYTES + D * VT_ROW;
  constexpr int NSB = STAGE / 32;          // 32-key score blocks per tile
  constexpr int NDB = D / 32;              // 32-wide head-dim blocks of O^T
  __shared__ __attribute__((aligned(16))) char smem[2 * BUF_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;    // wave half
  const int n = lane & 31;    // query column of this lane / LDS row within a block
  const int split = blockIdx.x;
  const int hkv = blockIdx.y / p.row_chunks;
  const int rc = blockIdx.y - hkv * p.row_chunks;
  const int b = blockIdx.z;
  const int R = p.group * p.block_len;
  const int64_t N = p.keys.n_pre + p.keys.n_blk;
  const int t0 = (int)((int64_t)split * p.tiles / p.splits);
  const int t1 = (int)((int64_t)(split + 1) * p.tiles / p.splits);
  const int nst = t1 - t0;
  const int64_t kbeg = (int64_t)t0 * STAGE;

  SeqView sv;
  sv.kpre = (const uint16_t*)p.keys.k_pre + b * p.keys.kp_sb + hkv * p.keys.kp_sh;
  sv.vpre = (const uint16_t*)p.keys.v_pre + b * p.keys.vp_sb + hkv * p.keys.vp_sh;
  sv.kblk = (const uint16_t*)p.keys.k_blk + b * p.keys.kb_sb + hkv * p.keys.kb_sh;
  sv.vblk = (const uint16_t*)p.keys.v_blk + b * p.keys.vb_sb + hkv * p.keys.vb_sh;
  sv.idx = p.keys.idx ? p.keys.idx + ((int64_t)b * p.kv_heads + hkv) * p.keys.n_pre : nullptr;
  sv.kp_st = p.keys.kp_st, sv.vp_st = p.keys.vp_st, sv.kb_st = p.keys.kb_st, sv.vb_st = p.keys.vb_st;
  sv.n_pre = p.keys.n_pre, sv.p_rows = p.keys.p_rows;

  // ---- query fragment (B operand of S^T = K Q^T), resident for the loop ----
  const int prow = rc * p.rows_per_wg + wave * 32 + n;  // packed row of this lane
  const bool row_ok = prow < R;
  int g = 0, qi = 0;
  if (row_ok) {
    g = prow / p.block_len;
    qi = prow - g * p.block_len;
  }
  const int hq = hkv * p.group + g;
  bf16x8_t qf[D / 16];
  {
    const uint16_t* qrow = (const uint16_t*)p.q + b * p.q_sb + hq * p.q_sh + qi * p.q_st;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row_ok) v = *(const uint4*)(qrow + 16 * kk + 8 * h);
      qf[kk] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // ---- staging registers and the tile loader ----
  // K: item e -> key e / CPR, 16-byte chunk e % CPR (consecutive lanes read one
  // row contiguously). V: item u -> key pair u / CPR, chunk u % CPR; the pair is
  // interleaved into 32-bit (key, key+1) words of V^T rows.
  uint4 kreg[KIT];
  uint4 vreg[VIT][2];

  auto issue = [&](int st) {
    const int64_t key0 = kbeg + (int64_t)st * STAGE;
    const int64_t rem = N - key0;
    const int nvalid = rem < STAGE ? (int)rem : STAGE;
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const int e = tid + it * NT;
      const int key = e / CPR, j = e % CPR;
      kreg[it] = make_uint4(0, 0, 0, 0);
      if ((KCH % NT == 0 || e < KCH) && key < nvalid)
        kreg[it] = *(const uint4*)(k_row(sv, key0 + key) + 8 * j);
    }
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int u = tid + it * NT;
      const int k0 = 2 * (u / CPR), j = u % CPR;
      vreg[it][0] = make_uint4(0, 0, 0, 0);
      vreg[it][1] = make_uint4(0, 0, 0, 0);
      if (VUN % NT == 0 || u < VUN) {
        if (k0 < nvalid) vreg[it][0] = *(const uint4*)(v_row(sv, key0 + k0) + 8 * j);
        if (k0 + 1 < nvalid) vreg[it][1] = *(const uint4*)(v_row(sv, key0 + k0 + 1) + 8 * j);
      }
    }
  };

  auto commit = [&](int buf) {
    char* kb = smem + buf * BUF_BYTES;
#pragma unroll
    for (int it = 0; it < KIT; ++it) {
      const int e = tid + it * NT;
      if (KCH % NT == 0 || e < KCH) {
        const int key = e / CPR, j = e % CPR;
        *(uint4*)(kb + key * K_ROW + 16 * j) = kreg[it];
      }
    }
    char* vt = kb + K_BYTES;
#pragma unroll
    for (int it = 0; it < VIT; ++it) {
      const int u = tid + it * NT;
      if (VUN % NT == 0 || u < VUN) {
        const int k0 = 2 * (u / CPR), j = u % CPR;
        char* dst = vt + (8 * j) * VT_ROW + 2 * vt_pos(k0);
        const uint32_t a[4] = {vreg[it][0].x, vreg[it][0].y, vreg[it][0].z, vreg[it][0].w};
        const uint32_t c[4] = {vreg[it][1].x, vreg[it][1].y, vreg[it][1].z, vreg[it][1].w};
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
          const uint32_t w = (dd & 1) ? ((a[dd >> 1] >> 16) | (c[dd >> 1] & 0xffff0000u))
                                      : ((a[dd >> 1] & 0xffffu) | (c[dd >> 1] << 16));
          *(uint32_t*)(dst + dd * VT_ROW) = w;
        }
      }
    }
  };

  // ---- running state: O^T accumulators, base-2 running max, lane-partial sum ----
  f32x16_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
  float m2 = -INFINITY;
  float lsum = 0.0f;
  const float c2 = p.scale_log2;
  // per-lane operand base offsets (the rest are immediates)
  const int k_off = n * K_ROW + 16 * h;
  const int v_off = n * VT_ROW + 16 * h;

  if (nst > 0) {
    issue(0);
    commit(0);
    if (nst > 1) issue(1);
  }
  __syncthreads();

  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    if (st + 1 < nst) {
      commit(buf ^ 1);
      if (st + 2 < nst) issue(st + 2);
    }
    const char* kb = smem + buf * BUF_BYTES + k_off;
    const char* vt = smem + buf * BUF_BYTES + K_BYTES + v_off;

    // S^T blocks: keys 32*sb + (8*(r/4) + 4*h + r%4) x query n
    f32x16_t sacc[NSB];
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[sb][r] = 0.0f;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const uint4 a = *(const uint4*)(kb + (32 * sb) * K_ROW + 32 * kk);
        sacc[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), qf[kk],
                                                           sacc[sb], 0, 0, 0);
      }
    }

    // keys past the end of the sequence (last tile only) get no weight
    const int64_t rem = N - (kbeg + (int64_t)st * STAGE);
    if (rem < STAGE) {
      const int nvalid = (int)rem;
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * sb + 8 * (r >> 2) + 4 * h + (r & 3);
          if (key >= nvalid) sacc[sb][r] = -INFINITY;
        }
    }

    // online softmax (eqs. 2-5), base 2
    float mx = sacc[0][0];
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[sb][r]);
    mx = pair_max(mx);
    const float mnew = fmaxf(m2, mx * c2);
    const float alpha = __builtin_amdgcn_exp2f(m2 - mnew);
    m2 = mnew;
    float ps = 0.0f;
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(fmaf(sacc[sb][r], c2, -mnew));
        sacc[sb][r] = e;
        ps += e;
      }
    lsum = fmaf(lsum, alpha, ps);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;

    // O^T += V^T P^T (eq. 6); chunk cc covers tile keys 16*cc .. 16*cc+15
#pragma unroll
    for (int cc = 0; cc < STAGE / 16; ++cc) {
      bf16x8_t pb;
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[i] = (__bf16)sacc[cc >> 1][8 * (cc & 1) + i];
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const uint4 a = *(const uint4*)(vt + (32 * db) * VT_ROW + 32 * cc);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), pb,
                                                           oacc[db], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // ---- finish: o = O~ / l, L = m + ln l (natural-log units) ----
  const float ltot = pair_sum(lsum);
  const bool live = ltot > 0.0f;
  const float inv = live ? 1.0f / ltot : 0.0f;
  if (!row_ok) return;
  const int64_t prow_flat = ((int64_t)b * p.q_heads + hq) * p.block_len + qi;
  if (p.out.mode == kOutFinal) {
    uint16_t* orow = (uint16_t*)p.out.o + b * p.out.o_sb + hq * p.out.o_sh + qi * p.out.o_st;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = 32 * db + 8 * r4 + 4 * h;
        __bf16 v0 = (__bf16)(oacc[db][4 * r4 + 0] * inv);
        __bf16 v1 = (__bf16)(oacc[db][4 * r4 + 1] * inv);
        __bf16 v2 = (__bf16)(oacc[db][4 * r4 + 2] * inv);
        __bf16 v3 = (__bf16)(oacc[db][4 * r4 + 3] * inv);
        uint2 w;
        w.x = (uint32_t)__builtin_bit_cast(uint16_t, v0) | ((uint32_t)__builtin_bit_cast(uint16_t, v1) << 16);
        w.y = (uint32_t)__builtin_bit_cast(uint16_t, v2) | ((uint32_t)__builtin_bit_cast(uint16_t, v3) << 16);
        *(uint2*)(orow + d0) = w;
      }
    if (p.out.lse != nullptr && h == 0)
      p.out.lse[prow_flat] = live ? (m2 + __log2f(ltot)) * kLn2 : -INFINITY;
  } else {
    const int64_t base = (int64_t)split * p.out.split_rows + prow_flat;
    float* orow = p.out.po + base * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = 32 * db + 8 * r4 + 4 * h;
        float4 w = make_float4(oacc[db][4 * r4 + 0] * inv, oacc[db][4 * r4 + 1] * inv,
                               oacc[db][4 * r4 + 2] * inv, oacc[db][4 * r4 + 3] * inv);
        *(float4*)(orow + d0) = w;
      }
    if (h == 0) {
      p.out.pm[base] = live ? m2 * kLn2 : -INFINITY;
      p.out.pl[base] = ltot;
    }
  }
}

template <int D, int NW>
hipError_t launch_d_nw(const AttnParams& p, hipStream_t stream) {
  constexpr int STAGE = NW == 1 ? 32 : 64;
  dim3 grid(p.splits, p.kv_heads * p.row_chunks, p.batch);
  hipLaunchKernelGGL((attn_bf16_kernel<D, STAGE, NW>), grid, dim3(64 * NW), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnParams& p, int waves, hipStream_t stream) {
  switch (waves) {
    case 1: return launch_d_nw<D, 1>(p, stream);
    case 2: return launch_d_nw<D, 2>(p, stream);
    case 3: return launch_d_nw<D, 3>(p, stream);
    case 4: return launch_d_nw<D, 4>(p, stream);
    case 5: return launch_d_nw<D, 5>(p, stream);
    case 6: return launch_d_nw<D, 6>(p, stream);
    case 7: return launch_d_nw<D, 7>(p, stream);
    case 8: return launch_d_nw<D, 8>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int bf16_tile_keys(int waves) { return waves == 1 ? 32 : 64; }

hipError_t launch_attn_bf16(const AttnParams& p, int waves, hipStream_t stream) {
  if (p.head_dim == 128) return launch_d<128>(p, waves, stream);
  if (p.head_dim == 64) return launch_d<64>(p, waves, stream);
  return hipErrorInvalidValue;
}

}  // namespace blkattn
