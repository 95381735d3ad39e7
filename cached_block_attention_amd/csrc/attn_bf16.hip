// Partial attention of packed block-query rows over one key split, bf16 in,
// fp32 accumulate, for gfx950 (CDNA4, wave64, MFMA 32x32x16 bf16).
//
// What it computes: for every (batch, kv-head) and every query row of the G
// q-heads sharing that kv-head, the online-softmax state (m, l, O~) over the
// keys of one split of the concatenated sequence [prefix (optionally gathered
// through retained-row indices); block], streamed tile by tile with the
// recurrence of eqs. 2-6 in section 3.3.3 of "LaCache: Exact Caching and
// Precision-Adaptive Inference for Diffusion Large Language Models" (running
// max, rescale by exp(m_old - m_new), P~ = exp(S - m), l and O~ updates),
// finished as o = O~ / l (same page, Appendix J pseudocode). There is no mask:
// the block is bidirectional.
//
// How it maps to the hardware:
//  * One workgroup per (key split, kv-head, packed-row chunk, batch). The rows
//    of all G q-heads of a kv-head are packed (row = g * Bq + i), so every K/V
//    tile staged in LDS feeds all of them: K/V is read from HBM once per
//    kv-head and split (GQA packing).
//  * K/V tiles stream HBM -> LDS with direct-to-LDS DMA loads
//    (global_load_lds_dwordx4: 64 lanes x 16 bytes per instruction, no
//    register staging) into a ring of NS stages, so NS-1 tiles are in flight
//    while one is computed; one barrier per tile. Rows are stored with an XOR
//    swizzle of their 16-byte chunks, chosen on the global side of the DMA.
//  * Each wave owns 32 packed rows. Scores are computed transposed,
//    S^T = K Q^T (v_mfma_f32_32x32x16_bf16; keys on the M side read from LDS,
//    queries on the N side held in registers for the whole loop), so a lane
//    holds one query row's scores for 16 keys per 32-key block: the row max
//    and sum are lane-local plus one exchange between the wave halves.
//  * The output is accumulated transposed, O^T += V^T P^T: P^T comes straight
//    from the score registers (converted to bf16), and V^T is read from the
//    row-major V tile with ds_read_b64_tr_b16 (transposing LDS reads).
//  * Softmax runs in base 2 (scale * log2(e) folded into one FMA before
//    v_exp_f32). The reference max is only moved when a tile's max exceeds it
//    by more than kSlack (2^8): the O~ rescale is skipped otherwise, which is
//    exact because l and O~ always share the same reference. The true running
//    max is tracked separately and exported in natural-log units.
//  * The weights enter the PV product rounded to bf16. O~ is normalised by the
//    sum of those rounded weights (v_dot2_f32_bf16 against (1, 1)), so o is an
//    exact convex combination of V rows with the weights actually used; l and
//    the log-sum-exp use the sum of the unrounded weights.
#include "launch.h"

#include <math.h>

namespace blkattn {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;
constexpr float kSlack = 8.0f;  // log2 of the largest unnormalised weight allowed

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// XOR swizzle of the 16-byte chunk index of K row r (CPR chunks per row):
// 16 consecutive rows read at one logical chunk land on distinct banks.
template <int CPR>
__device__ __forceinline__ int swz_k(int r) {
  return CPR == 16 ? (r & 15) : ((r ^ (r >> 3)) & 7);
}

// XOR swizzle of V row r for the transposing reads, where one read of 32 lanes
// covers 4 rows x 64 bytes: it spreads the 4 rows over distinct chunk groups.
template <int CPR>
__device__ __forceinline__ int swz_v(int r) {
  return CPR == 16 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2);
}

__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// s_waitcnt vmcnt(n) leaving the other counters free (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most `ahead` later stages of this wave's DMAs are in flight.
template <int IPW, int NS>
__device__ __forceinline__ void wait_stage(int ahead) {
  if (NS >= 4 && ahead >= 2) wait_vm<(NS >= 4 ? 2 : 0) * IPW>();
  else if (NS >= 3 && ahead >= 1) wait_vm<(NS >= 3 ? 1 : 0) * IPW>();
  else wait_vm<0>();
}

// Workgroup barrier without the memory fence of __syncthreads(): the fence
// would drain every outstanding DMA (vmcnt(0)) at each tile. LDS data is
// ordered explicitly instead: DMA completion by s_waitcnt vmcnt before the
// barrier, and every LDS read of a tile is consumed by an MFMA before the
// barrier that lets its ring slot be refilled.
__device__ __forceinline__ void tile_barrier() {
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
}

// One direct-to-LDS DMA: 64 lanes x 16 bytes from per-lane global addresses
// into 1 KB of LDS at lds_addr (wave-uniform, through M0). Written as inline
// asm so that the compiler does not see an LDS write in flight and drain the
// whole DMA ring (vmcnt(0)) before every LDS read; completion is ordered
// explicitly by wait_stage() before the tile barrier. The instruction has no
// register results.
__device__ __forceinline__ void dma_1k(const void* gptr, uint32_t lds_addr) {
  __asm__ __volatile__(
      "s_mov_b32 m0, %0\n\t"
      "global_load_lds_dwordx4 %1, off"
      :
      : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(gptr)
      : "memory", "m0");
}

constexpr int kIdxCap = 2048;  // retained-row indices staged per split

template <int D, int NW, int TK, int NS>
__global__ __launch_bounds__(64 * NW) void attn_bf16_kernel(const AttnParams p) {
  constexpr int ROWB = D * 2;              // bytes per K/V row
  constexpr int CPR = ROWB / 16;           // 16-byte chunks per row
  constexpr int KBYTES = TK * ROWB;        // K part of a stage
  constexpr int STB = 2 * KBYTES;          // bytes per stage (K then V)
  constexpr int INS = STB / 1024;          // DMA instructions per stage
  constexpr int IPW = INS / NW;            // per wave
  constexpr int RPI = 1024 / ROWB;         // rows per DMA instruction
  constexpr int NSB = TK / 32;             // 32-key score blocks per tile
  constexpr int NCC = TK / 16;             // 16-key chunks of the PV product
  constexpr int NDB = D / 32;              // 32-wide head-dim blocks of O^T
  static_assert(INS % NW == 0, "every wave issues the same number of DMAs");
  static_assert(IPW * (NS - 2) < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) char ring[NS * STB];
  __shared__ int32_t sidx[kIdxCap];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;    // wave half
  const int n = lane & 31;    // query column of this lane / operand row within a block
  const int split = blockIdx.x;
  const int hkv = blockIdx.y / p.row_chunks;
  const int rc = blockIdx.y - hkv * p.row_chunks;
  const int b = blockIdx.z;
  const int R = p.group * p.block_len;
  const int t0 = (int)((int64_t)split * p.tiles / p.splits);
  const int t1 = (int)((int64_t)(split + 1) * p.tiles / p.splits);
  const int nst = t1 - t0;
  const int64_t kbeg = (int64_t)t0 * TK;

  // key sequence of this (batch, kv-head): byte pointers and row strides
  const char* kpre = (const char*)p.keys.k_pre + 2 * (b * p.keys.kp_sb + hkv * p.keys.kp_sh);
  const char* vpre = (const char*)p.keys.v_pre + 2 * (b * p.keys.vp_sb + hkv * p.keys.vp_sh);
  const char* kblk = (const char*)p.keys.k_blk + 2 * (b * p.keys.kb_sb + hkv * p.keys.kb_sh);
  const char* vblk = (const char*)p.keys.v_blk + 2 * (b * p.keys.vb_sb + hkv * p.keys.vb_sh);
  const int64_t kp_st = 2 * p.keys.kp_st, vp_st = 2 * p.keys.vp_st;
  const int64_t kb_st = 2 * p.keys.kb_st, vb_st = 2 * p.keys.vb_st;
  const int64_t n_pre = p.keys.n_pre;
  const int64_t n_all = p.keys.n_pre + p.keys.n_blk;
  const bool indexed = p.keys.idx != nullptr;

  // ---- retained-row indices of this split's prefix keys, staged in LDS ----
  if (indexed) {
    const int64_t lo = kbeg < n_pre ? kbeg : n_pre;
    const int64_t hi0 = kbeg + (int64_t)nst * TK;
    const int64_t hi = hi0 < n_pre ? hi0 : n_pre;
    const int32_t* src = p.keys.idx + ((int64_t)b * p.kv_heads + hkv) * n_pre;
    for (int64_t j = lo + tid; j < hi; j += 64 * NW) {
      int64_t r = src[j];
      r = r < 0 ? 0 : (r >= p.keys.p_rows ? p.keys.p_rows - 1 : r);
      sidx[j - kbeg] = (int32_t)r;
    }
    __syncthreads();
  }

  // ---- query fragment (B operand of S^T = K Q^T), resident for the loop ----
  const int prow = rc * p.rows_per_wg + wave * 32 + n;  // packed row of this lane
  const bool computes = wave * 32 < p.rows_per_wg && rc * p.rows_per_wg + wave * 32 < R;  // wave-uniform
  const bool row_ok = computes && prow < R;
  int g = 0, qi = 0;
  if (row_ok) {
    g = prow / p.block_len;
    qi = prow - g * p.block_len;
  }
  const int hq = hkv * p.group + g;
  const int64_t srow = qi + (qi >= p.rows.q_hole ? p.rows.q_hole_len : 0);  // sequence row
  const int64_t mrow = ((int64_t)b * p.q_heads + hq) * p.rows.row_pitch + srow;  // per-row arrays
  bf16x8_t qf[D / 16];
  {
    const uint16_t* qrow = (const uint16_t*)p.q + b * p.q_sb + hq * p.q_sh + srow * p.q_st;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row_ok) v = *(const uint4*)(qrow + 16 * kk + 8 * h);
      qf[kk] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  // ---- DMA of one tile into a ring slot ----
  // Instruction k of a stage fills 1 KB: K rows for k < INS/2, V rows after.
  // Lane t writes LDS slot (row, physical chunk t % CPR), which holds the
  // row's logical chunk (t % CPR) ^ swizzle(row).
  const int lrow = lane / CPR;
  const int lchunk = lane % CPR;
  auto issue = [&](int t) {
    char* slot = ring + (t % NS) * STB;
    const int64_t key0 = kbeg + (int64_t)t * TK;
    const bool dense = !indexed && key0 + TK <= n_pre;  // tile inside the dense prefix
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int k = wave * IPW + j;   // wave-uniform
      const bool isv = k >= INS / 2;
      const int kk = isv ? k - INS / 2 : k;
      const int r = kk * RPI + lrow;
      const int lc = lchunk ^ (isv ? swz_v<CPR>(r) : swz_k<CPR>(r));
      const char* base = isv ? vpre : kpre;
      int64_t st = isv ? vp_st : kp_st;
      int64_t row = key0 + r;
      if (dense) {
        row += row >= p.keys.k_hole ? p.keys.k_hole_len : 0;
      } else {
        int64_t key = row < n_all ? row : n_all - 1;  // rows past the end: any valid row (weight 0)
        if (key < n_pre) {
          row = indexed ? (int64_t)sidx[key - kbeg] : key + (key >= p.keys.k_hole ? p.keys.k_hole_len : 0);
        } else {
          row = key - n_pre;
          base = isv ? vblk : kblk;
          st = isv ? vb_st : kb_st;
        }
      }
      dma_1k(base + row * st + 16 * lc,
             (uint32_t)(uintptr_t)LDS_PTR(char, slot + k * 1024));
    }
  };

  // ---- per-lane operand coordinates of the transposing V reads ----
  // Source lane s = lane % 16 of each 16-lane group reads V row
  // 16*cc + 8*rr + 4*h + s/4 at head-dim columns 32*db + 16*dh + 4*(s%4) .. +3;
  // output lane (h, m) then holds V[16*cc + 8*rr + 4*h + e][32*db + m], e = 0..3.
  const int vi = (lane & 15) >> 2;
  const int vq = lane & 3;
  const int vdh = (lane >> 4) & 1;

  // ---- running state ----
  f32x16_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
  float m2 = -INFINITY;     // reference max (base 2) shared by l and O~
  float mtrue = -INFINITY;  // exact running max (base 2)
  float lsum = 0.0f;        // lane-partial sum of weights
  float lhat = 0.0f;        // lane-partial sum of the bf16-rounded weights
  const float c2 = p.scale_log2;
  // Initial state from a cached partial (LaCache Appendix J: the running
  // (m, l, O~) of a later step starts from the cache): O~ = l * o, m in base 2,
  // l carried by the lanes of the first wave half.
  if (p.init_m != nullptr && row_ok) {
    const float mi = p.init_m[mrow];
    const float li = p.init_l[mrow];
    if (mi > -INFINITY && li > 0.0f) {
      m2 = mi * kLog2e;
      mtrue = m2;
      lsum = h == 0 ? li : 0.0f;
      lhat = lsum;
      const float* orow = p.init_o + mrow * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const float4 v = *(const float4*)(orow + 32 * db + 8 * r4 + 4 * h);
          oacc[db][4 * r4 + 0] = v.x * li;
          oacc[db][4 * r4 + 1] = v.y * li;
          oacc[db][4 * r4 + 2] = v.z * li;
          oacc[db][4 * r4 + 3] = v.w * li;
        }
    }
  }

  wait_vm<0>();  // the query fragment has landed before any DMA is counted
  const int npro = nst < NS - 1 ? nst : NS - 1;
  for (int t = 0; t < npro; ++t) issue(t);

  for (int t = 0; t < nst; ++t) {
    const int ahead = (nst - 1 - t) < (NS - 2) ? (nst - 1 - t) : (NS - 2);
    wait_stage<IPW, NS>(ahead);
    tile_barrier();
    if (t + NS - 1 < nst) issue(t + NS - 1);
    if (!computes) continue;

    const char* kb = ring + (t % NS) * STB;
    const char* vb = kb + KBYTES;

    // S^T blocks: keys 32*sb + (8*(r/4) + 4*h + r%4) x query n
    f32x16_t sacc[NSB];
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[sb][r] = 0.0f;
      const int krow = 32 * sb + n;
      const int ksw = swz_k<CPR>(krow);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const uint4 a = *(const uint4*)(kb + krow * ROWB + 16 * ((2 * kk + h) ^ ksw));
        sacc[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), qf[kk],
                                                           sacc[sb], 0, 0, 0);
      }
    }

    // keys past the end of the sequence (last tile only) get no weight
    const int64_t rem = n_all - (kbeg + (int64_t)t * TK);
    if (rem < TK) {
      const int nvalid = (int)rem;
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * sb + 8 * (r >> 2) + 4 * h + (r & 3);
          if (key >= nvalid) sacc[sb][r] = -INFINITY;
        }
    }

    // online softmax (eqs. 2-5) in base 2 with a lazily moved reference max
    float mx = sacc[0][0];
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[sb][r]);
    const float mt = pair_max(mx) * c2;
    mtrue = fmaxf(mtrue, mt);
    if (__any(mt > m2 + kSlack)) {
      const float mnew = fmaxf(m2, mt);
      const float alpha = __builtin_amdgcn_exp2f(m2 - mnew);
      m2 = mnew;
      lsum *= alpha;
      lhat *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    float ps = 0.0f;
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(fmaf(sacc[sb][r], c2, -m2));
        sacc[sb][r] = e;
        ps += e;
      }
    lsum += ps;

    // O^T += V^T P^T (eq. 6); chunk cc covers tile keys 16*cc .. 16*cc+15
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) {
      bf16x8_t pb;
#pragma unroll
      for (int i = 0; i < 8; ++i) pb[i] = (__bf16)sacc[cc >> 1][8 * (cc & 1) + i];
      {
        bf16x2_t one;
        one[0] = (__bf16)1.0f;
        one[1] = (__bf16)1.0f;
        lhat = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 0, 1), one, lhat, false);
        lhat = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 2, 3), one, lhat, false);
        lhat = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 4, 5), one, lhat, false);
        lhat = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 6, 7), one, lhat, false);
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        i16x4_t lo, hi;
        {
          const int row = 16 * cc + 4 * h + vi;
          const int pc = (4 * db + 2 * vdh + (vq >> 1)) ^ swz_v<CPR>(row);
          lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              LDS_PTR(i16x4_t, vb + row * ROWB + 16 * pc + 8 * (vq & 1)));
        }
        {
          const int row = 16 * cc + 8 + 4 * h + vi;
          const int pc = (4 * db + 2 * vdh + (vq >> 1)) ^ swz_v<CPR>(row);
          hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              LDS_PTR(i16x4_t, vb + row * ROWB + 16 * pc + 8 * (vq & 1)));
        }
        const bf16x8_t a = __builtin_bit_cast(
            bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[db], 0, 0, 0);
      }
    }
  }

  // ---- finish: o = O~ / l, L = m + ln l (natural-log units) ----
  const float ltot = pair_sum(lsum);
  const float lhtot = pair_sum(lhat);
  const bool live = ltot > 0.0f;
  const float inv = live ? 1.0f / lhtot : 0.0f;
  if (!row_ok) return;
  if (p.out.mode == kOutFinal) {
    uint16_t* orow = (uint16_t*)p.out.o + b * p.out.o_sb + hq * p.out.o_sh + srow * p.out.o_st;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = 32 * db + 8 * r4 + 4 * h;
        const __bf16 v0 = (__bf16)(oacc[db][4 * r4 + 0] * inv);
        const __bf16 v1 = (__bf16)(oacc[db][4 * r4 + 1] * inv);
        const __bf16 v2 = (__bf16)(oacc[db][4 * r4 + 2] * inv);
        const __bf16 v3 = (__bf16)(oacc[db][4 * r4 + 3] * inv);
        uint2 w;
        w.x = (uint32_t)__builtin_bit_cast(uint16_t, v0) | ((uint32_t)__builtin_bit_cast(uint16_t, v1) << 16);
        w.y = (uint32_t)__builtin_bit_cast(uint16_t, v2) | ((uint32_t)__builtin_bit_cast(uint16_t, v3) << 16);
        *(uint2*)(orow + d0) = w;
      }
    if (p.out.lse != nullptr && h == 0)
      p.out.lse[mrow] = live ? (m2 + __log2f(ltot)) * kLn2 : -INFINITY;
  } else {
    const int64_t base = p.out.mode == kOutSplit
                             ? (int64_t)split * p.out.split_rows + ((int64_t)b * p.q_heads + hq) * p.block_len + qi
                             : mrow;
    float* orow = p.out.po + base * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = 32 * db + 8 * r4 + 4 * h;
        *(float4*)(orow + d0) = make_float4(oacc[db][4 * r4 + 0] * inv, oacc[db][4 * r4 + 1] * inv,
                                            oacc[db][4 * r4 + 2] * inv, oacc[db][4 * r4 + 3] * inv);
      }
    if (h == 0) {
      // export the exact max: l is re-referenced from m2 to it
      p.out.pm[base] = live ? mtrue * kLn2 : -INFINITY;
      p.out.pl[base] = live ? ltot * __builtin_amdgcn_exp2f(m2 - mtrue) : 0.0f;
    }
  }
}

// Launch shapes: NW waves per workgroup (each 32 packed rows), TK keys per
// tile, NS ring stages.
template <int D, int NW>
hipError_t launch_d_nw(const AttnParams& p, hipStream_t stream) {
  constexpr int TK = NW == 1 ? 32 : 64;
  constexpr int NS = 4;
  dim3 grid(p.splits, p.kv_heads * p.row_chunks, p.batch);
  hipLaunchKernelGGL((attn_bf16_kernel<D, NW, TK, NS>), grid, dim3(64 * NW), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnParams& p, int waves, hipStream_t stream) {
  switch (waves) {
    case 1: return launch_d_nw<D, 1>(p, stream);
    case 2: return launch_d_nw<D, 2>(p, stream);
    case 4: return launch_d_nw<D, 4>(p, stream);
    case 8: return launch_d_nw<D, 8>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int bf16_tile_keys(int waves) { return waves == 1 ? 32 : 64; }

int bf16_waves_for_rows(int64_t rows) {
  if (rows <= 32) return 1;
  if (rows <= 64) return 2;
  if (rows <= 128) return 4;
  return 8;
}

int bf16_workgroups_per_cu(int waves) { return waves >= 4 ? 1 : 2; }

int bf16_index_cap() { return kIdxCap; }

hipError_t launch_attn_bf16(const AttnParams& p, int waves, hipStream_t stream) {
  if (p.head_dim == 128) return launch_d<128>(p, waves, stream);
  if (p.head_dim == 64) return launch_d<64>(p, waves, stream);
  return hipErrorInvalidValue;
}

}  // namespace blkattn
