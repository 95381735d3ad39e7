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
//    register staging) into rings of LDS tiles, several tiles in flight. Rows
//    are stored with an XOR swizzle of their 16-byte chunks, chosen on the
//    global side of the DMA. Where the workgroup has a wave that owns no rows,
//    that wave (and, in the ping-pong kernel, one more) issues the DMAs, so
//    the waves that compute never stall behind the memory pipeline.
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
//    sum of those rounded weights, taken by the matrix core next to the PV
//    product (one 16x16x32 MFMA per 16 keys against a selector of ones), so o
//    is an exact convex combination of V rows with the weights actually used;
//    l and the log-sum-exp use the sum of the unrounded weights.
//  * Eight-wave workgroups of 129 to 224 packed rows run the two halves of
//    the workgroup half a tile apart ("ping-pong"): waves 0-3 and 4-7 share
//    the four SIMDs pairwise, and while one wave of a pair issues the MFMAs of
//    a tile (PV of the previous tile, then the scores of this one) the other
//    runs the softmax of its tile on the vector ALU. The matrix cores and the
//    vector ALU of a SIMD then work at the same time instead of in turn.
#include "gfx950.h"
#include "launch.h"

#include <math.h>

#include <type_traits>

namespace blkattn {
namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;
constexpr float kSlack = 8.0f;  // log2 of the largest unnormalised weight allowed


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

// max(a, b, c) as one v_max3_f32. fmaxf() would first quiet possible
// signalling NaNs of MFMA results (one extra v_max per operand); scores are
// never NaN here.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  __asm__("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// x of lane l ^ 32. v_permlane32_swap exchanges the upper half of its first
// operand with the lower half of its second: with x in both, the first result
// holds the other half's x in lanes 32-63 and the second in lanes 0-31.
__device__ __forceinline__ float other_half(float x, int lane) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(lane < 32 ? r[1] : r[0]);
}

__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}


constexpr int kIdxCap = 2048;  // retained-row indices staged per split

// The key sequence of one (batch, kv-head), in bytes.
struct KeyRows {
  const char* kpre;
  const char* vpre;
  const char* kblk;
  const char* vblk;
  int64_t kp_st, vp_st, kb_st, vb_st;  // row strides in bytes
  int64_t n_pre, n_all, hole, hole_len;
  bool indexed, off32, gather32;
};

// A tile whose rows all come from one strided segment: the dense prefix on
// one side of the key hole, or the block. Rows past the segment's end (the
// last tile of the sequence) repeat its last row; their weight is 0.
struct SegTile {
  const char* base;  // row 0 of the tile
  int64_t st;        // row stride in bytes
  int valid;         // rows inside the segment
};

template <int TK>
__device__ __forceinline__ bool tile_is_fast(const KeyRows& kr, int64_t key0) {
  if (!kr.off32) return false;
  if (key0 >= kr.n_pre) return true;  // block rows
  return !kr.indexed && key0 + TK <= kr.n_pre && (key0 + TK <= kr.hole || key0 >= kr.hole);
}

template <int TK>
__device__ __forceinline__ SegTile seg_tile(const KeyRows& kr, bool isv, int64_t key0) {
  SegTile f;
  if (key0 >= kr.n_pre) {
    f.st = isv ? kr.vb_st : kr.kb_st;
    f.base = (isv ? kr.vblk : kr.kblk) + (key0 - kr.n_pre) * f.st;
    const int64_t left = kr.n_all - key0;
    f.valid = left < TK ? (int)left : TK;
  } else {
    f.st = isv ? kr.vp_st : kr.kp_st;
    f.base = (isv ? kr.vpre : kr.kpre) + (key0 + (key0 >= kr.hole ? kr.hole_len : 0)) * f.st;
    f.valid = TK;
  }
  f.base = uniform_ptr(f.base);
  return f;
}

template <int D, int TK, bool NT = false>
__device__ __forceinline__ void dma_one_fast(const SegTile& f, bool isv, uint32_t dst, int k, int lane) {
  constexpr int ROWB = D * 2;
  constexpr int CPR = ROWB / 16;
  constexpr int RPI = 1024 / ROWB;
  const int ln = opaque(lane);
  const int r = k * RPI + ln / CPR;
  const int rs = r < f.valid ? r : f.valid - 1;
  const int lc = (ln % CPR) ^ (isv ? swz_v<CPR>(r) : swz_k<CPR>(r));
  dma_1k_s<NT>(f.base, (uint32_t)rs * (uint32_t)f.st + 16 * lc, dst + k * 1024);
}

// A whole tile of contiguous rows (row stride = row bytes): 16 KB of memory
// onto 16 KB of LDS. Its DMAs go in groups of four that share the scalar base
// and M0 (instruction offsets 0, 1 KB, 2 KB, 3 KB), and a lane's offset within
// a group is a swizzle pattern that depends only on the DMA's place in the
// group (and for D = 64 on the group's parity), so the whole issue costs a
// few vector instructions instead of an address computation per DMA.
template <int D, int TK, bool NT = false>
__device__ __forceinline__ void dma_tile_contig(const char* sbase, bool isv, uint32_t dst, int lane) {
  constexpr int ROWB = D * 2;
  constexpr int CPR = ROWB / 16;
  constexpr int RPI = 1024 / ROWB;
  constexpr int INT = TK * ROWB / 1024;
  static_assert(INT % 4 == 0, "whole groups of four DMAs");
  const int ln = opaque(lane);
  const int rl = ln / CPR;
  const int cl = ln % CPR;
#pragma unroll
  for (int g = 0; g < INT / 4; ++g) {
    uint32_t v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (4 * g + i) * RPI + rl;
      const int lc = cl ^ (isv ? swz_v<CPR>(r) : swz_k<CPR>(r));
      v[i] = (uint32_t)(rl * ROWB + 16 * lc);
    }
    dma_4k_s<NT>(sbase + 4096 * g, v[0], v[1], v[2], v[3], dst + 4096 * g);
  }
}

// The per-lane offsets of dma_tile_contig for every DMA of a K and a V tile,
// for a wave that issues many tiles and has registers to spare: computed
// once, they make each later contiguous tile a run of scalar-addressed DMAs
// with no vector work.
template <int D, int TK>
struct ContigLanes {
  static constexpr int INT = TK * D * 2 / 1024;
  uint32_t k[INT];
  uint32_t v[INT];
};

template <int D, int TK>
__device__ __forceinline__ ContigLanes<D, TK> contig_lanes(int lane) {
  constexpr int ROWB = D * 2;
  constexpr int CPR = ROWB / 16;
  constexpr int RPI = 1024 / ROWB;
  ContigLanes<D, TK> c;
  const int rl = lane / CPR;
  const int cl = lane % CPR;
#pragma unroll
  for (int j = 0; j < ContigLanes<D, TK>::INT; ++j) {
    const int r = j * RPI + rl;
    c.k[j] = (uint32_t)(rl * ROWB + 16 * (cl ^ swz_k<CPR>(r)));
    c.v[j] = (uint32_t)(rl * ROWB + 16 * (cl ^ swz_v<CPR>(r)));
  }
  return c;
}

template <int D, int TK, bool NT = false>
__device__ __forceinline__ void dma_tile_contig_pre(const char* sbase, const uint32_t (&off)[TK * D * 2 / 1024],
                                                    uint32_t dst) {
  constexpr int INT = TK * D * 2 / 1024;
#pragma unroll
  for (int g = 0; g < INT / 4; ++g)
    dma_4k_s<NT>(sbase + 4096 * g, off[4 * g], off[4 * g + 1], off[4 * g + 2], off[4 * g + 3], dst + 4096 * g);
}

// A tile of retained (gathered) prefix rows whose byte offsets from the head's
// first row fit 31 bits: scalar head base plus per-lane offsets from the
// staged indices.
template <int TK>
__device__ __forceinline__ bool tile_is_gather(const KeyRows& kr, int64_t key0) {
  return kr.indexed && kr.gather32 && key0 + TK <= kr.n_pre;
}

// The DMA of one gathered tile: every instruction's staged index is read
// before the first DMA goes out. The DMA asm may touch memory, so an index
// read placed between two of them waits out a full LDS round trip before its
// own DMA; read first, the tile pays that latency once.
template <int D, int TK>
__device__ __forceinline__ void dma_tile_gather(const KeyRows& kr, bool isv, int64_t key0, uint32_t dst, int lane,
                                                const int32_t* sidx, int64_t kbeg) {
  constexpr int ROWB = D * 2;
  constexpr int CPR = ROWB / 16;
  constexpr int RPI = 1024 / ROWB;
  constexpr int INT = TK * ROWB / 1024;
  const char* sbase = uniform_ptr(isv ? kr.vpre : kr.kpre);
  const uint32_t st = (uint32_t)(isv ? kr.vp_st : kr.kp_st);
  const int ln = opaque(lane);
  const int32_t* tidx = sidx + (key0 - kbeg);
  uint32_t row[INT];
#pragma unroll
  for (int k = 0; k < INT; ++k) row[k] = (uint32_t)tidx[k * RPI + ln / CPR];
#pragma unroll
  for (int k = 0; k < INT; ++k) {
    const int r = k * RPI + ln / CPR;
    const int lc = (ln % CPR) ^ (isv ? swz_v<CPR>(r) : swz_k<CPR>(r));
    dma_1k_s(sbase, row[k] * st + 16 * lc, dst + k * 1024);
  }
}

// DMA instruction k of the K (isv = false) or V rows of one TK-key tile
// starting at key key0, into the LDS tile at byte address dst (TK * 2D bytes,
// TK*2D/1024 instructions of 1 KB). Instruction k covers tile rows
// k*RPI .. k*RPI + RPI - 1; lane t fills LDS chunk t % CPR of its row with
// logical chunk (t % CPR) ^ swizzle(row). Keys past the end of the sequence
// read a valid row (their weight is 0); retained-row indices come from sidx
// (this split's, from key kbeg on).
//
// The general form: a 64-bit address per lane, for any tile. Waves that
// issue only a few DMAs per tile between their own compute use it everywhere:
// the scalar-base forms above cost them more in readfirstlane and scalar
// address work than they save.
template <int D, int TK>
__device__ __forceinline__ void dma_one(const KeyRows& kr, bool isv, int64_t key0, uint32_t dst, int k, int lane,
                                        const int32_t* sidx, int64_t kbeg) {
  constexpr int ROWB = D * 2;
  constexpr int CPR = ROWB / 16;
  constexpr int RPI = 1024 / ROWB;
  const bool dense = !kr.indexed && key0 + TK <= kr.n_pre;
  const int r = k * RPI + lane / CPR;
  const int lc = (lane % CPR) ^ (isv ? swz_v<CPR>(r) : swz_k<CPR>(r));
  const char* base = isv ? kr.vpre : kr.kpre;
  int64_t st = isv ? kr.vp_st : kr.kp_st;
  int64_t row = key0 + r;
  if (dense) {
    row += row >= kr.hole ? kr.hole_len : 0;
  } else {
    const int64_t key = row < kr.n_all ? row : kr.n_all - 1;
    if (key < kr.n_pre) {
      row = kr.indexed ? (int64_t)sidx[key - kbeg] : key + (key >= kr.hole ? kr.hole_len : 0);
    } else {
      row = key - kr.n_pre;
      base = isv ? kr.vblk : kr.kblk;
      st = isv ? kr.vb_st : kr.kb_st;
    }
  }
  dma_1k(base + row * st + 16 * lc, dst + k * 1024);
}

// The whole DMA of one K (or V) tile, issued by one wave. On the fast path
// each instruction is a scalar base plus a per-lane offset recomputed from the
// lane index (a few VALU operations, no registers held across the loop); the
// other tiles loop over the general form without unrolling it. With NT the
// strided tiles (dense prefix and block) are loaded non-temporal.
template <int D, int TK, bool NT = false>
__device__ __forceinline__ void dma_tile_all(const KeyRows& kr, bool isv, int64_t key0, uint32_t dst, int lane,
                                             const int32_t* sidx, int64_t kbeg) {
  constexpr int INT = TK * D * 2 / 1024;
  if (tile_is_fast<TK>(kr, key0)) {
    const SegTile f = seg_tile<TK>(kr, isv, key0);
    if (f.valid == TK && f.st == 2 * D) {
      dma_tile_contig<D, TK, NT>(f.base, isv, dst, lane);
      return;
    }
#pragma unroll
    for (int k = 0; k < INT; ++k) dma_one_fast<D, TK, NT>(f, isv, dst, k, lane);
    return;
  }
  if (tile_is_gather<TK>(kr, key0)) {
    dma_tile_gather<D, TK>(kr, isv, key0, dst, lane, sidx, kbeg);
    return;
  }
#pragma unroll 1
  for (int k = 0; k < INT; ++k) dma_one<D, TK>(kr, isv, key0, dst, k, lane, sidx, kbeg);
}

// dma_tile_all for a wave holding the contiguous path's lane offsets.
template <int D, int TK, bool NT = false>
__device__ __forceinline__ void dma_tile_all_pre(const KeyRows& kr, bool isv, int64_t key0, uint32_t dst, int lane,
                                                 const int32_t* sidx, int64_t kbeg, const ContigLanes<D, TK>& cl) {
  if (tile_is_fast<TK>(kr, key0)) {
    const SegTile f = seg_tile<TK>(kr, isv, key0);
    if (f.valid == TK && f.st == 2 * D) {
      dma_tile_contig_pre<D, TK, NT>(f.base, isv ? cl.v : cl.k, dst);
      return;
    }
  }
  dma_tile_all<D, TK, NT>(kr, isv, key0, dst, lane, sidx, kbeg);
}

// This wave's share of the DMA of one K (or V) tile: with NW waves issuing,
// wave w issues instructions w*IPW .. w*IPW + IPW - 1, in the general form.
template <int D, int TK, int NW, bool IDX = false>
__device__ __forceinline__ void dma_tile(const KeyRows& kr, bool isv, int64_t key0, uint32_t dst, int wave,
                                         int lane, const int32_t* sidx, int64_t kbeg) {
  constexpr int IPW = TK * D * 2 / 1024 / NW;
  if (IDX && key0 + TK <= kr.n_pre) {
    // a retained-row tile (IDX: launches with retained-row indices): this
    // wave's indices are read before its DMAs go out (an index read between
    // two DMAs waits out an LDS round trip)
    constexpr int ROWB = D * 2;
    constexpr int CPR = ROWB / 16;
    constexpr int RPI = 1024 / ROWB;
    const int32_t* tidx = sidx + (key0 - kbeg);
    int64_t row[IPW];
#pragma unroll
    for (int j = 0; j < IPW; ++j) row[j] = tidx[(wave * IPW + j) * RPI + lane / CPR];
    const char* base = isv ? kr.vpre : kr.kpre;
    const int64_t st = isv ? kr.vp_st : kr.kp_st;
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int k = wave * IPW + j;
      const int r = k * RPI + lane / CPR;
      const int lc = (lane % CPR) ^ (isv ? swz_v<CPR>(r) : swz_k<CPR>(r));
      dma_1k(base + row[j] * st + 16 * lc, dst + k * 1024);
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < IPW; ++j) dma_one<D, TK>(kr, isv, key0, dst, wave * IPW + j, lane, sidx, kbeg);
}

// S^T = K Q^T for one tile: sacc[sb] holds keys 32*sb + 8*(r/4) + 4*h + r%4
// (register r) against this lane's query. Scheduling is left to the compiler,
// which interleaves these MFMAs with the vector work around them.
template <int D, int TK>
__device__ __forceinline__ void tile_scores(f32x16_t (&sacc)[TK / 32], const char* kb,
                                            const bf16x8_t (&qf)[D / 16], int n, int h) {
  constexpr int ROWB = D * 2;
  constexpr int CPR = ROWB / 16;
#pragma unroll
  for (int sb = 0; sb < TK / 32; ++sb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[sb][r] = 0.0f;
    const int krow = 32 * sb + n;
    const int ksw = swz_k<CPR>(krow);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const uint4 a = *(const uint4*)(kb + krow * ROWB + 16 * ((2 * kk + h) ^ ksw));
      sacc[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), qf[kk], sacc[sb], 0, 0, 0);
    }
  }
}

// The sum of the bf16-rounded weights, taken by the matrix core: one
// v_mfma_f32_16x16x32_bf16 per 16-key chunk, with the chunk's weights (the B
// operand of the PV product, lane (h, n): query n) as its B operand. There
// lane l = 32h + n stands for column n % 16 and key group 2h + n / 16, so
// column c carries the keys of query c in the even groups and of query c + 16
// in the odd ones. A selector A operand of zeros and ones adds the even groups
// into rows 0-7 and the odd ones into rows 8-15, so every register of a lane
// holds the full sum of one query: of its own query where h = n / 16 (bits 5
// and 4 of the lane agree), else of query n ^ 16, the query of lane l ^ 16.
// Accumulated in fp32 exactly as the PV product sees the weights; one MFMA
// replaces four v_dot2_f32_bf16, which cannot overlap the matrix core's work.
__device__ __forceinline__ bool lsum_lane_is_own(int lane) { return ((lane >> 5) & 1) == ((lane >> 4) & 1); }

__device__ __forceinline__ bf16x8_t lsum_selector(int lane) {
  const bool one = ((lane & 15) < 8) == (((lane >> 4) & 1) == 0);
  bf16x8_t a;
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = one ? (__bf16)1.0f : (__bf16)0.0f;
  return a;
}

__device__ __forceinline__ void sum_weights_mfma(f32x4_t& lacc, const bf16x8_t& sel, const bf16x8_t& pb) {
  lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, pb, lacc, 0, 0, 0);
}

// The value of x held by the lane whose query this lane's weight sum belongs
// to (lane l ^ 16 for the lanes that hold another query's sum).
__device__ __forceinline__ float for_lsum_lane(float x, int lane) {
  const float other = __shfl_xor(x, 16);
  return lsum_lane_is_own(lane) ? x : other;
}

// Running online-softmax state of one lane's query row.
template <int D>
struct RowState {
  f32x16_t oacc[D / 32];  // O~^T: head dims 32*db + 8*(r/4) + 4*h + r%4
  float m2;               // reference max (base 2) shared by l and O~
  float mtrue;            // exact running max (base 2)
  float lsum;             // lane-partial sum of the weights
  f32x4_t lacc;           // sum of the bf16-rounded weights of query n or n ^ 16 (sum_weights_mfma)
};

// Eqs. 2-5 for one tile: mask keys past `nvalid`, move the reference max if
// needed (rescaling O~ and the sums), weights P~ = 2^(s*c2 - m2) into the sum
// l and, rounded to bf16, into the PV operand pb (chunk cc: 16 keys). The
// rounded weights are summed by the matrix core where the PV product
// consumes pb (sum_weights_mfma).
template <int D, int TK>
__device__ __forceinline__ void tile_softmax(f32x16_t (&sacc)[TK / 32], bf16x8_t (&pb)[TK / 16],
                                             RowState<D>& st, float c2, int64_t nvalid, int lane) {
  const int h = lane >> 5;
  constexpr int NSB = TK / 32;
  if (nvalid < TK) {
    const int nv = (int)nvalid;
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * sb + 8 * (r >> 2) + 4 * h + (r & 3);
        if (key >= nv) sacc[sb][r] = -INFINITY;
      }
  }
  // Four independent chains in every reduction: a lone wave gets no latency
  // hiding from other waves while its SIMD partner runs MFMAs.
  // chain j covers registers r with r % 4 == j: values k = sb*16 + r
  float mx4[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float m = sacc[0][j];
#pragma unroll
    for (int k = 4; k + 4 < NSB * 16; k += 8)
      m = max3f(m, sacc[k / 16][(k % 16) + j], sacc[(k + 4) / 16][((k + 4) % 16) + j]);
    m = max3f(m, m, sacc[NSB - 1][12 + j]);
    mx4[j] = m;
  }
  const float mt = pair_max(max3f(max3f(mx4[0], mx4[1], mx4[2]), mx4[3], mx4[3])) * c2;
  st.mtrue = fmaxf(st.mtrue, mt);
  if (__any(mt > st.m2 + kSlack)) {
    const float mnew = fmaxf(st.m2, mt);
    const float alpha = __builtin_amdgcn_exp2f(st.m2 - mnew);
    st.m2 = mnew;
    st.lsum *= alpha;
    st.lacc *= for_lsum_lane(alpha, lane);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) st.oacc[db] *= alpha;
  }
  const float neg_m2 = -st.m2;
  float ps[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = __builtin_amdgcn_exp2f(fmaf(sacc[sb][r], c2, neg_m2));
      sacc[sb][r] = e;
      ps[r & 3] += e;
    }
  st.lsum += (ps[0] + ps[1]) + (ps[2] + ps[3]);
#pragma unroll
  for (int cc = 0; cc < TK / 16; ++cc)
#pragma unroll
    for (int i = 0; i < 8; ++i) pb[cc][i] = (__bf16)sacc[cc >> 1][8 * (cc & 1) + i];
}

// O^T += V^T P^T (eq. 6) for one tile. Chunk cc covers tile keys 16*cc ..
// 16*cc + 15; in the B operand lane (h, n) element i is key
// 16*cc + 8*(i/4) + 4*h + i%4 (the order of the score registers), and the
// transposing reads give the A operand the same key order: source lane
// s = lane % 16 of each 16-lane group reads V row 16*cc + 8*rr + 4*h + s/4 at
// head-dim columns 32*db + 16*dh + 4*(s%4) .. +3.
template <int D, int TK>
__device__ __forceinline__ void tile_pv(f32x16_t (&oacc)[D / 32], f32x4_t& lacc, const bf16x8_t (&pb)[TK / 16],
                                        const char* vb, int lane) {
  const bf16x8_t sel = lsum_selector(lane);
  constexpr int ROWB = D * 2;
  constexpr int CPR = ROWB / 16;
  const int h = lane >> 5;
  const int vi = (lane & 15) >> 2;
  const int vq = lane & 3;
  const int vdh = (lane >> 4) & 1;
#pragma unroll
  for (int cc = 0; cc < TK / 16; ++cc)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      i16x4_t lo, hi;
      {
        const int row = 16 * cc + 4 * h + vi;
        const int pc = (4 * db + 2 * vdh + (vq >> 1)) ^ swz_v<CPR>(row);
        lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4_t, vb + row * ROWB + 16 * pc + 8 * (vq & 1)));
      }
      {
        const int row = 16 * cc + 8 + 4 * h + vi;
        const int pc = (4 * db + 2 * vdh + (vq >> 1)) ^ swz_v<CPR>(row);
        hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4_t, vb + row * ROWB + 16 * pc + 8 * (vq & 1)));
      }
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[cc], oacc[db], 0, 0, 0);
      if (db == 0) sum_weights_mfma(lacc, sel, pb[cc]);
    }
}

// LDS reads at integer byte addresses.
__device__ __forceinline__ bf16x8_t lds_b128(uint32_t a) {
  return __builtin_bit_cast(bf16x8_t, *(const __attribute__((address_space(3))) uint4*)(uintptr_t)a);
}

__device__ __forceinline__ bf16x8_t lds_tr_pair(uint32_t lo, uint32_t hi) {
  const i16x4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(uintptr_t)lo);
  const i16x4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)(uintptr_t)hi);
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// The MFMA phase of the ping-pong kernel when it has both parts: O^T += V^T P^T
// for the previous tile (V tile at LDS byte address va) and S^T = K Q^T for
// this tile (K tile at ka), issued as one sequence of MFMAs whose LDS operands
// are read PD MFMAs ahead. Operand layouts as in tile_pv and tile_scores.
template <int D, int TK>
__device__ __forceinline__ void mfma_phase_both(f32x16_t (&oacc)[D / 32], const bf16x8_t (&pb)[TK / 16],
                                                uint32_t va, f32x16_t (&sacc)[TK / 32], uint32_t ka,
                                                const bf16x8_t (&qf)[D / 16], int lane, f32x4_t& lacc,
                                                const bf16x8_t& sel) {
  constexpr int ROWB = D * 2;
  constexpr int CPR = ROWB / 16;
  constexpr int NCC = TK / 16;
  constexpr int NDB = D / 32;
  constexpr int NK = D / 16;
  constexpr int NSB = TK / 32;
  constexpr int NPV = NCC * NDB;
  constexpr int NOPS = NPV + NK * NSB;
  constexpr int PD = 3;
  const int h = lane >> 5;
  const int n = lane & 31;
  // V^T operands: rows 16*cc + 8*rr + 4*h + vi share the swizzle of row
  // 4*h + vi, so block db has one base and cc, rr are immediate offsets.
  const int vi = (lane & 15) >> 2;
  const int vq = lane & 3;
  const int vdh = (lane >> 4) & 1;
  uint32_t vbase[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int row = 4 * h + vi;
    const int pc = (4 * db + 2 * vdh + (vq >> 1)) ^ swz_v<CPR>(row);
    vbase[db] = va + opaque(row * ROWB + 16 * pc + 8 * (vq & 1));
  }
  // K operands: (ka + base of row 32*sb + n) ^ (32*kk); the ring slots are
  // 16 KB aligned, so adding the slot does not disturb the XORed bits.
  uint32_t kaddr[NSB];
#pragma unroll
  for (int sb = 0; sb < NSB; ++sb) {
    const int r = 32 * sb + n;
    kaddr[sb] = ka + opaque(r * ROWB + 16 * (h ^ swz_k<CPR>(r)));
  }
  bf16x8_t buf[PD + 1];
  auto load = [&](int i) __attribute__((always_inline)) {
    if (i < NPV) {
      const int cc = i / NDB, db = i % NDB;
      buf[i % (PD + 1)] = lds_tr_pair(vbase[db] + 16 * cc * ROWB, vbase[db] + (16 * cc + 8) * ROWB);
    } else {
      const int kk = (i - NPV) / NSB, sb = (i - NPV) % NSB;
      buf[i % (PD + 1)] = lds_b128(kaddr[sb] ^ (32 * kk));
    }
  };
  const f32x16_t zero = {};
#pragma unroll
  for (int i = 0; i < PD; ++i) load(i);
#pragma unroll
  for (int i = 0; i < NOPS; ++i) {
    if (i + PD < NOPS) load(i + PD);
    if (i < NPV) {
      const int cc = i / NDB, db = i % NDB;
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(buf[i % (PD + 1)], pb[cc], oacc[db], 0, 0, 0);
      if (db == 0) sum_weights_mfma(lacc, sel, pb[cc]);
    } else {
      const int kk = (i - NPV) / NSB, sb = (i - NPV) % NSB;
      sacc[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(buf[i % (PD + 1)], qf[kk], kk == 0 ? zero : sacc[sb],
                                                         0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Everything a workgroup needs before its tile loop.
template <int D>
struct Setup {
  KeyRows kr;
  int64_t kbeg;      // first key of this split
  int nst;           // tiles of this split
  bool computes;     // this wave owns packed rows (wave-uniform)
};

template <int D, int TK, int NW>
__device__ __forceinline__ Setup<D> setup(const AttnParams& p, int32_t* sidx, int wave) {
  Setup<D> s;
  const int tid = threadIdx.x;
  const int split = blockIdx.x;
  const int hkv = blockIdx.y / p.row_chunks;
  const int rc = blockIdx.y - hkv * p.row_chunks;
  const int b = blockIdx.z;
  const int R = p.group * p.block_len;
  const int t0 = (int)((int64_t)split * p.tiles / p.splits);
  const int t1 = (int)((int64_t)(split + 1) * p.tiles / p.splits);
  s.nst = t1 - t0;
  s.kbeg = (int64_t)t0 * TK;

  KeyRows& kr = s.kr;
  kr.kpre = (const char*)p.keys.k_pre + 2 * (b * p.keys.kp_sb + hkv * p.keys.kp_sh);
  kr.vpre = (const char*)p.keys.v_pre + 2 * (b * p.keys.vp_sb + hkv * p.keys.vp_sh);
  kr.kblk = (const char*)p.keys.k_blk + 2 * (b * p.keys.kb_sb + hkv * p.keys.kb_sh);
  kr.vblk = (const char*)p.keys.v_blk + 2 * (b * p.keys.vb_sb + hkv * p.keys.vb_sh);
  kr.kp_st = 2 * p.keys.kp_st, kr.vp_st = 2 * p.keys.vp_st;
  kr.kb_st = 2 * p.keys.kb_st, kr.vb_st = 2 * p.keys.vb_st;
  kr.n_pre = p.keys.n_pre;
  kr.n_all = p.keys.n_pre + p.keys.n_blk;
  kr.hole = p.keys.k_hole, kr.hole_len = p.keys.k_hole_len;
  kr.indexed = p.keys.idx != nullptr;
  kr.off32 = p.keys.off32 != 0;
  kr.gather32 = p.keys.gather32 != 0;

  // retained-row indices of this split's prefix keys, staged in LDS
  if (kr.indexed) {
    const int64_t lo = s.kbeg < kr.n_pre ? s.kbeg : kr.n_pre;
    const int64_t hi0 = s.kbeg + (int64_t)s.nst * TK;
    const int64_t hi = hi0 < kr.n_pre ? hi0 : kr.n_pre;
    const int32_t* src = p.keys.idx + ((int64_t)b * p.kv_heads + hkv) * kr.n_pre;
    for (int64_t j = lo + tid; j < hi; j += 64 * NW) {
      int64_t r = src[j];
      r = r < 0 ? 0 : (r >= p.keys.p_rows ? p.keys.p_rows - 1 : r);
      sidx[j - s.kbeg] = (int32_t)r;
    }
    __syncthreads();
  }
  s.computes = wave * 32 < p.rows_per_wg && rc * p.rows_per_wg + wave * 32 < R;
  return s;
}

// The query row a lane owns: packed row prow = g * Bq + qi of q-head hq,
// sequence row srow (through the row map) and its index mrow in the per-row
// arrays. Cheap to recompute, so it is not kept alive across the tile loop.
struct RowInfo {
  int b, hq, g, qi;
  int64_t srow, mrow;
  bool row_ok;
};

__device__ __forceinline__ RowInfo row_info(const AttnParams& p, int wave, int lane) {
  RowInfo ri;
  const int hkv = blockIdx.y / p.row_chunks;
  const int rc = blockIdx.y - hkv * p.row_chunks;
  ri.b = blockIdx.z;
  const int R = p.group * p.block_len;
  const int prow = rc * p.rows_per_wg + wave * 32 + (lane & 31);
  ri.row_ok = wave * 32 < p.rows_per_wg && prow < R;
  ri.g = 0, ri.qi = 0;
  if (ri.row_ok) {
    ri.g = prow / p.block_len;
    ri.qi = prow - ri.g * p.block_len;
  }
  ri.hq = hkv * p.group + ri.g;
  ri.srow = ri.qi + (ri.qi >= p.rows.q_hole ? p.rows.q_hole_len : 0);
  ri.mrow = ((int64_t)ri.b * p.q_heads + ri.hq) * p.rows.row_pitch + ri.srow;
  return ri;
}

// Query fragment (B operand of S^T = K Q^T), resident for the loop.
template <int D>
__device__ __forceinline__ void load_q(bf16x8_t (&qf)[D / 16], const AttnParams& p, const RowInfo& s, int h) {
  const uint16_t* qrow = (const uint16_t*)p.q + s.b * p.q_sb + s.hq * p.q_sh + s.srow * p.q_st;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (s.row_ok) v = *(const uint4*)(qrow + 16 * kk + 8 * h);
    qf[kk] = __builtin_bit_cast(bf16x8_t, v);
  }
}

// Empty state, or the initial state from a cached partial (LaCache Appendix J:
// the running (m, l, O~) of a later step starts from the cache): O~ = l * o,
// m in base 2, l carried by the lanes of the first wave half. The cached o, m
// and l are loaded together and the empty-row test is applied afterwards as a
// select, so that no load waits for another (an empty row's o is ignored).
template <int D>
__device__ __forceinline__ void init_state(RowState<D>& st, const AttnParams& p, const RowInfo& s, int lane) {
  const int h = lane >> 5;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.oacc[db][r] = 0.0f;
  st.m2 = -INFINITY;
  st.mtrue = -INFINITY;
  st.lsum = 0.0f;
  if (p.init_m != nullptr && s.row_ok) {
    const float mi = p.init_m[s.mrow];
    const float li = p.init_l[s.mrow];
    const float* orow = p.init_o + s.mrow * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const float4 v = *(const float4*)(orow + 32 * db + 8 * r4 + 4 * h);
        st.oacc[db][4 * r4 + 0] = v.x;
        st.oacc[db][4 * r4 + 1] = v.y;
        st.oacc[db][4 * r4 + 2] = v.z;
        st.oacc[db][4 * r4 + 3] = v.w;
      }
    const bool live = mi > -INFINITY && li > 0.0f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.oacc[db][r] = live ? st.oacc[db][r] * li : 0.0f;
    if (live) {
      st.m2 = mi * kLog2e;
      st.mtrue = st.m2;
      st.lsum = h == 0 ? li : 0.0f;
    }
  }
  // The rounded-weight sum starts at 0; the finish adds the cached l, moved to
  // the final reference max (init_sum), so that no initial value of it has to
  // stay alive through the tile loop.
#pragma unroll
  for (int r = 0; r < 4; ++r) st.lacc[r] = 0.0f;
}

// The cached l of an initial state, moved from its reference max to the final
// one m2 (base 2): the rescales of the loop multiplied O~ by the product of
// exp2(m_old - m_new), which telescopes to exp2(m_init - m2).
__device__ __forceinline__ float init_sum(const AttnParams& p, const RowInfo& s, float m2) {
  if (p.init_m == nullptr) return 0.0f;
  const float mi = p.init_m[s.mrow];
  const float li = p.init_l[s.mrow];
  return mi > -INFINITY && li > 0.0f ? li * __builtin_amdgcn_exp2f(mi * kLog2e - m2) : 0.0f;
}

// Finish: o = O~ / l, L = m + ln l (natural-log units), to the final O + LSE,
// a caller's partial, or the split workspace. In the split workspace o is
// stored as fp16 times 2^(14 - k), where the row's largest |o| lies in
// [2^(k-1), 2^k): that element lands in [2^13, 2^14), below the fp16 range's
// end whatever the magnitude of V, and every element keeps an error of at
// most 2^-12 of the row's largest (fp16 rounding), far below the bf16
// rounding of the merged O. The inverse scale 2^(k - 14) goes with m and l.
// FM restricts the output modes compiled in (kFinishAny: all three, chosen at
// run time; kFinishSplit: the split workspace only; kFinishDirect: the final
// O or a caller's partial), for kernels whose registers cannot hold the code
// of all three.
constexpr int kFinishAny = 0, kFinishSplit = 1, kFinishDirect = 2;

template <int D, int FM = kFinishAny>
__device__ __forceinline__ void finish(const RowState<D>& st, const AttnParams& p, const RowInfo& s, int lane) {
  const int h = lane >> 5;
  const int mode = FM == kFinishSplit ? (int)kOutSplit : p.out.mode;
  const bool split = FM != kFinishDirect && mode == kOutSplit;
  const float ltot = pair_sum(st.lsum);
  // the sum of the rounded weights of this lane's query: its own register,
  // or that of lane l ^ 32 (which holds this query's)
  const float lown = st.lacc[0];
  const float lother = other_half(lown, lane);
  const float lhrun = lsum_lane_is_own(lane) ? lown : lother;
  float omax = 0.0f;  // largest |O~| of the row (both wave halves), split workspace only
  if (split) {
    float a = 0.0f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) a = fmaxf(a, fabsf(st.oacc[db][r]));
    omax = pair_max(a);
  }
  if (!s.row_ok) return;
  const float lhtot = lhrun + init_sum(p, s, st.m2);
  const bool live = ltot > 0.0f;
  const float inv = live ? 1.0f / lhtot : 0.0f;
  if (!split && mode == kOutFinal) {
    uint16_t* orow = (uint16_t*)p.out.o + s.b * p.out.o_sb + s.hq * p.out.o_sh + s.srow * p.out.o_st;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = 32 * db + 8 * r4 + 4 * h;
        const __bf16 v0 = (__bf16)(st.oacc[db][4 * r4 + 0] * inv);
        const __bf16 v1 = (__bf16)(st.oacc[db][4 * r4 + 1] * inv);
        const __bf16 v2 = (__bf16)(st.oacc[db][4 * r4 + 2] * inv);
        const __bf16 v3 = (__bf16)(st.oacc[db][4 * r4 + 3] * inv);
        uint2 w;
        w.x = (uint32_t)__builtin_bit_cast(uint16_t, v0) | ((uint32_t)__builtin_bit_cast(uint16_t, v1) << 16);
        w.y = (uint32_t)__builtin_bit_cast(uint16_t, v2) | ((uint32_t)__builtin_bit_cast(uint16_t, v3) << 16);
        *(uint2*)(orow + d0) = w;
      }
    if (p.out.lse != nullptr && h == 0)
      p.out.lse[s.mrow] = live ? (st.m2 + __log2f(ltot)) * kLn2 : -INFINITY;
  } else if (split) {
    const int64_t base =
        (int64_t)blockIdx.x * p.out.split_rows + ((int64_t)s.b * p.q_heads + s.hq) * p.block_len + s.qi;
    int k = __builtin_amdgcn_frexp_expf(omax * inv);  // the row's largest |o| is in [2^(k-1), 2^k)
    k = k < -100 ? -100 : k;
    const float sc = __builtin_ldexpf(inv, 14 - k);
    uint16_t* orow = (uint16_t*)p.out.po + base * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = 32 * db + 8 * r4 + 4 * h;
        const f32x2_t a = {st.oacc[db][4 * r4 + 0] * sc, st.oacc[db][4 * r4 + 1] * sc};
        const f32x2_t b = {st.oacc[db][4 * r4 + 2] * sc, st.oacc[db][4 * r4 + 3] * sc};
        uint2 w;
        w.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(a, f16x2_t));
        w.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(b, f16x2_t));
        *(uint2*)(orow + d0) = w;
      }
    if (h == 0) {
      // export the exact max: l is re-referenced from m2 to it
      p.out.pmls[base] = make_float4(live ? st.mtrue * kLn2 : -INFINITY,
                                     live ? ltot * __builtin_amdgcn_exp2f(st.m2 - st.mtrue) : 0.0f,
                                     __builtin_ldexpf(1.0f, k - 14), 0.0f);
    }
  } else {
    const int64_t base = s.mrow;
    float* orow = p.out.po + base * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = 32 * db + 8 * r4 + 4 * h;
        *(float4*)(orow + d0) = make_float4(st.oacc[db][4 * r4 + 0] * inv, st.oacc[db][4 * r4 + 1] * inv,
                                            st.oacc[db][4 * r4 + 2] * inv, st.oacc[db][4 * r4 + 3] * inv);
      }
    if (h == 0) {
      // export the exact max: l is re-referenced from m2 to it
      p.out.pm[base] = live ? st.mtrue * kLn2 : -INFINITY;
      p.out.pl[base] = live ? ltot * __builtin_amdgcn_exp2f(st.m2 - st.mtrue) : 0.0f;
    }
  }
}


// Wait until at most `ahead` later stages of this wave's DMAs are in flight
// (IPS instructions per stage).
template <int IPS, int NS>
__device__ __forceinline__ void wait_stage(int ahead) {
  if (NS >= 4 && ahead >= 2) wait_vm<(NS >= 4 ? 2 : 0) * IPS>();
  else if (NS >= 3 && ahead >= 1) wait_vm<(NS >= 3 ? 1 : 0) * IPS>();
  else wait_vm<0>();
}


// One to four row waves (up to 128 packed rows), or eight (225 to 256 rows):
// every wave runs scores, softmax and PV of a tile in turn, the K/V tiles of a
// stage stored together in a ring of NS stages, NS - 1 tiles in flight, one
// barrier per tile. The row waves issue the DMAs, each its share of every
// tile; with DMAW one more wave (wave NW, no rows) issues them all instead, so
// that a row wave never stalls behind the memory pipeline between its
// products.
template <int D, int NW, int TK, int NS, bool DMAW = false, bool NT = false, bool IDX = false>
__global__ __launch_bounds__(64 * (NW + DMAW)) void attn_bf16_kernel(const AttnParams p) {
  constexpr int TB = TK * D * 2;                       // bytes of a K (or V) tile
  constexpr int IPW = DMAW ? TB / 1024 : TB / 1024 / NW;  // DMA instructions per issuing wave per K (or V) tile
  static_assert(IPW >= 1 && (DMAW || IPW * NW * 1024 == TB), "every wave issues the same number of DMAs");
  static_assert(2 * IPW * (NS - 2) < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) char ring[NS * 2 * TB];
  __shared__ int32_t sidx[kIdxCap];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5;
  const int n = lane & 31;
  // the query and initial-state loads go first, so that their latency
  // overlaps that of the retained-index staging
  bf16x8_t qf[D / 16];
  RowState<D> st;
  {
    const RowInfo ri = row_info(p, wave, lane);
    load_q<D>(qf, p, ri, h);
    init_state<D>(st, p, ri, lane);
  }
  const Setup<D> s = setup<D, TK, NW + DMAW>(p, sidx, wave);
  const uint32_t ring_lds = lds_addr(ring);
  const bool issuer = !DMAW || wave == NW;  // wave-uniform
  auto issue = [&](int t) __attribute__((always_inline)) {
    const uint32_t slot = ring_lds + (t % NS) * 2 * TB;
    const int64_t key0 = s.kbeg + (int64_t)t * TK;
    if (DMAW) {
      dma_tile_all<D, TK, NT>(s.kr, false, key0, slot, lane, sidx, s.kbeg);
      dma_tile_all<D, TK, NT>(s.kr, true, key0, slot + TB, lane, sidx, s.kbeg);
    } else {
      dma_tile<D, TK, NW, IDX>(s.kr, false, key0, slot, wave, lane, sidx, s.kbeg);
      dma_tile<D, TK, NW, IDX>(s.kr, true, key0, slot + TB, wave, lane, sidx, s.kbeg);
    }
  };

  wait_vm<0>();  // the query fragment and initial state have landed before any DMA is counted
  const int nst = s.nst;
  const int npro = nst < NS - 1 ? nst : NS - 1;
  if (issuer)
    for (int t = 0; t < npro; ++t) issue(t);

  for (int t = 0; t < nst; ++t) {
    const int ahead = (nst - 1 - t) < (NS - 2) ? (nst - 1 - t) : (NS - 2);
    if (issuer) wait_stage<2 * IPW, NS>(ahead);
    tile_barrier();
    if (issuer && t + NS - 1 < nst) issue(t + NS - 1);
    if (!s.computes) continue;
    const char* kb = ring + (t % NS) * 2 * TB;
    f32x16_t sacc[TK / 32];
    bf16x8_t pb[TK / 16];
    tile_scores<D, TK>(sacc, kb, qf, n, h);
    tile_softmax<D, TK>(sacc, pb, st, p.scale_log2, s.kr.n_all - (s.kbeg + (int64_t)t * TK), lane);
    tile_pv<D, TK>(st.oacc, st.lacc, pb, kb + TB, lane);
  }
  finish<D>(st, p, row_info(p, wave, opaque(lane)), lane);
}

// Eight waves (at most 224 packed rows), ping-pong. Per tile t every wave runs
// an MFMA phase M(t) = {PV of tile t-1, scores of tile t} and a softmax phase
// X(t). Waves 0-3 run M(t) then X(t); waves 4-7 run one phase later, so at
// every moment each SIMD holds one wave in an MFMA phase and one in a softmax
// phase (wave w and w+4 share a SIMD). Two barriers per tile separate the
// phases: slot 2t holds M(t) of the leading half and X(t-1) of the lagging
// half, slot 2t+1 X(t) of the leading half and M(t) of the lagging half.
//
// K and V have rings of their own. K of tile t is read in M(t) (slots 2t and
// 2t+1), V of tile t in M(t+1) (slots 2t+2 and 2t+3); a DMA issued after the
// barrier that opens a slot may overwrite only ring slots whose last reader
// ran before that barrier.
//
// Wave 7 owns no rows and issues every DMA, two tiles ahead, in the order
// K0, V0, K1, V1, ...: K of tile t+2 after the barrier of slot 2t (into the
// ring slot of K(t-1), ring of three), V of tile t+2 after that of slot 2t+1
// (V(t-1) is still read in slot 2t+1, so the V ring has four slots). vmcnt
// counts the wave's loads in issue order, so the wait before the barrier of
// slot 2t leaves in flight only V(t), K(t+1) and V(t+1): K(t) and V(t-1) have
// landed. The wave waits until at most 47 loads are counted before each group
// of 16 so the count stays in the field's range. No computing wave waits
// behind the memory pipeline to issue a load.
//
// SO (the split workspace as output, chosen at launch) compiles in only that
// finish: a run-time choice among all three would keep values alive through
// the loop that the 256 VGPRs cannot hold.
template <int D, bool NT = false, bool SO = false>
__global__ __launch_bounds__(512) void attn_bf16_pp_kernel(const AttnParams p) {
  constexpr int NW = 8;
  constexpr int TK = 64;
  constexpr int NSK = 3;
  constexpr int NSV = 4;
  constexpr int AHEAD = 2;  // K and V tiles issued ahead of the one being read
  constexpr int TB = TK * D * 2;
  constexpr int IPW = TB / 1024;  // DMA instructions per K (or V) tile
  static_assert(3 * IPW + IPW <= 64, "three tiles in flight plus one group fit the vmcnt range");
  __shared__ __attribute__((aligned(1024))) char kring[NSK * TB];
  __shared__ __attribute__((aligned(1024))) char vring[NSV * TB];
  __shared__ int32_t sidx[kIdxCap];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5;
  const int n = lane & 31;
  const Setup<D> s = setup<D, TK, NW>(p, sidx, wave);
  bf16x8_t qf[D / 16];
  RowState<D> st;
  {
    const RowInfo ri = row_info(p, wave, lane);
    load_q<D>(qf, p, ri, h);
    init_state<D>(st, p, ri, lane);
  }

  const int T = s.nst;
  const uint32_t kring_lds = lds_addr(kring);
  const uint32_t vring_lds = lds_addr(vring);
  const bf16x8_t lsel = lsum_selector(lane);
  const bool issuer = wave == NW - 1;  // wave-uniform; the launch leaves it without rows
  // (issuer only) cl: the contiguous path's lane offsets, computed once
  auto issue_tile = [&](bool isv, int tt, const ContigLanes<D, TK>& cl) __attribute__((always_inline)) {
    if (tt < 0 || tt >= T) return;
    const int64_t key0 = s.kbeg + (int64_t)tt * TK;
    const uint32_t dst = isv ? vring_lds + (tt % NSV) * TB : kring_lds + (tt % NSK) * TB;
    wait_vm<63 - IPW>();
    dma_tile_all_pre<D, TK, NT>(s.kr, isv, key0, dst, lane, sidx, s.kbeg, cl);
  };

  f32x16_t sacc[TK / 32];
  bf16x8_t pb[TK / 16];
  // M(t): PV of tile t-1 (t >= 1) and scores of tile t (t < T). The first and
  // last tiles are peeled out of the loops, whose bodies run the pipelined
  // two-part form.
  auto m_first = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    tile_scores<D, TK>(sacc, kring, qf, n, h);
    __builtin_amdgcn_s_setprio(0);
  };
  auto m_mid = [&](int t) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    mfma_phase_both<D, TK>(st.oacc, pb, vring_lds + ((t - 1) % NSV) * TB, sacc, kring_lds + (t % NSK) * TB, qf,
                           lane, st.lacc, lsel);
    __builtin_amdgcn_s_setprio(0);
  };
  auto m_last = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    tile_pv<D, TK>(st.oacc, st.lacc, pb, vring + ((T - 1) % NSV) * TB, lane);
    __builtin_amdgcn_s_setprio(0);
  };
  auto x_phase = [&](int t) __attribute__((always_inline)) {
    tile_softmax<D, TK>(sacc, pb, st, p.scale_log2, s.kr.n_all - (s.kbeg + (int64_t)t * TK), lane);
  };

  // Slot 2t opens with M(t) of the leading half, which reads K of tile t and
  // V of tile t-1. The issuer waits until only the loads issued after K(t)
  // remain (V(t), K(t+1), V(t+1), those that exist), barrier, then K of tile
  // t+2 is issued. Slot 2t+1: barrier, then V of tile t+2. The issuing wave
  // runs this barrier sequence in a loop of its own, so the computing waves
  // carry no DMA code (and no registers for it).
  using Issue = std::integral_constant<bool, true>;
  using NoIssue = std::integral_constant<bool, false>;
  auto even_slot = [&](int t, auto issue, const auto& cl) __attribute__((always_inline)) {
    if constexpr (decltype(issue)::value)
      wait_at_most<3 * IPW, 2 * IPW, IPW, 0>(IPW * ((t < T ? 1 : 0) + (t + 1 < T ? 2 : 0)));
    tile_barrier();
    if constexpr (decltype(issue)::value) issue_tile(false, t + AHEAD, cl);
  };
  auto odd_slot = [&](int t, auto issue, const auto& cl) __attribute__((always_inline)) {
    tile_barrier();
    if constexpr (decltype(issue)::value) issue_tile(true, t + AHEAD, cl);
  };
  const bool work = s.computes && T > 0;  // wave-uniform
  const int none = 0;                      // the computing waves pass no lane offsets
  if (issuer) {
    const ContigLanes<D, TK> cl = contig_lanes<D, TK>(lane);
    wait_vm<0>();  // nothing of this wave's own is counted with the DMAs
    for (int tt = 0; tt < AHEAD; ++tt) {
      issue_tile(false, tt, cl);
      issue_tile(true, tt, cl);
    }
    for (int t = 0; t <= T; ++t) {
      even_slot(t, Issue{}, cl);
      odd_slot(t, Issue{}, cl);
    }
  } else if (wave < NW / 2) {
    // leading half: M(t) in slot 2t, X(t) in slot 2t+1
    even_slot(0, NoIssue{}, none);
    if (work) m_first();
    odd_slot(0, NoIssue{}, none);
    if (work) x_phase(0);
    for (int t = 1; t < T; ++t) {
      even_slot(t, NoIssue{}, none);
      if (work) m_mid(t);
      odd_slot(t, NoIssue{}, none);
      if (work) x_phase(t);
    }
    if (T > 0) {
      even_slot(T, NoIssue{}, none);
      if (work) m_last();
      odd_slot(T, NoIssue{}, none);
    }
  } else {
    // lagging half: X(t-1) in slot 2t, M(t) in slot 2t+1
    even_slot(0, NoIssue{}, none);
    odd_slot(0, NoIssue{}, none);
    if (work) m_first();
    for (int t = 1; t < T; ++t) {
      even_slot(t, NoIssue{}, none);
      if (work) x_phase(t - 1);
      odd_slot(t, NoIssue{}, none);
      if (work) m_mid(t);
    }
    if (T > 0) {
      even_slot(T, NoIssue{}, none);
      if (work) x_phase(T - 1);
      odd_slot(T, NoIssue{}, none);
      if (work) m_last();
    }
  }
  finish<D, SO ? kFinishSplit : kFinishDirect>(st, p, row_info(p, wave, opaque(lane)), lane);
}

// Launch shapes: NW waves per workgroup (each 32 packed rows), TK keys per
// tile, NS ring stages.
template <int D, int NW>
hipError_t launch_d_nw(const AttnParams& p, hipStream_t stream, KernelEvents ev) {
  dim3 grid(p.splits, p.kv_heads * p.row_chunks, p.batch);
  const bool nt = p.keys.stream_nt != 0;  // a dense prefix longer than the last-level cache
  if constexpr (NW == 1) {
    // one row wave: a second wave issues the DMAs, so that the row wave never
    // stalls behind the memory pipeline, and so that the first tiles are
    // requested while the row wave's query and initial state are in flight
    if (nt)
      hipExtLaunchKernelGGL((attn_bf16_kernel<D, 1, 32, 4, true, true>), grid, dim3(128), 0, stream, ev.start,
                            ev.stop, 0, p);
    else
      hipExtLaunchKernelGGL((attn_bf16_kernel<D, 1, 32, 4, true>), grid, dim3(128), 0, stream, ev.start, ev.stop, 0,
                            p);
  } else if (NW == 8 && p.rows_per_wg <= 32 * (NW - 1)) {
    const bool so = p.out.mode == kOutSplit;
    if (nt && so)
      hipExtLaunchKernelGGL((attn_bf16_pp_kernel<D, true, true>), grid, dim3(512), 0, stream, ev.start, ev.stop, 0,
                            p);
    else if (nt)
      hipExtLaunchKernelGGL((attn_bf16_pp_kernel<D, true>), grid, dim3(512), 0, stream, ev.start, ev.stop, 0, p);
    else if (so)
      hipExtLaunchKernelGGL((attn_bf16_pp_kernel<D, false, true>), grid, dim3(512), 0, stream, ev.start, ev.stop, 0,
                            p);
    else
      hipExtLaunchKernelGGL((attn_bf16_pp_kernel<D>), grid, dim3(512), 0, stream, ev.start, ev.stop, 0, p);
  } else {
    constexpr int TK = 64;
    constexpr int NS = 4;
    if (p.keys.idx != nullptr)  // retained rows: the gathered form of each wave's DMA share
      hipExtLaunchKernelGGL((attn_bf16_kernel<D, NW, TK, NS, false, false, true>), grid, dim3(64 * NW), 0, stream,
                            ev.start, ev.stop, 0, p);
    else
      hipExtLaunchKernelGGL((attn_bf16_kernel<D, NW, TK, NS>), grid, dim3(64 * NW), 0, stream, ev.start, ev.stop,
                            0, p);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnParams& p, int waves, hipStream_t stream, KernelEvents ev) {
  switch (waves) {
    case 1: return launch_d_nw<D, 1>(p, stream, ev);
    case 2: return launch_d_nw<D, 2>(p, stream, ev);
    case 4: return launch_d_nw<D, 4>(p, stream, ev);
    case 8: return launch_d_nw<D, 8>(p, stream, ev);
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

hipError_t launch_attn_bf16(const AttnParams& p, int waves, hipStream_t stream, KernelEvents ev) {
  if (p.head_dim == 128) return launch_d<128>(p, waves, stream, ev);
  if (p.head_dim == 64) return launch_d<64>(p, waves, stream, ev);
  return hipErrorInvalidValue;
}

}  // namespace blkattn
