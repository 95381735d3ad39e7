// Attention mass of the prefix keys and selection of the retained rows, for
// gfx950.
//
// Sparse-dLLM (abstract, on the aitopics "kv state" tag page) keeps the
// critical tokens of the cache and evicts the rest, guided by attention. The
// plainest score of a prefix key under that reading is the attention
// probability it receives, summed over the queries that read it: for kv head
// h, over the G q-heads of its group and the Bq block queries,
//
//     mass[b, h, j] = sum_{g, i} exp(s_{g,i,j} - LSE_{g,i}),   s = scale <q, k_j>,
//
// with the row LSE over all keys of the row ([prefix; block], as returned by
// blkattn_full). The retained set is then the n_keep keys of largest mass,
// listed in ascending row order, the index layout the fused gather expects.
//
// mass: scores by MFMA as in the attention kernel (S^T = K Q^T, bf16 in, fp32
// out), p = exp2(s * scale * log2 e - LSE * log2 e), then a column sum over the
// 32 query rows of each wave (a transposing halving reduction across lanes:
// 31 lane exchanges turn 32 registers x 32 lanes into one column total per
// lane) and over the waves in a fixed order (no floating-point atomics: the
// result is bitwise reproducible).
//
// selection: one workgroup per (batch, kv head); a most-significant-digit
// radix select over the fp32 bit patterns (non-negative floats order like
// their bits) finds the n_keep-th largest value T, then an ordered compaction
// takes every key above T and the lowest-indexed keys equal to T.
#include "gfx950.h"
#include "launch.h"

#include <math.h>

namespace blkattn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2eM = 1.442695040888963407f;
constexpr int kMassWaves = 8;
constexpr int kMassTile = 64;

template <int CPR>
__device__ __forceinline__ int mswz(int r) {
  return CPR == 16 ? (r & 15) : ((r ^ (r >> 3)) & 7);
}

// bf16: one workgroup of 8 waves per (key split, batch * kv head) and pass of
// up to 32 * 8 * RBW packed rows; wave w owns the 32-row blocks w, w + 8, ...
// (RBW of them) of the pass. Scores come out as S = Q K^T (query rows in the
// M dimension of v_mfma_f32_32x32x16_bf16, keys in N), so a lane holds one key
// column: its 16 accumulator registers are 16 of the block's rows, and the
// column sum is an in-register sum plus one exchange between the wave halves.
// Each K fragment read from LDS feeds every row block of the wave.
//
// The two halves of the workgroup run half a tile apart (waves w and w + 4
// share a SIMD): per 64-key tile u a wave runs an MFMA phase M(u) (the scores)
// and a vector phase X(u) (the exponentials and this wave's column sums into
// LDS); waves 0-3 run M(u) in slot 2u and X(u) in slot 2u+1, waves 4-7 one
// slot later, so each SIMD has one wave on the matrix cores while the other
// is on the vector ALU. Wave 0 adds the eight waves' column sums of tile u in
// slot 2u+3, in wave order, and writes the mass. K tiles stream into a ring of
// four LDS slots through direct-to-LDS DMA, three tiles ahead, issued by waves
// 6 and 7 (half of each tile each) right after the barrier that opens an even
// slot; each waits for its half of tile u before the barrier that opens slot
// 2u, the first phase that reads it.
template <int D, int RBW>
__global__ __launch_bounds__(64 * kMassWaves) void mass_bf16_kernel(const MassParams p) {
  constexpr int NW = kMassWaves, TK = kMassTile;
  constexpr int ROWB = D * 2;
  constexpr int CPR = ROWB / 16;
  constexpr int RPI = 1024 / ROWB;  // K rows per DMA instruction
  constexpr int TB = TK * ROWB;     // bytes of a K tile
  constexpr int NSB = TK / 32;
  constexpr int KPB = D / 16;
  constexpr int NS = 4;             // K ring slots
  constexpr int KA = NS - 1;        // tiles issued ahead of the one being read
  constexpr int NI = 2;             // issuing waves
  constexpr int IPW = TB / 1024 / NI;
  static_assert(IPW * NI * 1024 == TB && KA * IPW < 64, "DMA split");
  __shared__ __attribute__((aligned(1024))) char kring[NS * TB];
  __shared__ float red[2][NW][TK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int n = lane & 31;
  const int split = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / p.kv_heads;
  const int hkv = bh - b * p.kv_heads;
  const int t0 = (int)((int64_t)split * p.tiles / p.splits);
  const int t1 = (int)((int64_t)(split + 1) * p.tiles / p.splits);
  const int T = t1 - t0;
  const float c2 = p.scale_log2;

  // A-operand query fragments (row n of each block) and, for the 16 rows the
  // accumulator registers hold (row 8 (r / 4) + 4 h + r % 4 of the block),
  // -LSE in base 2; rows past the pass get -inf, so their weights are exactly 0
  bf16x8_t qf[RBW][KPB];
  float nl2[RBW][16];
  bool has[RBW];
  auto row_of = [&](int prow, int& hq, int& qi) __attribute__((always_inline)) {
    const int g = prow / p.block_len;
    qi = prow - g * p.block_len;
    hq = hkv * p.group + g;
  };
#pragma unroll
  for (int j = 0; j < RBW; ++j) {
    const int rb0 = p.row0 + 32 * (wave + NW * j);  // first packed row of the block
    has[j] = rb0 < p.row_end;                        // wave-uniform
    {
      const int prow = rb0 + n;
      const bool ok = prow < p.row_end;
      int hq = 0, qi = 0;
      if (ok) row_of(prow, hq, qi);
      const uint16_t* qrow = (const uint16_t*)p.q + b * p.q_sb + hq * p.q_sh + qi * p.q_st;
#pragma unroll
      for (int kk = 0; kk < KPB; ++kk) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (ok) v = *(const uint4*)(qrow + 16 * kk + 8 * h);
        qf[j][kk] = __builtin_bit_cast(bf16x8_t, v);
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int prow = rb0 + 8 * (r >> 2) + 4 * h + (r & 3);
      float v = -INFINITY;
      if (prow < p.row_end) {
        int hq, qi;
        row_of(prow, hq, qi);
        v = -p.lse[((int64_t)b * p.q_heads + hq) * p.block_len + qi] * kLog2eM;
      }
      nl2[j][r] = v;
    }
  }

  // K tile u (keys (t0 + u) * TK ..) into ring slot u % NS: issuing wave i
  // fills instructions i*IPW .. i*IPW + IPW - 1, RPI rows each, lane l the
  // LDS chunk l % CPR of its row with logical chunk (l % CPR) ^ swizzle(row).
  // Rows past the prefix read its last row (their mass is never written).
  const char* kbase = (const char*)p.k + 2 * ((int64_t)b * p.k_sb + (int64_t)hkv * p.k_sh);
  const int64_t kst = 2 * p.k_st;
  const bool issuer = wave >= NW - NI;  // wave-uniform
  const int k0 = (wave - (NW - NI)) * IPW;
  const uint32_t kring_lds = lds_addr(kring);
  auto issue = [&](int u) __attribute__((always_inline)) {
    if (u >= T) return;
    const uint32_t dst = kring_lds + (u % NS) * TB;
    const int64_t key0 = (int64_t)(t0 + u) * TK;
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int k = k0 + j;
      const int r = k * RPI + lane / CPR;
      int64_t key = key0 + r;
      key = key < p.n_keys ? key : p.n_keys - 1;
      const int lc = (lane % CPR) ^ mswz<CPR>(r);
      dma_1k(kbase + key * kst + 16 * lc, dst + k * 1024);
    }
  };
  // DMA instructions of this issuer for the tiles of [a, b] that exist
  auto insts = [&](int a, int bb) __attribute__((always_inline)) {
    const int lo = a > 0 ? a : 0;
    const int hi = bb < T - 1 ? bb : T - 1;
    return hi >= lo ? (hi - lo + 1) * IPW : 0;
  };

  f32x16_t sacc[RBW][NSB];
  auto m_phase = [&](int u) __attribute__((always_inline)) {
    const char* kb = kring + (u % NS) * TB;
#pragma unroll
    for (int j = 0; j < RBW; ++j)
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[j][sb][r] = 0.0f;
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kk = 0; kk < KPB; ++kk)
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
        const int krow = 32 * sb + n;
        const uint4 a = *(const uint4*)(kb + krow * ROWB + 16 * ((2 * kk + h) ^ mswz<CPR>(krow)));
#pragma unroll
        for (int j = 0; j < RBW; ++j)
          if (has[j])
            sacc[j][sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[j][kk], __builtin_bit_cast(bf16x8_t, a),
                                                                  sacc[j][sb], 0, 0, 0);
      }
    __builtin_amdgcn_s_setprio(0);
  };
  // column sums: key 32 sb + n over this wave's rows, fixed order (j, r)
  auto x_phase = [&](int u) __attribute__((always_inline)) {
    float cs[NSB];
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
      float acc = 0.0f;
#pragma unroll
      for (int j = 0; j < RBW; ++j)
        if (has[j]) {
#pragma unroll
          for (int r = 0; r < 16; ++r) acc += __builtin_amdgcn_exp2f(fmaf(sacc[j][sb][r], c2, nl2[j][r]));
        }
      cs[sb] = acc + __shfl_xor(acc, 32);  // the other half's 16 rows of each block
    }
    if (h == 0) {
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) red[u & 1][wave][32 * sb + n] = cs[sb];
    }
  };
  float* mrow = p.mass + ((int64_t)b * p.kv_heads + hkv) * p.n_keys;
  auto reduce = [&](int u) __attribute__((always_inline)) {
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) sum += red[u & 1][w][lane];
    const int64_t key = (int64_t)(t0 + u) * TK + lane;
    if (key < p.n_keys) mrow[key] = p.accumulate ? mrow[key] + sum : sum;
  };

  wait_vm<0>();  // the query fragments have landed before any DMA is counted
  if (issuer)
    for (int u = 0; u < KA; ++u) issue(u);
  // slot 2u: the issuers wait for their halves of tile u, barrier, issue
  // tile u + KA; slot 2u + 1: barrier
  auto even_slot = [&](int u) __attribute__((always_inline)) {
    if (issuer) wait_at_most<(KA - 1) * IPW, IPW, 0>(insts(u + 1, u + KA - 1));
    tile_barrier();
    if (issuer) issue(u + KA);
  };
  if (wave < NW / 2) {
    // leading half: M(u) in slot 2u, X(u) in slot 2u + 1; wave 0 reduces
    // tile u - 1 in slot 2u + 1
    for (int u = 0; u <= T; ++u) {
      even_slot(u);
      if (u < T) m_phase(u);
      tile_barrier();
      if (u < T) x_phase(u);
      if (wave == 0 && u >= 1) reduce(u - 1);
    }
  } else {
    // lagging half: X(u - 1) in slot 2u, M(u) in slot 2u + 1
    for (int u = 0; u <= T; ++u) {
      even_slot(u);
      if (u >= 1) x_phase(u - 1);
      tile_barrier();
      if (u < T) m_phase(u);
    }
  }
}

// fp32: one thread per prefix key, looping over the packed rows.
template <int D>
__global__ __launch_bounds__(64) void mass_f32_kernel(const MassParams p) {
  const int bh = blockIdx.y;
  const int b = bh / p.kv_heads;
  const int hkv = bh - b * p.kv_heads;
  const int64_t key = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (key >= p.n_keys) return;
  const float* krow = (const float*)p.k + (int64_t)b * p.k_sb + (int64_t)hkv * p.k_sh + key * p.k_st;
  float kr[D];
#pragma unroll
  for (int d = 0; d < D; ++d) kr[d] = krow[d];
  float acc = 0.0f;
  for (int g = 0; g < p.group; ++g) {
    const int hq = hkv * p.group + g;
    for (int i = 0; i < p.block_len; ++i) {
      const float* qrow = (const float*)p.q + (int64_t)b * p.q_sb + (int64_t)hq * p.q_sh + (int64_t)i * p.q_st;
      float s = 0.0f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = fmaf(qrow[d], kr[d], s);
      acc += expf(s * p.scale - p.lse[((int64_t)b * p.q_heads + hq) * p.block_len + i]);
    }
  }
  p.mass[((int64_t)b * p.kv_heads + hkv) * p.n_keys + key] = acc;
}

// Selection of the n_keep largest masses of each (batch, kv head), ties to the
// lower index, written in ascending index order. Masses are finite and >= 0,
// so their bit patterns (with -0 folded onto +0) order like the values. An
// exact radix select finds the n_keep-th largest pattern T, 8 bits per pass from
// the top; every pass spreads each group's row over `chunks` workgroups that
// write per-chunk histograms, and each workgroup of the next pass sums those
// histograms to find the digit itself. A count pass and an ordered write pass
// then emit the rows above T and the lowest-indexed rows equal to T.
//
// Workspace (uint32): hist [4][G][C][256], counts [G][C][2], state [5][G][2]
// with state[p] = (prefix of T fixed before pass p, rows still to take among
// those matching it); state[4] = (T, ties taken).
constexpr int kSelThreads = 256;
constexpr int kSelMaxChunks = 32;
constexpr int kSelBatch = 16;  // rows per thread loaded before any is used

// Rows base + i * kSelThreads + threadIdx.x (i < kSelBatch) of a group's
// masses below `end`, as ordered keys; rows at or past `end` read as 0.
__device__ __forceinline__ void sel_load(const uint32_t* row, int64_t base, int64_t end, uint32_t* xs) {
#pragma unroll
  for (int i = 0; i < kSelBatch; ++i) {
    const int64_t j = base + (int64_t)i * kSelThreads + threadIdx.x;
    xs[i] = j < end ? row[j] : 0u;
  }
#pragma unroll
  for (int i = 0; i < kSelBatch; ++i) xs[i] = xs[i] == 0x80000000u ? 0u : xs[i];
}

struct SelParams {
  const uint32_t* bits;  // [G, n]
  int32_t* idx;          // [G, k]
  uint32_t* hist;
  uint32_t* counts;
  uint32_t* state;
  int64_t n, k, chunk;
  int groups, chunks;
};

// From the previous pass's state and its per-chunk histograms, the digit of T
// at `shift` and the state after it. Every thread returns the same values.
__device__ void sel_derive(const SelParams& p, int g, int pass_prev, uint32_t prev_prefix, uint32_t prev_need,
                           uint32_t* s_bins, uint32_t* s_out, uint32_t& prefix, uint32_t& need) {
  const int tid = threadIdx.x;
  if (tid == 0) {  // kept only if the masses break the precondition
    s_out[0] = prev_prefix;
    s_out[1] = prev_need;
  }
  const uint32_t* h = p.hist + ((int64_t)pass_prev * p.groups + g) * p.chunks * 256;
  // every chunk's bin in flight at once (clamped indices keep the loads in
  // bounds and the code straight-line), then summed in chunk order
  uint32_t hv[kSelMaxChunks];
#pragma unroll
  for (int ch = 0; ch < kSelMaxChunks; ++ch) hv[ch] = h[(ch < p.chunks ? ch : p.chunks - 1) * 256 + tid];
  uint32_t c = 0;
#pragma unroll
  for (int ch = 0; ch < kSelMaxChunks; ++ch) c += ch < p.chunks ? hv[ch] : 0u;
  s_bins[tid] = c;
  __syncthreads();
  // inclusive suffix sums: s_bins[t] = rows whose digit is >= t
  for (int off = 1; off < 256; off <<= 1) {
    const uint32_t add = tid + off < 256 ? s_bins[tid + off] : 0u;
    __syncthreads();
    s_bins[tid] += add;
    __syncthreads();
  }
  const uint32_t incl = s_bins[tid];
  const uint32_t above = incl - c;
  if (above < prev_need && prev_need <= incl) {
    s_out[0] = prev_prefix | ((uint32_t)tid << (24 - 8 * pass_prev));
    s_out[1] = prev_need - above;
  }
  __syncthreads();
  prefix = s_out[0];
  need = s_out[1];
}

__global__ __launch_bounds__(kSelThreads) void select_hist_kernel(SelParams p, int pass) {
  __shared__ uint32_t s_hist[256];
  __shared__ uint32_t s_bins[256];
  __shared__ uint32_t s_out[2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int c = blockIdx.x, g = blockIdx.y;
  if (p.k >= p.n) return;
  const uint32_t* row = p.bits + (int64_t)g * p.n;
  const int64_t j0 = (int64_t)c * p.chunk;
  const int64_t j1 = j0 + p.chunk < p.n ? j0 + p.chunk : p.n;
  uint32_t xs[kSelBatch];
  sel_load(row, j0, j1, xs);  // in flight while the digit so far is derived
  uint32_t prefix = 0, need = (uint32_t)p.k;
  if (pass > 0) {
    uint32_t pp = 0, pn = (uint32_t)p.k;
    if (pass > 1) {
      pp = p.state[((pass - 1) * p.groups + g) * 2];
      pn = p.state[((pass - 1) * p.groups + g) * 2 + 1];
    }
    sel_derive(p, g, pass - 1, pp, pn, s_bins, s_out, prefix, need);
    if (c == 0 && tid == 0) {
      p.state[(pass * p.groups + g) * 2] = prefix;
      p.state[(pass * p.groups + g) * 2 + 1] = need;
    }
  }
  s_hist[tid] = 0;
  __syncthreads();
  const int shift = 24 - 8 * pass;
  const uint32_t hmask = pass == 0 ? 0u : (0xffffffffu << (shift + 8));
  for (int64_t base = j0; base < j1; base += (int64_t)kSelThreads * kSelBatch) {
    if (base != j0) sel_load(row, base, j1, xs);
#pragma unroll
    for (int i = 0; i < kSelBatch; ++i) {
      const int64_t j = base + (int64_t)i * kSelThreads + tid;
      const uint32_t x = xs[i];
      const bool m = j < j1 && (x & hmask) == prefix;
      const uint32_t dg = (x >> shift) & 255u;
      // the wave's most common case (all rows in one bin) becomes a single atomic
      const uint64_t act = __ballot(m);
      if (act != 0) {
        const int lead = __ffsll((unsigned long long)act) - 1;
        const uint32_t d0 = __shfl(dg, lead);
        const bool same = m && dg == d0;
        const uint64_t smask = __ballot(same);
        if (same) {
          if (lane == lead) atomicAdd(&s_hist[d0], (uint32_t)__popcll(smask));
        } else if (m) {
          atomicAdd(&s_hist[dg], 1u);
        }
      }
    }
  }
  __syncthreads();
  p.hist[(((int64_t)pass * p.groups + g) * p.chunks + c) * 256 + tid] = s_hist[tid];
}

__global__ __launch_bounds__(kSelThreads) void select_count_kernel(SelParams p) {
  __shared__ uint32_t s_bins[256];
  __shared__ uint32_t s_out[2];
  __shared__ uint32_t s_red[2][kSelThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x, g = blockIdx.y;
  if (p.k >= p.n) return;
  const uint32_t* row = p.bits + (int64_t)g * p.n;
  const int64_t j0 = (int64_t)c * p.chunk;
  const int64_t j1 = j0 + p.chunk < p.n ? j0 + p.chunk : p.n;
  uint32_t xs[kSelBatch];
  sel_load(row, j0, j1, xs);  // in flight while T is derived
  uint32_t T, ties;
  sel_derive(p, g, 3, p.state[(3 * p.groups + g) * 2], p.state[(3 * p.groups + g) * 2 + 1], s_bins, s_out, T,
             ties);
  if (c == 0 && tid == 0) {
    p.state[(4 * p.groups + g) * 2] = T;
    p.state[(4 * p.groups + g) * 2 + 1] = ties;
  }
  uint32_t gt = 0, eq = 0;
  for (int64_t base = j0; base < j1; base += (int64_t)kSelThreads * kSelBatch) {
    if (base != j0) sel_load(row, base, j1, xs);
#pragma unroll
    for (int i = 0; i < kSelBatch; ++i) {
      const bool in = base + (int64_t)i * kSelThreads + tid < j1;
      gt += in && xs[i] > T ? 1u : 0u;
      eq += in && xs[i] == T ? 1u : 0u;
    }
  }
  for (int off = 32; off >= 1; off >>= 1) {
    gt += __shfl_xor(gt, off);
    eq += __shfl_xor(eq, off);
  }
  if (lane == 0) {
    s_red[0][wave] = gt;
    s_red[1][wave] = eq;
  }
  __syncthreads();
  if (tid < 2) {
    uint32_t t = 0;
    for (int w = 0; w < kSelThreads / 64; ++w) t += s_red[tid][w];
    p.counts[((int64_t)g * p.chunks + c) * 2 + tid] = t;
  }
}

__global__ __launch_bounds__(kSelThreads) void select_write_kernel(SelParams p) {
  constexpr int NW = kSelThreads / 64;
  __shared__ uint32_t s_w[2][2][NW];  // [parity][gt, eq][wave]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = blockIdx.x, g = blockIdx.y;
  int32_t* out = p.idx + (int64_t)g * p.k;
  const int64_t j0 = (int64_t)c * p.chunk;
  const int64_t j1 = j0 + p.chunk < p.n ? j0 + p.chunk : p.n;
  if (p.k >= p.n) {  // every row is kept
    for (int64_t j = j0 + tid; j < j1; j += kSelThreads) out[j] = (int32_t)j;
    return;
  }
  const uint32_t* row = p.bits + (int64_t)g * p.n;
  uint32_t xs[kSelBatch];
  sel_load(row, j0, j1, xs);
  const uint32_t T = p.state[(4 * p.groups + g) * 2];
  const int64_t ties = p.state[(4 * p.groups + g) * 2 + 1];
  // rows above T and equal to T in the chunks before this one: every count in
  // flight at once (clamped, straight-line), summed in chunk order
  uint2 cv[kSelMaxChunks];
#pragma unroll
  for (int ch = 0; ch < kSelMaxChunks; ++ch)
    cv[ch] = *(const uint2*)(p.counts + ((int64_t)g * p.chunks + (ch < c ? ch : 0)) * 2);
  int64_t gt_before = 0, eq_before = 0;
#pragma unroll
  for (int ch = 0; ch < kSelMaxChunks; ++ch)
    if (ch < c) gt_before += cv[ch].x, eq_before += cv[ch].y;
  auto clamp_take = [](int64_t avail, int64_t cnt) -> int64_t {  // min(max(avail, 0), cnt)
    return avail <= 0 ? 0 : (avail < cnt ? avail : cnt);
  };
  int64_t pos_run = gt_before + clamp_take(ties, eq_before);  // rows taken in earlier chunks
  int64_t eq_run = eq_before;                                  // rank of the next row equal to T
  const uint64_t lt = (1ull << lane) - 1ull;
  int it = 0;
  for (int64_t jb = j0; jb < j1; jb += kSelThreads, ++it) {
    const int bi = it % kSelBatch;
    if (bi == 0 && jb != j0) sel_load(row, jb, j1, xs);
    const int64_t j = jb + tid;
    const bool in = j < j1;
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < kSelBatch; ++i) x = i == bi ? xs[i] : x;  // register select, no scratch
    const bool gt = in && x > T;
    const bool eq = in && x == T;
    const uint64_t gm = __ballot(gt), em = __ballot(eq);
    const int par = it & 1;
    if (lane == 0) {
      s_w[par][0][wave] = (uint32_t)__popcll(gm);
      s_w[par][1][wave] = (uint32_t)__popcll(em);
    }
    __syncthreads();
    int64_t gt_pre = 0, eq_pre = 0, gt_tot = 0, eq_tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int64_t a = s_w[par][0][w], b = s_w[par][1][w];
      if (w < wave) gt_pre += a, eq_pre += b;
      gt_tot += a, eq_tot += b;
    }
    const int64_t eq_base = eq_run + eq_pre;  // rank of this wave's first row equal to T
    const int64_t eq_lane = __popcll(em & lt);
    const bool take = gt || (eq && eq_base + eq_lane < ties);
    if (take) {
      const int64_t pos = pos_run + gt_pre + clamp_take(ties - eq_run, eq_pre) + __popcll(gm & lt) +
                          clamp_take(ties - eq_base, eq_lane);
      if (pos < p.k) out[pos] = (int32_t)j;
    }
    pos_run += gt_tot + clamp_take(ties - eq_run, eq_tot);
    eq_run += eq_tot;
  }
}

template <int D>
hipError_t launch_mass_d(const MassParams& p0, hipStream_t stream) {
  const int R = p0.group * p0.block_len;
  constexpr int kPassRows = 32 * kMassWaves * 2;
  dim3 grid(p0.splits, p0.batch * p0.kv_heads);
  // passes over the packed rows run in order on the stream; later passes add
  // their column sums onto the earlier ones (fixed order: reproducible)
  for (int row0 = 0; row0 < R; row0 += kPassRows) {
    MassParams p = p0;
    p.row0 = row0;
    p.row_end = row0 + kPassRows < R ? row0 + kPassRows : R;
    p.accumulate = row0 > 0;
    if (p.row_end - row0 > 32 * kMassWaves)
      hipLaunchKernelGGL((mass_bf16_kernel<D, 2>), grid, dim3(64 * kMassWaves), 0, stream, p);
    else
      hipLaunchKernelGGL((mass_bf16_kernel<D, 1>), grid, dim3(64 * kMassWaves), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

int mass_tile_keys() { return kMassTile; }

hipError_t launch_mass(const MassParams& p, hipStream_t stream) {
  if (p.n_keys == 0 || p.batch == 0 || p.kv_heads == 0) return hipSuccess;
  if (p.dtype == 0) {
    dim3 grid((unsigned)((p.n_keys + 63) / 64), p.batch * p.kv_heads);
    if (p.head_dim == 64)
      hipLaunchKernelGGL(mass_f32_kernel<64>, grid, dim3(64), 0, stream, p);
    else if (p.head_dim == 128)
      hipLaunchKernelGGL(mass_f32_kernel<128>, grid, dim3(64), 0, stream, p);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  }
  if (p.head_dim == 128) return launch_mass_d<128>(p, stream);
  if (p.head_dim == 64) return launch_mass_d<64>(p, stream);
  return hipErrorInvalidValue;
}

SelectPlan select_plan(int64_t groups, int64_t n) {
  SelectPlan sp{1, n > 0 ? n : 1, 0};
  if (groups <= 0 || n <= 0) return sp;
  int64_t c = (n + 1023) / 1024;                 // chunks of at least 1024 rows
  const int64_t fill = (512 + groups - 1) / groups;  // about 256-512 workgroups in all
  if (c > fill) c = fill;
  if (c > kSelMaxChunks) c = kSelMaxChunks;
  if (c < 1) c = 1;
  int64_t chunk = (n + c - 1) / c;
  chunk = (chunk + kSelThreads - 1) / kSelThreads * kSelThreads;
  sp.chunk = chunk;
  sp.chunks = (int)((n + chunk - 1) / chunk);
  sp.ws_bytes = (size_t)(groups * sp.chunks * (4 * 256 + 2) + 5 * groups * 2) * sizeof(uint32_t);
  return sp;
}

hipError_t launch_select(const float* mass, int32_t* idx, void* ws, int64_t groups, int64_t n, int64_t k,
                         hipStream_t stream) {
  if (groups == 0 || k == 0 || n == 0) return hipSuccess;
  const SelectPlan sp = select_plan(groups, n);
  SelParams p;
  p.bits = reinterpret_cast<const uint32_t*>(mass);
  p.idx = idx;
  p.hist = static_cast<uint32_t*>(ws);
  p.counts = p.hist + groups * sp.chunks * 4 * 256;
  p.state = p.counts + groups * sp.chunks * 2;
  p.n = n, p.k = k, p.chunk = sp.chunk;
  p.groups = (int)groups, p.chunks = sp.chunks;
  const dim3 grid((unsigned)sp.chunks, (unsigned)groups);
  if (k < n) {
    for (int pass = 0; pass < 4; ++pass)
      hipLaunchKernelGGL(select_hist_kernel, grid, dim3(kSelThreads), 0, stream, p, pass);
    hipLaunchKernelGGL(select_count_kernel, grid, dim3(kSelThreads), 0, stream, p);
  }
  hipLaunchKernelGGL(select_write_kernel, grid, dim3(kSelThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace blkattn
