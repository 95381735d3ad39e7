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
#include "launch.h"

#include <math.h>

namespace blkattn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLog2eM = 1.442695040888963407f;
constexpr int kMassWaves = 8;
constexpr int kMassTile = 64;

template <int CPR>
__device__ __forceinline__ int mswz(int r) {
  return CPR == 16 ? (r & 15) : ((r ^ (r >> 3)) & 7);
}

// bf16: one workgroup of 8 waves per (key split, batch * kv head); wave w owns
// the 32-row blocks w, w + 8, ... (RBW of them) of the G * Bq packed rows.
template <int D, int RBW>
__global__ __launch_bounds__(64 * kMassWaves) void mass_bf16_kernel(const MassParams p) {
  constexpr int NW = kMassWaves, TK = kMassTile;
  constexpr int ROWB = D * 2;
  constexpr int CPR = ROWB / 16;
  constexpr int KBYTES = TK * ROWB;
  constexpr int CHUNKS = KBYTES / 16;           // 16-byte chunks per tile
  constexpr int CPT = CHUNKS / (64 * NW);       // chunks per thread
  constexpr int NSB = TK / 32;
  constexpr int KPB = D / 16;
  static_assert(CHUNKS % (64 * NW) == 0, "whole chunks per thread");
  __shared__ __attribute__((aligned(16))) char kbuf[2][KBYTES];
  __shared__ float red[NW][TK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int n = lane & 31;
  const int split = blockIdx.x;
  const int bh = blockIdx.y;
  const int b = bh / p.kv_heads;
  const int hkv = bh - b * p.kv_heads;
  const int R = p.group * p.block_len;
  const int t0 = (int)((int64_t)split * p.tiles / p.splits);
  const int t1 = (int)((int64_t)(split + 1) * p.tiles / p.splits);
  const float c2 = p.scale_log2;

  // query fragments and -LSE (base 2) of this wave's rows; rows past R get
  // -inf, so their weights are exactly 0
  bf16x8_t qf[RBW][KPB];
  float nl2[RBW];
  bool has[RBW];
#pragma unroll
  for (int j = 0; j < RBW; ++j) {
    const int rb = wave + NW * j;
    has[j] = 32 * rb < R;  // wave-uniform
    const int prow = 32 * rb + n;
    const bool ok = prow < R;
    const int g = ok ? prow / p.block_len : 0;
    const int qi = ok ? prow - g * p.block_len : 0;
    const int hq = hkv * p.group + g;
    const uint16_t* qrow = (const uint16_t*)p.q + b * p.q_sb + hq * p.q_sh + qi * p.q_st;
#pragma unroll
    for (int kk = 0; kk < KPB; ++kk) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (ok) v = *(const uint4*)(qrow + 16 * kk + 8 * h);
      qf[j][kk] = __builtin_bit_cast(bf16x8_t, v);
    }
    nl2[j] = ok ? -p.lse[((int64_t)b * p.q_heads + hq) * p.block_len + qi] * kLog2eM : -INFINITY;
  }

  // K tile t: thread tid stages chunks tid + 512 * i; rows past the prefix read
  // row 0 (their mass is never written)
  const char* kbase = (const char*)p.k + 2 * ((int64_t)b * p.k_sb + (int64_t)hkv * p.k_sh);
  const int64_t kst = 2 * p.k_st;
  uint4 stage[CPT];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + 64 * NW * i;
      const int row = c / CPR, ch = c - (c / CPR) * CPR;
      int64_t key = (int64_t)t * TK + row;
      key = key < p.n_keys ? key : 0;
      stage[i] = *(const uint4*)(kbase + key * kst + 16 * ch);
    }
  };
  auto store_tile = [&](int slot) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + 64 * NW * i;
      const int row = c / CPR, ch = c - (c / CPR) * CPR;
      *(uint4*)(kbuf[slot] + row * ROWB + 16 * (ch ^ mswz<CPR>(row))) = stage[i];
    }
  };

  // lane (h, n) ends the reduction with the column of register n: key
  const int kid = 32 * (n >> 4) + 8 * ((n & 15) >> 2) + 4 * h + (n & 3);
  float* mrow = p.mass + ((int64_t)b * p.kv_heads + hkv) * p.n_keys;

  if (t0 < t1) {
    load_tile(t0);
    store_tile(0);
  }
  __syncthreads();
  for (int t = t0; t < t1; ++t) {
    const int cur = (t - t0) & 1;
    if (t + 1 < t1) load_tile(t + 1);  // in flight while this tile is computed
    const char* kb = kbuf[cur];
    float acc = 0.0f;
#pragma unroll
    for (int j = 0; j < RBW; ++j) {
      if (!has[j]) continue;
      f32x16_t sacc[NSB];
#pragma unroll
      for (int sb = 0; sb < NSB; ++sb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[sb][r] = 0.0f;
        const int krow = 32 * sb + n;
#pragma unroll
        for (int kk = 0; kk < KPB; ++kk) {
          const uint4 a = *(const uint4*)(kb + krow * ROWB + 16 * ((2 * kk + h) ^ mswz<CPR>(krow)));
          sacc[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), qf[j][kk],
                                                             sacc[sb], 0, 0, 0);
        }
      }
      float v[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = __builtin_amdgcn_exp2f(fmaf(sacc[i >> 4][i & 15], c2, nl2[j]));
      // sum over the 32 rows (lanes n of this half): halve the register count
      // at every lane exchange; lane n keeps register n's column total
#pragma unroll
      for (int m = 16; m >= 1; m >>= 1) {
        const bool upper = (n & m) != 0;
#pragma unroll
        for (int i = 0; i < m; ++i) {
          const float send = upper ? v[i] : v[i + m];
          const float keep = upper ? v[i + m] : v[i];
          v[i] = keep + __shfl_xor(send, m);
        }
      }
      acc += v[0];
    }
    red[wave][kid] = acc;
    __syncthreads();  // red complete; every wave is done with kbuf[cur]
    if (wave == 0) {
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) s += red[w][lane];
      const int64_t key = (int64_t)t * TK + lane;
      if (key < p.n_keys) mrow[key] = s;
    }
    if (t + 1 < t1) store_tile(cur ^ 1);
    __syncthreads();  // next tile staged; red read
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

// Selection of the n_keep largest masses of one (batch, kv head), ties to the
// lower index, written in ascending index order.
constexpr int kSelThreads = 1024;

__global__ __launch_bounds__(kSelThreads) void select_kernel(const float* mass, int32_t* idx, int64_t n,
                                                             int64_t k) {
  __shared__ uint32_t hist[256];
  __shared__ int64_t scan[kSelThreads];
  __shared__ uint32_t s_prefix;
  __shared__ int64_t s_need;
  const int tid = threadIdx.x;
  const uint32_t* bits = (const uint32_t*)mass + (int64_t)blockIdx.x * n;
  int32_t* out = idx + (int64_t)blockIdx.x * k;
  if (k <= 0) return;
  if (k >= n) {  // everything is kept
    for (int64_t j = tid; j < n; j += kSelThreads) out[j] = (int32_t)j;
    return;
  }
  // radix select of the k-th largest bit pattern, 8 bits per pass from the top
  if (tid == 0) {
    s_prefix = 0;
    s_need = k;
  }
  __syncthreads();
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    const uint32_t prefix = s_prefix;
    const uint32_t hmask = shift == 24 ? 0u : (0xffffffffu << (shift + 8));
    for (int64_t j = tid; j < n; j += kSelThreads) {
      const uint32_t x = bits[j];
      if ((x & hmask) == prefix) atomicAdd(&hist[(x >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      int64_t need = s_need, above = 0;
      int dsel = 0;
      for (int dg = 255; dg >= 0; --dg) {
        if (above + hist[dg] >= need) {
          dsel = dg;
          break;
        }
        above += hist[dg];
      }
      s_prefix = prefix | ((uint32_t)dsel << shift);
      s_need = need - above;  // still to take among keys equal to the prefix so far
    }
    __syncthreads();
  }
  const uint32_t T = s_prefix;
  const int64_t ties_taken = s_need;  // keys equal to T that are kept: the lowest-indexed ones
  // ordered compaction: contiguous chunks per thread, two block scans
  const int64_t chunk = (n + kSelThreads - 1) / kSelThreads;
  const int64_t j0 = (int64_t)tid * chunk;
  const int64_t j1 = j0 + chunk < n ? j0 + chunk : n;
  int64_t ties = 0;
  for (int64_t j = j0; j < j1; ++j) ties += bits[j] == T ? 1 : 0;
  scan[tid] = ties;
  __syncthreads();
  if (tid == 0) {
    int64_t run = 0;
    for (int i = 0; i < kSelThreads; ++i) {
      const int64_t c = scan[i];
      scan[i] = run;
      run += c;
    }
  }
  __syncthreads();
  const int64_t ties_before = scan[tid];
  int64_t sel = 0;
  {
    int64_t tb = ties_before;
    for (int64_t j = j0; j < j1; ++j) {
      const uint32_t x = bits[j];
      if (x > T) {
        ++sel;
      } else if (x == T) {
        if (tb < ties_taken) ++sel;
        ++tb;
      }
    }
  }
  __syncthreads();
  scan[tid] = sel;
  __syncthreads();
  if (tid == 0) {
    int64_t run = 0;
    for (int i = 0; i < kSelThreads; ++i) {
      const int64_t c = scan[i];
      scan[i] = run;
      run += c;
    }
  }
  __syncthreads();
  int64_t pos = scan[tid];
  int64_t tb = ties_before;
  for (int64_t j = j0; j < j1; ++j) {
    const uint32_t x = bits[j];
    bool take = false;
    if (x > T) {
      take = true;
    } else if (x == T) {
      take = tb < ties_taken;
      ++tb;
    }
    if (take && pos < k) out[pos++] = (int32_t)j;
  }
}

template <int D>
hipError_t launch_mass_d(const MassParams& p, hipStream_t stream) {
  const int R = p.group * p.block_len;
  const int rbw = (R + 32 * kMassWaves - 1) / (32 * kMassWaves);  // row blocks per wave
  dim3 grid(p.splits, p.batch * p.kv_heads);
  switch (rbw) {
    case 1: hipLaunchKernelGGL((mass_bf16_kernel<D, 1>), grid, dim3(64 * kMassWaves), 0, stream, p); break;
    case 2: hipLaunchKernelGGL((mass_bf16_kernel<D, 2>), grid, dim3(64 * kMassWaves), 0, stream, p); break;
    case 3: hipLaunchKernelGGL((mass_bf16_kernel<D, 3>), grid, dim3(64 * kMassWaves), 0, stream, p); break;
    case 4: hipLaunchKernelGGL((mass_bf16_kernel<D, 4>), grid, dim3(64 * kMassWaves), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int mass_max_rows() { return 32 * kMassWaves * 4; }
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

hipError_t launch_select(const float* mass, int32_t* idx, int64_t groups, int64_t n, int64_t k,
                         hipStream_t stream) {
  if (groups == 0 || k == 0) return hipSuccess;
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)groups), dim3(kSelThreads), 0, stream, mass, idx, n, k);
  return hipGetLastError();
}

}  // namespace blkattn
