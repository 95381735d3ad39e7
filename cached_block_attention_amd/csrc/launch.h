// Internal launch descriptors shared by the host API and the HIP kernels of
// libblkattn.so. Not part of the public ABI (include/blkattn.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

namespace blkattn {

// Keys per staged tile of the bf16 MFMA kernel and of the split plan.
constexpr int kTileKeys = 64;

// The concatenated key sequence one (batch, kv-head) attends:
// [prefix rows (optionally gathered through idx); block rows].
struct KeySeq {
  const void* k_pre;
  const void* v_pre;
  int64_t kp_sb, kp_sh, kp_st;  // element strides of k_pre
  int64_t vp_sb, vp_sh, vp_st;  // element strides of v_pre
  const int32_t* idx;           // [B, Hkv, n_pre] or nullptr
  int64_t p_rows;               // rows of k_pre/v_pre (clamp bound for idx)
  int64_t n_pre;                // prefix keys attended (P, or n_keep with idx)
  // Dense prefix key j reads row j + (j >= k_hole ? k_hole_len : 0): a prefix
  // that skips the rows of a block sitting inside the sequence.
  int64_t k_hole, k_hole_len;
  int32_t off32;                // byte offsets within any 64-row tile (prefix or block) fit 31 bits
  int32_t gather32;             // with idx: byte offsets of every prefix row (p_rows of them) fit 31 bits
  int32_t stream_nt;            // dense prefix tiles are loaded non-temporal (a long single-pass stream)
  const void* k_blk;
  const void* v_blk;
  int64_t kb_sb, kb_sh, kb_st;
  int64_t vb_sb, vb_sh, vb_st;
  int32_t n_blk;                // block keys attended (Bq, or 0)
};

// Where a partial-attention launch writes.
enum OutMode : int32_t {
  kOutFinal = 0,    // O in the input dtype (strided) + optional LSE, at mapped rows
  kOutPartial = 1,  // the caller's fp32 partial (o, m, l), at mapped rows
  kOutSplit = 2,    // workspace partials, packed rows; split s at offset s * split_rows
};

// In the split workspace of the bf16 kernels, o is stored as fp16 scaled by a
// power of two per (split, row) so that the row's largest |o| lies in
// [2^13, 2^14), and m, l and the inverse scale form one 16-byte record per
// (split, row) ({m, l, 1/scale, 0} at pmls). fp32 kernels store o as fp32 and
// m, l in arrays of their own.


struct OutDesc {
  int32_t mode;
  void* o;                      // final O
  int64_t o_sb, o_sh, o_st;
  float* lse;                   // final LSE or nullptr
  float* po;                    // partial o base
  float* pm;                    // partial m base
  float* pl;                    // partial l base
  int64_t split_rows;           // rows of one split's partial (B*Hq*Bq) in kOutSplit
  float4* pmls;                 // kOutSplit, bf16 kernels: {m, l, 1/scale, 0} per row (o is fp16 at po)
};

// Query-row map. Packed row qi of a head reads sequence row
// qi + (qi >= q_hole ? q_hole_len : 0) of q and of the final O; the per-row
// arrays outside the split workspace (LSE, a caller's partial, the initial
// state) hold that row at ((b * Hq + hq) * row_pitch + sequence row). With
// q_hole_len == 0 and row_pitch == block_len this is the identity.
struct RowMap {
  int64_t q_hole, q_hole_len, row_pitch;
};

struct AttnParams {
  int32_t batch, q_heads, kv_heads, group, head_dim, block_len;
  const void* q;
  int64_t q_sb, q_sh, q_st;
  KeySeq keys;
  OutDesc out;
  float scale;          // score scale (natural-log units)
  float scale_log2;     // scale * log2(e): scores in base-2 units
  int32_t splits;       // key splits (gridDim.x)
  int32_t tiles;        // ceil((n_pre + n_blk) / tile keys of this kernel)
  int32_t rows_per_wg;  // packed (q-head, query) rows one workgroup owns
  int32_t row_chunks;   // workgroups along the packed rows of one kv-head
  RowMap rows;
  // Optional initial state (one key split only): contiguous fp32 partial
  // (o [rows, d], m, l [rows]) the running state starts from instead of the
  // empty state; nullptr when absent.
  const float* init_o;
  const float* init_m;
  const float* init_l;
};

// Inputs of an N-way log-sum-exp merge of partials (same rows, disjoint keys).
struct MergeParams {
  int32_t batch, q_heads, block_len, head_dim;
  int32_t nsrc;               // number of partials merged
  const float* src_o[2];      // explicit sources (nsrc == 2 and strided == 0)
  const float* src_m[2];
  const float* src_l[2];
  int32_t strided;            // 1: sources are src_*[0] + s * split_rows
  int64_t split_rows;
  const float4* src_mls;      // strided sources: {m, l, 1/scale, 0} records (o fp16), or nullptr (o fp32)
  int32_t out_dtype;          // BLKATTN_F32 / BLKATTN_BF16 for o_final
  void* o_final;              // strided O or nullptr
  int64_t o_sb, o_sh, o_st;
  float* lse;                 // or nullptr
  float* out_o;               // merged partial or nullptr
  float* out_m;
  float* out_l;
  RowMap rows;                // outputs and explicit sources at mapped rows;
                              // strided (workspace) sources at packed rows
};

struct GatherParams {
  int32_t batch, kv_heads, head_dim, elt_bytes;
  int64_t p_rows, n_keep;
  const int32_t* idx;
  const void* k_full;
  const void* v_full;
  int64_t kf_sb, kf_sh, kf_st, vf_sb, vf_sh, vf_st;
  void* k_out;
  void* v_out;
  int64_t ko_sb, ko_sh, ko_st, vo_sb, vo_sh, vo_st;
};

// Attention mass of the dense prefix keys (see mass_topk.hip).
struct MassParams {
  int32_t batch, q_heads, kv_heads, group, head_dim, block_len;
  int32_t dtype;                // BLKATTN_F32 / BLKATTN_BF16
  const void* q;
  int64_t q_sb, q_sh, q_st;
  const void* k;                // prefix keys [B, Hkv, n_keys, d]
  int64_t k_sb, k_sh, k_st;
  int64_t n_keys;
  const float* lse;             // [B, Hq, Bq] row log-sum-exp over all keys
  float* mass;                  // [B, Hkv, n_keys]
  float scale;
  float scale_log2;
  int32_t splits;               // bf16: key splits (gridDim.x)
  int32_t tiles;                // bf16: ceil(n_keys / mass_tile_keys())
  int32_t row0, row_end;        // bf16: packed rows of this pass (set by the launcher)
  int32_t accumulate;           // bf16: add onto mass (passes after the first)
};

// Optional timing events of one attention launch: the dispatch itself stamps
// them with its begin and end (hipExtLaunchKernel), so their elapsed time is
// the kernel's own duration, without the gaps that separate event records put
// around it.
struct KernelEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// Kernel launchers (return the hipError_t of the launch).
hipError_t launch_attn_bf16(const AttnParams& p, int waves, hipStream_t stream, KernelEvents ev = {});
hipError_t launch_attn_f32(const AttnParams& p, hipStream_t stream, KernelEvents ev = {});
hipError_t launch_merge(const MergeParams& p, hipStream_t stream);
hipError_t launch_gather(const GatherParams& p, hipStream_t stream);
hipError_t launch_fill_empty(float* o, float* m, float* l, int64_t rows, int head_dim,
                             hipStream_t stream);
hipError_t launch_mass(const MassParams& p, hipStream_t stream);
// Chunking of the selection: `chunks` workgroups of `chunk` rows per group, and
// the workspace bytes it needs.
struct SelectPlan {
  int chunks;
  int64_t chunk;
  size_t ws_bytes;
};
SelectPlan select_plan(int64_t groups, int64_t n);
hipError_t launch_select(const float* mass, int32_t* idx, void* ws, int64_t groups, int64_t n, int64_t k,
                         hipStream_t stream);
int mass_tile_keys();  // keys per tile of the bf16 mass kernel

// Launch shape of the bf16 kernel: waves per workgroup for a chunk of packed
// rows (1, 2, 4 or 8), keys per staged tile, workgroups resident per CU, and
// the most retained-row indices one key split may stage.
int bf16_waves_for_rows(int64_t rows);
int bf16_tile_keys(int waves);
int bf16_workgroups_per_cu(int waves);
int bf16_index_cap();

}  // namespace blkattn
