/*
 * blkattn.h - block-diffusion attention over a cached prefix, for AMD MI355X
 * (gfx950). C ABI of libblkattn.so.
 *
 * The operation. In block diffusion the finalised tokens before the current
 * block are a fixed, cached prefix, and the Bq tokens of the current block are
 * denoised together: every block query attends bidirectionally (no causal
 * mask) to all prefix keys and to all Bq block keys ("Fixed State, Long Reach:
 * What a Constant-Size Cache Buys Block Diffusion at Scale", abstract; "LaCache:
 * Exact Caching and Precision-Adaptive Inference for Diffusion Large Language
 * Models", section 3.3.1, where U holds the unchanged tokens and C the current
 * block). With s_j = scale * <q, k_j>:
 *
 *     O   = sum_j softmax(s)_j v_j          LSE = ln sum_j e^{s_j}
 *
 * The prefix and the block are evaluated as two online-softmax partial states
 * (o, m, l): m = max_j s_j, l = sum_j e^{s_j - m}, o = sum_j e^{s_j - m} v_j / l
 * (LaCache section 3.3.3, eqs. 2-6, whose unnormalised accumulator is O~ = l*o),
 * and combined by a log-sum-exp merge. A prefix partial computed once per block
 * can thus be reused at later denoising steps and merged with a fresh block
 * partial (LaCache section 3.3.3 FACache; "FlashBlock: Attention Caching for
 * Efficient Long-Context Block Diffusion", abstract, which caches the
 * block-external attention and recomputes the block-internal part). The prefix
 * may also be a retained subset of a longer cache named by row indices
 * (aitopics tag page "kv state", Sparse-dLLM abstract: keep the critical
 * tokens, evict the rest).
 *
 * Conventions shared by every entry point:
 *  - All data pointers are DEVICE pointers (hipMalloc / torch CUDA tensors)
 *    except the dims and tensor descriptor structs, which are host memory read
 *    during the call only. The library never allocates, frees or synchronises,
 *    keeps no pointer after returning, and enqueues its kernels on `stream`
 *    (a hipStream_t; NULL = the default stream). Results are ready when the
 *    stream reaches that point; device faults surface at the caller's next
 *    synchronisation.
 *  - Tensors are [B, H, T, d] with element strides for B, H and T and a unit
 *    stride along d (head_dim). Base pointers and the B/H/T strides (in bytes)
 *    must be multiples of 16 bytes.
 *  - GQA: query head h reads kv head h / (q_heads / kv_heads); q_heads must be
 *    a multiple of kv_heads.
 *  - dtype: BLKATTN_F32 (fp32 everywhere) or BLKATTN_BF16 (bf16 Q, K, V and O;
 *    fp32 accumulation; LSE and partials are always fp32).
 *  - Supported head_dim: 64 or 128.
 *  - Errors: a negative status. Arguments are validated on the host before
 *    anything is enqueued; on error nothing is enqueued and no output is
 *    touched. blkattn_last_error() returns a thread-local message.
 *  - Degenerate sizes: batch, q_heads or block_len equal to 0 is a no-op that
 *    returns BLKATTN_OK. An empty prefix (prefix_len == 0, or n_keep == 0 with
 *    indices) gives the empty partial o = 0, m = -inf, l = 0.
 *  - Outputs must not alias inputs, except where an entry point says so.
 *  - Results are bitwise reproducible for a given shape, split count and
 *    device: the split plan is a function of the dims, merges run in a fixed
 *    order and no floating-point atomics are used.
 *  - Concurrency: no global state is modified; calls on different streams may
 *    run concurrently (with disjoint workspaces).
 */
#ifndef BLKATTN_H
#define BLKATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BLKATTN_ABI_VERSION 1

/* dtype codes */
#define BLKATTN_F32 0
#define BLKATTN_BF16 1

/* status codes */
#define BLKATTN_OK 0
#define BLKATTN_ERR_INVALID_ARG (-1) /* null pointer, negative size, bad GQA ratio, bad scale */
#define BLKATTN_ERR_UNSUPPORTED (-2) /* dtype / head_dim combination not built */
#define BLKATTN_ERR_MISALIGNED (-3)  /* pointer or stride not a multiple of 16 bytes */
#define BLKATTN_ERR_WORKSPACE (-4)   /* workspace missing or smaller than required */
#define BLKATTN_ERR_HIP (-5)         /* a HIP launch failed; see blkattn_last_error() */

/* op codes for blkattn_workspace_bytes / blkattn_plan_splits */
#define BLKATTN_OP_FULL 0
#define BLKATTN_OP_PREFIX_PARTIAL 1
#define BLKATTN_OP_SELECT 2 /* blkattn_select_retained */
#define BLKATTN_OP_SEQUENCE 3 /* blkattn_sequence_step */

/* Problem sizes. */
typedef struct blkattn_dims {
  int32_t batch;      /* B */
  int32_t q_heads;    /* Hq */
  int32_t kv_heads;   /* Hkv; Hq % Hkv == 0 */
  int32_t head_dim;   /* d */
  int32_t block_len;  /* Bq: block queries, and also the number of block keys */
  int32_t n_keep;     /* prefix rows kept when an index array is given; must be 0
                         when idx is NULL */
  int64_t prefix_len; /* P: rows of the prefix K/V tensors (P_full when indexed) */
  int32_t dtype;      /* BLKATTN_F32 or BLKATTN_BF16 */
  float scale;        /* score scale, finite and > 0; 1/sqrt(d) for standard attention */
  int32_t splits;     /* 0: automatic split plan over the keys; > 0: use this many
                         key splits (clamped to the number of 64-key tiles) */
  int32_t reserved;   /* must be 0 */
} blkattn_dims;

/* A strided [B, H, T, d] tensor; strides in elements, unit stride along d. */
typedef struct blkattn_tensor {
  void* data;
  int64_t stride_b;
  int64_t stride_h;
  int64_t stride_t;
} blkattn_tensor;

/*
 * A partial online-softmax state of the block queries over one key set
 * (LaCache section 3.3.3: the cached (m, l, O~) with O~ = l * o).
 * Contiguous fp32: o [B, Hq, Bq, d], m [B, Hq, Bq], l [B, Hq, Bq].
 * m is the maximum scaled score (natural-log units), l = sum e^{s - m},
 * o = O~ / l; an empty key set is (0, -inf, 0).
 */
typedef struct blkattn_partial {
  float* o;
  float* m;
  float* l;
} blkattn_partial;

/*
 * blkattn_full - O and LSE of the block queries over [prefix; block].
 *   q      [B, Hq, Bq, d]             block queries
 *   k_pre, v_pre [B, Hkv, P, d]       cached prefix (P = prefix_len rows)
 *   idx    int32 [B, Hkv, n_keep], contiguous, or NULL. When given, the prefix
 *          is the rows idx[b, h, 0..n_keep) of k_pre/v_pre, in that order
 *          (retained-token eviction, "kv state" page, Sparse-dLLM). Entries
 *          must lie in [0, prefix_len); out-of-range entries are clamped into
 *          range (memory-safe, result unspecified). Sorted ascending indices
 *          give the best memory locality.
 *   k_blk, v_blk [B, Hkv, Bq, d]      the current block's keys and values
 *   o      [B, Hq, Bq, d]             output, dtype of q
 *   lse    fp32 [B, Hq, Bq] contiguous, or NULL
 *   workspace / workspace_bytes: device scratch of at least
 *          blkattn_workspace_bytes(dims, BLKATTN_OP_FULL) bytes (may be NULL
 *          when that is 0). Contents on entry are ignored.
 * Passages: FACache's lossless result equals plain attention (LaCache sections
 * 3.3 and 3.3.3); output normalisation O = O~/l and L = m + log l (LaCache
 * Appendix J pseudocode).
 */
int blkattn_full(const blkattn_dims* dims, const blkattn_tensor* q, const blkattn_tensor* k_pre,
                 const blkattn_tensor* v_pre, const int32_t* idx, const blkattn_tensor* k_blk,
                 const blkattn_tensor* v_blk, const blkattn_tensor* o, float* lse, void* workspace,
                 size_t workspace_bytes, void* stream);

/*
 * blkattn_full_noalloc - blkattn_full for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the key-split scratch comes from an array of 64 MiB that
 * the library holds in static device memory on every GPU it runs on, so the
 * call allocates nothing and takes no workspace. Arguments and results are
 * those of blkattn_full.
 * Errors: BLKATTN_ERR_WORKSPACE when blkattn_workspace_bytes(dims,
 * BLKATTN_OP_FULL) exceeds 64 MiB (use blkattn_full), BLKATTN_ERR_HIP when the
 * array's address cannot be obtained on the current device.
 * Every call on one GPU shares that GPU's array: calls that may overlap on one
 * GPU (other streams, other threads) race and must not be issued; calls in
 * order on one stream are safe (nothing in the array must start at zero, and
 * each call writes every part of it that it reads).
 */
int blkattn_full_noalloc(const blkattn_dims* dims, const blkattn_tensor* q, const blkattn_tensor* k_pre,
                         const blkattn_tensor* v_pre, const int32_t* idx, const blkattn_tensor* k_blk,
                         const blkattn_tensor* v_blk, const blkattn_tensor* o, float* lse, void* stream);

/*
 * blkattn_prefix_partial - partial state of the block queries over the prefix
 * only: the state FACache stores at the first denoising step of a block
 * (LaCache section 3.3.3; FlashBlock abstract, block-external attention).
 * Arguments as blkattn_full; `out` receives the partial (contiguous fp32).
 * With prefix_len == 0 (or n_keep == 0 when indexed) `out` is the empty state.
 */
int blkattn_prefix_partial(const blkattn_dims* dims, const blkattn_tensor* q,
                           const blkattn_tensor* k_pre, const blkattn_tensor* v_pre,
                           const int32_t* idx, const blkattn_partial* out, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * blkattn_block_partial - partial state of the block queries over the block's
 * own Bq keys, bidirectional (no mask): the part recomputed at every denoising
 * step (FlashBlock abstract, block-internal attention; LaCache section 3.3.3,
 * the tiles overlapping the current block). prefix_len, n_keep are ignored.
 *   q [B, Hq, Bq, d]; k_blk, v_blk [B, Hkv, Bq, d]; out: contiguous fp32.
 */
int blkattn_block_partial(const blkattn_dims* dims, const blkattn_tensor* q,
                          const blkattn_tensor* k_blk, const blkattn_tensor* v_blk,
                          const blkattn_partial* out, void* stream);

/*
 * blkattn_block_step - one denoising step of the reuse path in one launch:
 * every block query's running online-softmax state starts from the cached
 * prefix partial and continues over the block's own Bq keys (no mask), then
 * O and LSE are finalised. This is LaCache's initialisation of (m, l, O~) from
 * the cache followed by the recurrence over the tiles of the current block
 * (section 3.3.3 eqs. 2-6 and the Appendix J pseudocode); it equals
 * blkattn_block_partial followed by blkattn_merge with the cached partial, up
 * to rounding, without the block partial passing through memory.
 *   q [B, Hq, Bq, d]; k_blk, v_blk [B, Hkv, Bq, d]
 *   cached  contiguous fp32 partial [B, Hq, Bq, (d)] of the same queries over
 *           the prefix (read only; an empty state is allowed)
 *   o       [B, Hq, Bq, d] output in dims->dtype; must not alias an input
 *   lse     fp32 [B, Hq, Bq], or NULL
 * prefix_len, n_keep and splits are ignored.
 */
int blkattn_block_step(const blkattn_dims* dims, const blkattn_tensor* q, const blkattn_tensor* k_blk,
                       const blkattn_tensor* v_blk, const blkattn_partial* cached,
                       const blkattn_tensor* o, float* lse, void* stream);

/*
 * blkattn_merge - log-sum-exp merge of two partial states of the same queries
 * over disjoint key sets: M = max(m_a, m_b), w_x = l_x e^{m_x - M},
 * l = w_a + w_b, o = (w_a o_a + w_b o_b) / l, LSE = M + ln l. Continuing the
 * online-softmax recurrence from a cached state over the remaining tiles gives
 * the same result (LaCache section 3.3.3 and the Appendix J pseudocode, which
 * initialise (m, l, O~) from the cache at later steps).
 *   a, b   input partials (contiguous fp32 [B, Hq, Bq, (d)])
 *   o      [B, Hq, Bq, d] output in dims->dtype, or NULL
 *   lse    fp32 [B, Hq, Bq], or NULL
 *   ab     merged partial, or NULL; it may alias a or b exactly (in-place
 *          update of a cached state)
 * Both sides empty gives o = 0, LSE = -inf and the empty partial.
 * prefix_len, n_keep and kv_heads are ignored (kv_heads must still be > 0).
 */
int blkattn_merge(const blkattn_dims* dims, const blkattn_partial* a, const blkattn_partial* b,
                  const blkattn_tensor* o, float* lse, const blkattn_partial* ab, void* stream);

/*
 * blkattn_gather_prefix - bit copy of the retained prefix rows:
 *   k_out[b, h, r, :] = k_full[b, h, idx[b, h, r], :], same for v
 * ("kv state" page, Sparse-dLLM abstract: retained critical tokens).
 *   k_full, v_full [B, Hkv, prefix_len, d]; idx int32 [B, Hkv, n_keep]
 *   contiguous (entries clamped into [0, prefix_len)); k_out, v_out
 *   [B, Hkv, n_keep, d]. Element type from dims->dtype.
 */
int blkattn_gather_prefix(const blkattn_dims* dims, const blkattn_tensor* k_full,
                          const blkattn_tensor* v_full, const int32_t* idx,
                          const blkattn_tensor* k_out, const blkattn_tensor* v_out, void* stream);

/*
 * blkattn_sequence_step - first-layer attention of every token of the sequence
 * at one denoising step of a block, with FACache (LaCache section 3.3.3 and
 * the Appendix J pseudocode of its first-layer FlashAttention). The block C is
 * the rows [block_start, block_start + block_len) of the N = prefix_len
 * sequence rows; U is every other row (prompt, earlier blocks and the masked
 * suffix), whose q, k and v stay fixed while the block is denoised.
 *   gen_step != 0 (the block's first step): cache <- the partial state of the
 *     U queries over the U keys (section 3.3.3: the tiles with both queries and
 *     keys in U). Then, at every step:
 *   U queries: the running state starts from the cache and continues over the
 *     block's keys only (the tiles overlapping C), giving their O and LSE;
 *   C queries: attention over all N keys.
 * The result is plain attention over the whole sequence as long as the U rows
 * are the ones the cache was built from (the cache is exact, not approximate).
 *   q      [B, Hq, N, d];  k, v [B, Hkv, N, d]
 *   cache  contiguous fp32 partial over the sequence rows: o [B, Hq, N, d],
 *          m, l [B, Hq, N]. Written when gen_step != 0, read otherwise; its
 *          block rows are neither read nor written. Same layout and meaning as
 *          blkattn_partial elsewhere (o normalised, m in natural-log units).
 *   o      [B, Hq, N, d] output, dtype of q;  lse fp32 [B, Hq, N] or NULL
 *   workspace / workspace_bytes: blkattn_workspace_bytes(dims,
 *          BLKATTN_OP_SEQUENCE) bytes, 16-byte aligned (NULL when 0).
 * dims: prefix_len = N, block_len = the block's rows (>= 1), n_keep = 0;
 * splits applies to the launches over many keys. Up to three kernels (four with
 * split merges) are enqueued on `stream` in order; o, lse and cache must not
 * alias q, k or v.
 */
int blkattn_sequence_step(const blkattn_dims* dims, int64_t block_start, int gen_step, const blkattn_tensor* q,
                          const blkattn_tensor* k, const blkattn_tensor* v, const blkattn_partial* cache,
                          const blkattn_tensor* o, float* lse, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * blkattn_prefix_mass - attention mass of every dense prefix row:
 *   mass[b, h, j] = sum over the q-heads g of kv head h and the block queries i
 *                   of exp(scale * <q[b, g, i], k_pre[b, h, j]> - lse[b, g, i])
 * i.e. the attention probability key j receives, summed over the queries that
 * read it; the score that guides which prefix rows to retain (Sparse-dLLM
 * abstract on the aitopics "kv state" page: keep the critical tokens, evict
 * the rest).
 *   q      [B, Hq, Bq, d]
 *   k_pre  [B, Hkv, prefix_len, d] (dense: n_keep and indices play no part)
 *   lse    fp32 [B, Hq, Bq] contiguous: each row's log-sum-exp over all keys it
 *          attends (as blkattn_full returns it)
 *   mass   fp32 [B, Hkv, prefix_len] contiguous output
 * The column sums run in a fixed order (bitwise reproducible); with more than
 * 512 query rows per kv head (q_heads / kv_heads * block_len) the rows are
 * taken in passes of 512 launched in order on `stream`.
 */
int blkattn_prefix_mass(const blkattn_dims* dims, const blkattn_tensor* q, const blkattn_tensor* k_pre,
                        const float* lse, float* mass, void* stream);

/*
 * blkattn_select_retained - per (batch, kv head), the n_keep prefix rows of
 * largest mass, ties broken towards the lower row, listed in ascending row
 * order: the index layout of blkattn_full / blkattn_gather_prefix.
 *   mass  fp32 [B, Hkv, prefix_len] contiguous, finite and >= 0 (-0 counts as 0)
 *   idx   int32 [B, Hkv, n_keep] contiguous output
 *   workspace / workspace_bytes: device scratch of at least
 *         blkattn_workspace_bytes(dims, BLKATTN_OP_SELECT) bytes, 16-byte
 *         aligned; contents on entry are ignored. May be NULL when
 *         n_keep == prefix_len (every row kept).
 * Requires n_keep <= prefix_len <= INT32_MAX. Deterministic: an exact radix
 * selection of the n_keep-th largest mass over several kernels on `stream`.
 */
int blkattn_select_retained(const blkattn_dims* dims, const float* mass, int32_t* idx, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Workspace bytes blkattn_full / blkattn_prefix_partial need for these dims
 * (0 when the plan uses a single key split), or blkattn_select_retained
 * (op BLKATTN_OP_SELECT) or blkattn_sequence_step (op BLKATTN_OP_SEQUENCE) need. The prefix is taken as indexed
 * with n_keep rows when n_keep > 0, else as prefix_len dense rows; an indexed
 * call with n_keep == 0 needs no more than this. Returns 0 for invalid dims. */
size_t blkattn_workspace_bytes(const blkattn_dims* dims, int op);

/* Number of key splits the plan uses for these dims and op (>= 1; for
 * BLKATTN_OP_SELECT the workgroups per (batch, kv head)), or a negative status
 * for invalid dims. */
int blkattn_plan_splits(const blkattn_dims* dims, int op);

/*
 * Measurement hook: the next blkattn_full or blkattn_prefix_partial call made
 * by this thread hands `start` and `stop` to the launch of its attention
 * (partial) kernel, whose dispatch stamps them with the kernel's own begin and
 * end (hipExtLaunchKernel), then forgets both; hipEventElapsedTime(start,
 * stop) is that kernel's duration. Events are hipEvent_t handles created and
 * owned by the caller. Pass NULL, NULL to clear.
 */
void blkattn_set_kernel_events(void* start, void* stop);

const char* blkattn_strerror(int status);
const char* blkattn_last_error(void);
int blkattn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BLKATTN_H */
