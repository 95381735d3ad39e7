// Host side of libblkattn.so: argument validation, the key-split plan,
// workspace layout and kernel launches behind the C ABI of include/blkattn.h.
//
// The library is stateless apart from a thread-local error message and the
// thread-local one-shot measurement events; it never allocates, frees or
// synchronises, and enqueues everything on the caller's stream.
#include "blkattn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>

#include "launch.h"

namespace {

using namespace blkattn;

thread_local char g_err[512] = "";
thread_local void* g_ev_start = nullptr;
thread_local void* g_ev_stop = nullptr;

// The automatic plan aims for as many workgroups as the 256 compute units of
// an MI355X hold at once. A fixed target keeps the plan (and so the bits of the
// result) a function of the dims alone.
constexpr int64_t kComputeUnits = 256;
// Each key split keeps at least this many 64-key tiles, which bounds the
// split-partial traffic (d+2 fp32 per row per split) relative to the K/V
// stream.
constexpr int64_t kMinTilesPerSplit = 4;
// Finest packed-row chunk a small launch is cut into, and the longest key
// range for which that is done (each chunk reads the range again).
constexpr int64_t kMinChunkRows = 32;
// The MI355X last-level (Infinity) cache.
constexpr int64_t kLastLevelCacheBytes = (int64_t)256 << 20;
constexpr int64_t kFineChunkKeys = 8192;
// Packed rows of one ping-pong workgroup (seven row waves), and the fewest
// 64-key tiles per workgroup for which that kernel is chosen over finer
// chunks of a launch that would not fill the GPU.
constexpr int64_t kPingPongRows = 224;
constexpr int64_t kPingPongMinTiles = 8;
constexpr size_t kWsAlign = 256;

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return BLKATTN_OK;
}

int elt_bytes(int dtype) { return dtype == BLKATTN_F32 ? 4 : 2; }

int check_dims(const blkattn_dims* d) {
  if (d == nullptr) return fail(BLKATTN_ERR_INVALID_ARG, "dims is NULL");
  if (d->reserved != 0) return fail(BLKATTN_ERR_INVALID_ARG, "dims.reserved must be 0");
  if (d->batch < 0 || d->q_heads < 0 || d->block_len < 0 || d->prefix_len < 0 || d->n_keep < 0 ||
      d->splits < 0)
    return fail(BLKATTN_ERR_INVALID_ARG, "negative size in dims");
  if (d->kv_heads <= 0) return fail(BLKATTN_ERR_INVALID_ARG, "kv_heads must be > 0");
  if (d->q_heads % d->kv_heads != 0)
    return fail(BLKATTN_ERR_INVALID_ARG, "q_heads (%d) is not a multiple of kv_heads (%d)", d->q_heads,
                d->kv_heads);
  if (d->dtype != BLKATTN_F32 && d->dtype != BLKATTN_BF16)
    return fail(BLKATTN_ERR_UNSUPPORTED, "dtype %d is not supported", d->dtype);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(BLKATTN_ERR_UNSUPPORTED, "head_dim %d is not supported (64 or 128)", d->head_dim);
  if (!(d->scale > 0.0f) || !std::isfinite(d->scale))
    return fail(BLKATTN_ERR_INVALID_ARG, "scale must be finite and > 0");
  return BLKATTN_OK;
}

// A [B, H, T, d] tensor with `rows` rows; with rows == 0 it may be absent.
int check_tensor(const blkattn_tensor* t, const char* name, int eb, int64_t rows) {
  if (rows == 0 && (t == nullptr || t->data == nullptr)) return BLKATTN_OK;
  if (t == nullptr || t->data == nullptr) return fail(BLKATTN_ERR_INVALID_ARG, "%s is NULL", name);
  if (t->stride_b < 0 || t->stride_h < 0 || t->stride_t < 0)
    return fail(BLKATTN_ERR_INVALID_ARG, "%s has a negative stride", name);
  if (reinterpret_cast<uintptr_t>(t->data) % 16 != 0)
    return fail(BLKATTN_ERR_MISALIGNED, "%s data pointer is not 16-byte aligned", name);
  if ((t->stride_b * eb) % 16 != 0 || (t->stride_h * eb) % 16 != 0 || (t->stride_t * eb) % 16 != 0)
    return fail(BLKATTN_ERR_MISALIGNED, "%s strides are not multiples of 16 bytes", name);
  return BLKATTN_OK;
}

int check_partial(const blkattn_partial* p, const char* name, int64_t rows) {
  if (rows == 0 && p == nullptr) return BLKATTN_OK;
  if (p == nullptr || p->o == nullptr || p->m == nullptr || p->l == nullptr)
    return fail(BLKATTN_ERR_INVALID_ARG, "%s (or one of its o, m, l) is NULL", name);
  if (reinterpret_cast<uintptr_t>(p->o) % 16 != 0 || reinterpret_cast<uintptr_t>(p->m) % 4 != 0 ||
      reinterpret_cast<uintptr_t>(p->l) % 4 != 0)
    return fail(BLKATTN_ERR_MISALIGNED, "%s.o must be 16-byte aligned (m, l 4-byte)", name);
  return BLKATTN_OK;
}

struct Plan {
  int waves = 1;        // waves per workgroup (bf16 kernel)
  int rows_per_wg = 0;  // packed rows per workgroup
  int row_chunks = 1;
  int tile_keys = 64;   // keys per staged tile of the chosen kernel
  int tiles = 0;        // tiles of tile_keys over the key sequence
  int splits = 1;
};

// Key splits for a chunking of the packed rows (bf16) or for the fp32 kernel.
int64_t plan_splits(const blkattn_dims* d, const Plan& pl, int64_t base, int64_t per_cu, int64_t n_keys,
                    bool indexed) {
  const int64_t tiles64 = (n_keys + 63) / 64;
  int64_t s;
  if (d->splits > 0) {
    s = d->splits;
  } else {
    const int64_t target = kComputeUnits * per_cu;
    s = base > 0 ? (target + base - 1) / base : 1;
    const int64_t cap = tiles64 / kMinTilesPerSplit;
    if (s > cap) s = cap;
  }
  if (s > tiles64) s = tiles64;
  if (s > pl.tiles) s = pl.tiles;
  if (s < 1) s = 1;
  if (indexed && d->dtype == BLKATTN_BF16) {
    // every split stages its retained-row indices in LDS
    const int64_t per = bf16_index_cap() / pl.tile_keys;  // tiles per split at most
    const int64_t need = (pl.tiles + per - 1) / per;
    if (s < need) s = need;
  }
  return s;
}

Plan make_plan(const blkattn_dims* d, int64_t n_keys, bool indexed) {
  Plan pl;
  const int64_t G = d->q_heads / d->kv_heads;
  const int64_t R = G * d->block_len;
  if (d->dtype == BLKATTN_F32) {
    // One workgroup per (split, q-head, batch) walks its 32-key tiles one
    // after another, each tile a latency-bound chain: spread the tiles over
    // the compute units, down to one tile per split.
    pl.tile_keys = 32;
    pl.tiles = (int)((n_keys + pl.tile_keys - 1) / pl.tile_keys);
    const int64_t base = (int64_t)d->batch * d->q_heads;
    int64_t sp = d->splits > 0 ? d->splits : (kComputeUnits + base - 1) / base;
    if (sp > pl.tiles) sp = pl.tiles;
    if (sp < 1) sp = 1;
    pl.splits = (int)sp;
    return pl;
  }
  // More packed rows than one ping-pong workgroup holds (225 or more) over a
  // long key range, in a launch of at most one workgroup per compute unit:
  // chunks of 129 to 224 rows keep the ping-pong kernel, whose MFMA and
  // softmax phases run at the same time, even when the launch then holds
  // fewer workgroups than the GPU has compute units. Per 64-key tile and
  // packed row it costs about 40 % of the sequential four-wave kernel the
  // halving below would reach (large blocks: Bq 1024 over its own keys).
  // Launches of several rounds keep the 256-row chunks of the sequential
  // eight-wave kernel: 224-row chunks would add a partial round.
  if (R > kPingPongRows) {
    const int64_t c = (R + kPingPongRows - 1) / kPingPongRows;
    const int64_t rows = (R + c - 1) / c;
    if (bf16_waves_for_rows(rows) == 8) {
      Plan pp;
      pp.row_chunks = (int)c;
      pp.waves = 8;
      pp.rows_per_wg = (int)(32 * ((rows + 31) / 32));
      pp.tile_keys = bf16_tile_keys(8);
      pp.tiles = (int)((n_keys + pp.tile_keys - 1) / pp.tile_keys);
      const int64_t base = (int64_t)d->batch * d->kv_heads * c;
      pp.splits = (int)plan_splits(d, pp, base, bf16_workgroups_per_cu(8), n_keys, indexed);
      const int64_t wgs = base * pp.splits;
      if (2 * wgs >= kComputeUnits && wgs <= kComputeUnits && pp.tiles >= kPingPongMinTiles * pp.splits) return pp;
    }
  }
  // Packed-row chunks of at most `cap` rows, one workgroup each per key split.
  // The cap starts at 256 (eight waves); when the launch would still hold
  // fewer workgroups than the GPU has compute units (a short key range that
  // cannot be split further, as in a large block's own keys), it is halved,
  // down to one wave: every chunk then reads the key range again, which costs
  // little when the range is this short. A key range of one 32-key tile (the
  // block's keys for queries that continue from a cache) starts at one wave:
  // every chunk is then a short load-compute-store chain of its own, and
  // small workgroups keep those chains flowing through the CUs instead of in
  // rounds of eight-wave workgroups (measured 9 % faster on 4064 such rows per
  // head, behind a cache flush).
  for (int64_t cap = n_keys <= 32 ? kMinChunkRows : 256;; cap /= 2) {
    pl.row_chunks = R > cap ? (int)((R + cap - 1) / cap) : 1;
    const int64_t rows = (R + pl.row_chunks - 1) / pl.row_chunks;
    pl.waves = bf16_waves_for_rows(rows);
    pl.rows_per_wg = (int)(32 * ((rows + 31) / 32));  // whole 32-row waves per chunk
    pl.tile_keys = bf16_tile_keys(pl.waves);
    pl.tiles = (int)((n_keys + pl.tile_keys - 1) / pl.tile_keys);
    const int64_t base = (int64_t)d->batch * d->kv_heads * pl.row_chunks;
    const int64_t s = plan_splits(d, pl, base, bf16_workgroups_per_cu(pl.waves), n_keys, indexed);
    pl.splits = (int)s;
    if (base * s >= kComputeUnits || cap <= kMinChunkRows || R <= 32 || n_keys > kFineChunkKeys) break;
  }
  return pl;
}

struct WsLayout {
  size_t o = 0, m = 0, l = 0, total = 0;
  size_t mls = 0;  // bf16 kernels: {m, l, 1/scale, 0} records (o is fp16); 0 = none (m, l arrays)
};

size_t align_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

// Split partials of one call. bf16 kernels: o [splits][rows][d] fp16 (scaled
// per row), then one {m, l, 1/scale, 0} fp32 record per (split, row). fp32
// kernel: o [splits][rows][d] fp32, then m and l [splits][rows] fp32.
WsLayout ws_layout(const blkattn_dims* d, int splits) {
  WsLayout w;
  if (splits <= 1) return w;
  const size_t rows = (size_t)d->batch * d->q_heads * d->block_len;
  w.o = 0;
  if (d->dtype == BLKATTN_BF16) {
    w.mls = align_up((size_t)splits * rows * d->head_dim * 2);
    w.total = align_up(w.mls + (size_t)splits * rows * 16);
    return w;
  }
  w.m = align_up(w.o + (size_t)splits * rows * d->head_dim * sizeof(float));
  w.l = align_up(w.m + (size_t)splits * rows * sizeof(float));
  w.total = align_up(w.l + (size_t)splits * rows * sizeof(float));
  return w;
}

int64_t prefix_keys(const blkattn_dims* d, const int32_t* idx) { return idx ? d->n_keep : d->prefix_len; }

void fill_keys(KeySeq& ks, const blkattn_dims* d, const blkattn_tensor* k_pre, const blkattn_tensor* v_pre,
               const int32_t* idx, const blkattn_tensor* k_blk, const blkattn_tensor* v_blk, int64_t n_pre,
               int32_t n_blk) {
  ks = KeySeq{};
  ks.n_pre = n_pre;
  ks.n_blk = n_blk;
  ks.p_rows = d->prefix_len;
  ks.idx = idx;
  if (n_pre > 0) {
    ks.k_pre = k_pre->data;
    ks.kp_sb = k_pre->stride_b, ks.kp_sh = k_pre->stride_h, ks.kp_st = k_pre->stride_t;
    ks.v_pre = v_pre->data;
    ks.vp_sb = v_pre->stride_b, ks.vp_sh = v_pre->stride_h, ks.vp_st = v_pre->stride_t;
  }
  if (n_blk > 0) {
    ks.k_blk = k_blk->data;
    ks.kb_sb = k_blk->stride_b, ks.kb_sh = k_blk->stride_h, ks.kb_st = k_blk->stride_t;
    ks.v_blk = v_blk->data;
    ks.vb_sb = v_blk->stride_b, ks.vb_sh = v_blk->stride_h, ks.vb_st = v_blk->stride_t;
  }
  // Byte offsets inside any 64-row tile (plus the row itself) fit 31 bits, so
  // the kernels may address a tile as a 64-bit base plus 32-bit lane offsets.
  int64_t st = 0;
  for (int64_t x : {ks.kp_st, ks.vp_st, ks.kb_st, ks.vb_st}) st = x > st ? x : st;
  ks.off32 = st * elt_bytes(d->dtype) <= ((int64_t)1 << 25);
  if (idx != nullptr) {
    const int64_t pst = (ks.kp_st > ks.vp_st ? ks.kp_st : ks.vp_st) * elt_bytes(d->dtype);
    ks.gather32 = ks.p_rows * pst + pst <= ((int64_t)1 << 31);
  }
}

RowMap identity_rows(const blkattn_dims* d) { return RowMap{0, 0, d->block_len}; }

AttnParams attn_params(const blkattn_dims* d, const blkattn_tensor* q, const Plan& pl) {
  AttnParams p{};
  p.batch = d->batch;
  p.q_heads = d->q_heads;
  p.kv_heads = d->kv_heads;
  p.group = d->q_heads / d->kv_heads;
  p.head_dim = d->head_dim;
  p.block_len = d->block_len;
  p.q = q->data;
  p.q_sb = q->stride_b, p.q_sh = q->stride_h, p.q_st = q->stride_t;
  p.scale = d->scale;
  p.scale_log2 = (float)((double)d->scale * 1.4426950408889634);
  p.splits = pl.splits;
  p.tiles = pl.tiles;
  p.rows_per_wg = pl.rows_per_wg;
  p.row_chunks = pl.row_chunks;
  p.rows = identity_rows(d);
  return p;
}

int launch_attn(const blkattn_dims* d, const AttnParams& p0, const Plan& pl, hipStream_t stream) {
  // A dense prefix whose K/V (as read by this launch: once per row chunk)
  // fills the last-level cache is streamed with non-temporal loads: no later
  // call can find it cached. Shorter ones keep the normal policy, so that
  // repeated calls can hit the cache.
  AttnParams p = p0;
  const int64_t kv_bytes = 2 * (int64_t)d->batch * d->kv_heads * pl.row_chunks * p.keys.n_pre * d->head_dim *
                           elt_bytes(d->dtype);
  p.keys.stream_nt = p.keys.idx == nullptr && pl.row_chunks == 1 && kv_bytes >= kLastLevelCacheBytes;
  KernelEvents ev;
  ev.start = (hipEvent_t)g_ev_start;
  ev.stop = (hipEvent_t)g_ev_stop;
  g_ev_start = g_ev_stop = nullptr;
  hipError_t e = d->dtype == BLKATTN_F32 ? launch_attn_f32(p, stream, ev) : launch_attn_bf16(p, pl.waves, stream, ev);
  if (e != hipSuccess) return fail(BLKATTN_ERR_HIP, "attention kernel launch failed: %s", hipGetErrorString(e));
  return BLKATTN_OK;
}

int check_workspace(const WsLayout& wl, void* workspace, size_t workspace_bytes) {
  if (wl.total == 0) return BLKATTN_OK;
  if (workspace == nullptr || workspace_bytes < wl.total)
    return fail(BLKATTN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", wl.total,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
    return fail(BLKATTN_ERR_MISALIGNED, "workspace is not 16-byte aligned");
  return BLKATTN_OK;
}

// The attention kernel over the plan's key splits, then (with several) the
// fixed-order LSE merge of the split partials. Writes the final O (+ LSE)
// when `o` is given, else the caller's partial `out`; both at p.rows's rows.
int run_splits(const blkattn_dims* d, AttnParams& p, const Plan& pl, const blkattn_tensor* o, float* lse,
               const blkattn_partial* out, void* workspace, hipStream_t s) {
  int st;
  if (pl.splits == 1) {
    if (o != nullptr) {
      p.out.mode = kOutFinal;
      p.out.o = o->data;
      p.out.o_sb = o->stride_b, p.out.o_sh = o->stride_h, p.out.o_st = o->stride_t;
      p.out.lse = lse;
    } else {
      p.out.mode = kOutPartial;
      p.out.po = out->o, p.out.pm = out->m, p.out.pl = out->l;
    }
    if ((st = launch_attn(d, p, pl, s))) return st;
    return ok();
  }
  const WsLayout wl = ws_layout(d, pl.splits);
  const int64_t rows = (int64_t)d->batch * d->q_heads * d->block_len;
  char* ws = (char*)workspace;
  p.out.mode = kOutSplit;
  p.out.po = (float*)(ws + wl.o);
  p.out.pm = wl.mls != 0 ? nullptr : (float*)(ws + wl.m);
  p.out.pl = wl.mls != 0 ? nullptr : (float*)(ws + wl.l);
  p.out.pmls = wl.mls != 0 ? (float4*)(ws + wl.mls) : nullptr;
  p.out.split_rows = rows;
  if ((st = launch_attn(d, p, pl, s))) return st;
  MergeParams mp{};
  mp.batch = d->batch, mp.q_heads = d->q_heads, mp.block_len = d->block_len, mp.head_dim = d->head_dim;
  mp.nsrc = pl.splits;
  mp.strided = 1;
  mp.split_rows = rows;
  mp.src_o[0] = p.out.po, mp.src_m[0] = p.out.pm, mp.src_l[0] = p.out.pl;
  mp.src_mls = p.out.pmls;
  mp.out_dtype = d->dtype;
  mp.rows = p.rows;
  if (o != nullptr) {
    mp.o_final = o->data;
    mp.o_sb = o->stride_b, mp.o_sh = o->stride_h, mp.o_st = o->stride_t;
    mp.lse = lse;
  } else {
    mp.out_o = out->o, mp.out_m = out->m, mp.out_l = out->l;
  }
  hipError_t e = launch_merge(mp, s);
  if (e != hipSuccess) return fail(BLKATTN_ERR_HIP, "merge kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

int check_idx(const blkattn_dims* d, const int32_t* idx) {
  if (idx == nullptr) {
    if (d->n_keep != 0) return fail(BLKATTN_ERR_INVALID_ARG, "n_keep is set but idx is NULL");
    return BLKATTN_OK;
  }
  if (reinterpret_cast<uintptr_t>(idx) % 4 != 0)
    return fail(BLKATTN_ERR_MISALIGNED, "idx is not 4-byte aligned");
  if (d->n_keep > 0 && d->prefix_len == 0)
    return fail(BLKATTN_ERR_INVALID_ARG, "n_keep > 0 with an empty prefix to index");
  return BLKATTN_OK;
}

// The three launches of a full-sequence step. The sequence has N = prefix_len
// rows; the block C is rows [c0, c0 + Bq); U is the other N - Bq rows.
struct SeqPlans {
  blkattn_dims du;  // U queries (block_len = N - Bq)
  blkattn_dims dc;  // C queries (block_len = Bq)
  Plan cache;       // U queries over the U keys (first step of a block)
  Plan cont;        // U queries over the C keys, from the cache (one split)
  Plan block;       // C queries over all N keys
  size_t ws = 0;
};

SeqPlans seq_plans(const blkattn_dims* d) {
  SeqPlans sp;
  const int64_t N = d->prefix_len;
  sp.du = *d;
  sp.du.block_len = (int32_t)(N - d->block_len);
  sp.du.n_keep = 0;
  sp.dc = *d;
  sp.dc.n_keep = 0;
  sp.cache = make_plan(&sp.du, N - d->block_len, false);
  blkattn_dims du1 = sp.du;
  du1.splits = 1;
  sp.cont = make_plan(&du1, d->block_len, false);
  sp.block = make_plan(&sp.dc, N, false);
  const size_t a = ws_layout(&sp.du, sp.cache.splits).total;
  const size_t b = ws_layout(&sp.dc, sp.block.splits).total;
  sp.ws = a > b ? a : b;
  return sp;
}

blkattn_tensor rows_from(const blkattn_tensor* t, int64_t row0, int eb) {
  blkattn_tensor r = *t;
  r.data = (char*)t->data + row0 * t->stride_t * eb;
  return r;
}

// Scratch of blkattn_full_noalloc: one array per device, from the code
// object's static data (each GPU the library runs on holds it until the
// process ends). In host code `scratch` only names the symbol; its device
// address on each device comes from hipGetSymbolAddress, taken once per
// device with that device current.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The current device's scratch address, or nullptr (with the error) when it
// cannot be had.
void* device_scratch(hipError_t* err) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = e != hipSuccess ? e : hipErrorInvalidDevice;
    return nullptr;
  }
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? ptr : nullptr;
  });
  *err = g_scratch_err[dev];
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int blkattn_abi_version(void) { return BLKATTN_ABI_VERSION; }

const char* blkattn_last_error(void) { return g_err; }

const char* blkattn_strerror(int status) {
  switch (status) {
    case BLKATTN_OK: return "ok";
    case BLKATTN_ERR_INVALID_ARG: return "invalid argument";
    case BLKATTN_ERR_UNSUPPORTED: return "unsupported dtype or head_dim";
    case BLKATTN_ERR_MISALIGNED: return "pointer or stride not 16-byte aligned";
    case BLKATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case BLKATTN_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

void blkattn_set_kernel_events(void* start, void* stop) {
  g_ev_start = start;
  g_ev_stop = stop;
}

int blkattn_plan_splits(const blkattn_dims* d, int op) {
  int st = check_dims(d);
  if (st != BLKATTN_OK) return st;
  if (op == BLKATTN_OP_SELECT) return select_plan((int64_t)d->batch * d->kv_heads, d->prefix_len).chunks;
  if (op == BLKATTN_OP_SEQUENCE) {
    if (d->block_len > d->prefix_len) return fail(BLKATTN_ERR_INVALID_ARG, "block_len exceeds prefix_len");
    if (d->prefix_len - d->block_len > INT32_MAX) return fail(BLKATTN_ERR_UNSUPPORTED, "sequence too long");
    return seq_plans(d).block.splits;
  }
  if (op != BLKATTN_OP_FULL && op != BLKATTN_OP_PREFIX_PARTIAL)
    return fail(BLKATTN_ERR_INVALID_ARG, "unknown op %d", op);
  const bool indexed = d->n_keep > 0;
  const int64_t n_pre = indexed ? d->n_keep : d->prefix_len;
  const int64_t n_keys = n_pre + (op == BLKATTN_OP_FULL ? d->block_len : 0);
  return make_plan(d, n_keys, indexed).splits;
}

size_t blkattn_workspace_bytes(const blkattn_dims* d, int op) {
  const int s = blkattn_plan_splits(d, op);
  if (s < 1) return 0;
  if (op == BLKATTN_OP_SELECT) return select_plan((int64_t)d->batch * d->kv_heads, d->prefix_len).ws_bytes;
  if (op == BLKATTN_OP_SEQUENCE) return seq_plans(d).ws;
  return ws_layout(d, s).total;
}

int blkattn_full_noalloc(const blkattn_dims* d, const blkattn_tensor* q, const blkattn_tensor* k_pre,
                         const blkattn_tensor* v_pre, const int32_t* idx, const blkattn_tensor* k_blk,
                         const blkattn_tensor* v_blk, const blkattn_tensor* o, float* lse, void* stream) {
  int st = check_dims(d);
  if (st) return st;
  if (d->batch == 0 || d->q_heads == 0 || d->block_len == 0) return ok();
  const size_t need = blkattn_workspace_bytes(d, BLKATTN_OP_FULL);
  if (need > kNoAllocScratchBytes)
    return fail(BLKATTN_ERR_WORKSPACE,
                "blkattn_full_noalloc: these dims need %zu bytes of scratch, more than its %zu; "
                "use blkattn_full with a workspace",
                need, kNoAllocScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    hipError_t e;
    ws = device_scratch(&e);
    if (ws == nullptr)
      return fail(BLKATTN_ERR_HIP, "blkattn_full_noalloc: no scratch address on this device: %s",
                  hipGetErrorString(e));
  }
  return blkattn_full(d, q, k_pre, v_pre, idx, k_blk, v_blk, o, lse, ws, need, stream);
}

int blkattn_full(const blkattn_dims* d, const blkattn_tensor* q, const blkattn_tensor* k_pre,
                 const blkattn_tensor* v_pre, const int32_t* idx, const blkattn_tensor* k_blk,
                 const blkattn_tensor* v_blk, const blkattn_tensor* o, float* lse, void* workspace,
                 size_t workspace_bytes, void* stream) {
  int st = check_dims(d);
  if (st) return st;
  const int eb = elt_bytes(d->dtype);
  const int64_t n_pre = prefix_keys(d, idx);
  if (d->batch == 0 || d->q_heads == 0 || d->block_len == 0) return ok();
  if ((st = check_tensor(q, "q", eb, 1))) return st;
  if ((st = check_tensor(k_pre, "k_pre", eb, n_pre))) return st;
  if ((st = check_tensor(v_pre, "v_pre", eb, n_pre))) return st;
  if ((st = check_idx(d, idx))) return st;
  if ((st = check_tensor(k_blk, "k_blk", eb, 1))) return st;
  if ((st = check_tensor(v_blk, "v_blk", eb, 1))) return st;
  if ((st = check_tensor(o, "o", eb, 1))) return st;
  if (lse != nullptr && reinterpret_cast<uintptr_t>(lse) % 4 != 0)
    return fail(BLKATTN_ERR_MISALIGNED, "lse is not 4-byte aligned");
  const int64_t n_keys = n_pre + d->block_len;
  const Plan pl = make_plan(d, n_keys, idx != nullptr);
  if ((st = check_workspace(ws_layout(d, pl.splits), workspace, workspace_bytes))) return st;
  AttnParams p = attn_params(d, q, pl);
  fill_keys(p.keys, d, k_pre, v_pre, idx, k_blk, v_blk, n_pre, d->block_len);
  return run_splits(d, p, pl, o, lse, nullptr, workspace, (hipStream_t)stream);
}

int blkattn_prefix_partial(const blkattn_dims* d, const blkattn_tensor* q, const blkattn_tensor* k_pre,
                           const blkattn_tensor* v_pre, const int32_t* idx, const blkattn_partial* out,
                           void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_dims(d);
  if (st) return st;
  const int eb = elt_bytes(d->dtype);
  const int64_t n_pre = prefix_keys(d, idx);
  if (d->batch == 0 || d->q_heads == 0 || d->block_len == 0) return ok();
  const int64_t rows = (int64_t)d->batch * d->q_heads * d->block_len;
  if ((st = check_tensor(q, "q", eb, 1))) return st;
  if ((st = check_tensor(k_pre, "k_pre", eb, n_pre))) return st;
  if ((st = check_tensor(v_pre, "v_pre", eb, n_pre))) return st;
  if ((st = check_idx(d, idx))) return st;
  if ((st = check_partial(out, "out", rows))) return st;
  hipStream_t s = (hipStream_t)stream;
  if (n_pre == 0) {
    hipError_t e = launch_fill_empty(out->o, out->m, out->l, rows, d->head_dim, s);
    if (e != hipSuccess) return fail(BLKATTN_ERR_HIP, "fill kernel launch failed: %s", hipGetErrorString(e));
    return ok();
  }
  const Plan pl = make_plan(d, n_pre, idx != nullptr);
  if ((st = check_workspace(ws_layout(d, pl.splits), workspace, workspace_bytes))) return st;
  AttnParams p = attn_params(d, q, pl);
  fill_keys(p.keys, d, k_pre, v_pre, idx, nullptr, nullptr, n_pre, 0);
  return run_splits(d, p, pl, nullptr, nullptr, out, workspace, s);
}

int blkattn_block_partial(const blkattn_dims* d, const blkattn_tensor* q, const blkattn_tensor* k_blk,
                          const blkattn_tensor* v_blk, const blkattn_partial* out, void* stream) {
  int st = check_dims(d);
  if (st) return st;
  const int eb = elt_bytes(d->dtype);
  if (d->batch == 0 || d->q_heads == 0 || d->block_len == 0) return ok();
  const int64_t rows = (int64_t)d->batch * d->q_heads * d->block_len;
  if ((st = check_tensor(q, "q", eb, 1))) return st;
  if ((st = check_tensor(k_blk, "k_blk", eb, 1))) return st;
  if ((st = check_tensor(v_blk, "v_blk", eb, 1))) return st;
  if ((st = check_partial(out, "out", rows))) return st;
  blkattn_dims d1 = *d;
  d1.splits = 1;  // no workspace on this path: one split over the block's keys
  const Plan pl = make_plan(&d1, d->block_len, false);
  AttnParams p = attn_params(&d1, q, pl);
  fill_keys(p.keys, &d1, nullptr, nullptr, nullptr, k_blk, v_blk, 0, d->block_len);
  p.out.mode = kOutPartial;
  p.out.po = out->o, p.out.pm = out->m, p.out.pl = out->l;
  p.out.split_rows = rows;
  hipStream_t s = (hipStream_t)stream;
  if (d->dtype == BLKATTN_F32) {
    hipError_t e = launch_attn_f32(p, s);
    if (e != hipSuccess) return fail(BLKATTN_ERR_HIP, "attention kernel launch failed: %s", hipGetErrorString(e));
  } else {
    hipError_t e = launch_attn_bf16(p, pl.waves, s);
    if (e != hipSuccess) return fail(BLKATTN_ERR_HIP, "attention kernel launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}

int blkattn_block_step(const blkattn_dims* d, const blkattn_tensor* q, const blkattn_tensor* k_blk,
                       const blkattn_tensor* v_blk, const blkattn_partial* cached, const blkattn_tensor* o,
                       float* lse, void* stream) {
  int st = check_dims(d);
  if (st) return st;
  const int eb = elt_bytes(d->dtype);
  if (d->batch == 0 || d->q_heads == 0 || d->block_len == 0) return ok();
  const int64_t rows = (int64_t)d->batch * d->q_heads * d->block_len;
  if ((st = check_tensor(q, "q", eb, 1))) return st;
  if ((st = check_tensor(k_blk, "k_blk", eb, 1))) return st;
  if ((st = check_tensor(v_blk, "v_blk", eb, 1))) return st;
  if ((st = check_partial(cached, "cached", rows))) return st;
  if ((st = check_tensor(o, "o", eb, 1))) return st;
  if (lse != nullptr && reinterpret_cast<uintptr_t>(lse) % 4 != 0)
    return fail(BLKATTN_ERR_MISALIGNED, "lse is not 4-byte aligned");
  blkattn_dims d1 = *d;
  d1.splits = 1;  // the block's keys in one split, continuing the cached state
  const Plan pl = make_plan(&d1, d->block_len, false);
  AttnParams p = attn_params(&d1, q, pl);
  fill_keys(p.keys, &d1, nullptr, nullptr, nullptr, k_blk, v_blk, 0, d->block_len);
  p.init_o = cached->o, p.init_m = cached->m, p.init_l = cached->l;
  p.out.mode = kOutFinal;
  p.out.o = o->data;
  p.out.o_sb = o->stride_b, p.out.o_sh = o->stride_h, p.out.o_st = o->stride_t;
  p.out.lse = lse;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = d->dtype == BLKATTN_F32 ? launch_attn_f32(p, s) : launch_attn_bf16(p, pl.waves, s);
  if (e != hipSuccess) return fail(BLKATTN_ERR_HIP, "attention kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

int blkattn_merge(const blkattn_dims* d, const blkattn_partial* a, const blkattn_partial* b,
                  const blkattn_tensor* o, float* lse, const blkattn_partial* ab, void* stream) {
  int st = check_dims(d);
  if (st) return st;
  if (d->batch == 0 || d->q_heads == 0 || d->block_len == 0) return ok();
  const int64_t rows = (int64_t)d->batch * d->q_heads * d->block_len;
  if ((st = check_partial(a, "a", rows))) return st;
  if ((st = check_partial(b, "b", rows))) return st;
  if (o != nullptr && (st = check_tensor(o, "o", elt_bytes(d->dtype), 1))) return st;
  if (lse != nullptr && reinterpret_cast<uintptr_t>(lse) % 4 != 0)
    return fail(BLKATTN_ERR_MISALIGNED, "lse is not 4-byte aligned");
  if (ab != nullptr && (st = check_partial(ab, "ab", rows))) return st;
  if (o == nullptr && lse == nullptr && ab == nullptr) return ok();
  MergeParams mp{};
  mp.batch = d->batch, mp.q_heads = d->q_heads, mp.block_len = d->block_len, mp.head_dim = d->head_dim;
  mp.rows = identity_rows(d);
  mp.nsrc = 2;
  mp.strided = 0;
  mp.src_o[0] = a->o, mp.src_m[0] = a->m, mp.src_l[0] = a->l;
  mp.src_o[1] = b->o, mp.src_m[1] = b->m, mp.src_l[1] = b->l;
  mp.out_dtype = d->dtype;
  if (o != nullptr) {
    mp.o_final = o->data;
    mp.o_sb = o->stride_b, mp.o_sh = o->stride_h, mp.o_st = o->stride_t;
  }
  mp.lse = lse;
  if (ab != nullptr) mp.out_o = ab->o, mp.out_m = ab->m, mp.out_l = ab->l;
  hipError_t e = launch_merge(mp, (hipStream_t)stream);
  if (e != hipSuccess) return fail(BLKATTN_ERR_HIP, "merge kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

int blkattn_sequence_step(const blkattn_dims* d, int64_t block_start, int gen_step, const blkattn_tensor* q,
                          const blkattn_tensor* k, const blkattn_tensor* v, const blkattn_partial* cache,
                          const blkattn_tensor* o, float* lse, void* workspace, size_t workspace_bytes,
                          void* stream) {
  int st = check_dims(d);
  if (st) return st;
  const int64_t N = d->prefix_len;
  const int64_t Bq = d->block_len;
  if (d->n_keep != 0) return fail(BLKATTN_ERR_INVALID_ARG, "n_keep must be 0 for a sequence step");
  if (d->batch == 0 || d->q_heads == 0 || N == 0) return ok();
  if (Bq == 0) return fail(BLKATTN_ERR_INVALID_ARG, "a sequence step needs a block (block_len > 0)");
  if (block_start < 0 || block_start > N - Bq)
    return fail(BLKATTN_ERR_INVALID_ARG, "block rows [%lld, %lld) do not lie in the %lld sequence rows",
                (long long)block_start, (long long)(block_start + Bq), (long long)N);
  if (N - Bq > INT32_MAX) return fail(BLKATTN_ERR_UNSUPPORTED, "sequence too long");
  const int eb = elt_bytes(d->dtype);
  const int64_t nu = N - Bq;
  if ((st = check_tensor(q, "q", eb, 1))) return st;
  if ((st = check_tensor(k, "k", eb, 1))) return st;
  if ((st = check_tensor(v, "v", eb, 1))) return st;
  if ((st = check_tensor(o, "o", eb, 1))) return st;
  if ((st = check_partial(cache, "cache", nu))) return st;
  if (lse != nullptr && reinterpret_cast<uintptr_t>(lse) % 4 != 0)
    return fail(BLKATTN_ERR_MISALIGNED, "lse is not 4-byte aligned");
  const SeqPlans sp = seq_plans(d);
  if (sp.ws > 0 && (st = check_workspace(WsLayout{0, 0, 0, sp.ws}, workspace, workspace_bytes))) return st;
  hipStream_t s = (hipStream_t)stream;
  const RowMap rows_u{block_start, Bq, N};  // U queries skip the block's rows
  const RowMap rows_c{0, block_start, N};   // C queries start at the block's first row
  if (nu > 0) {
    if (gen_step) {
      // first step of the block: the cache is the U queries' state over the U keys
      AttnParams p = attn_params(&sp.du, q, sp.cache);
      p.rows = rows_u;
      fill_keys(p.keys, &sp.du, k, v, nullptr, nullptr, nullptr, nu, 0);
      p.keys.p_rows = N;
      p.keys.k_hole = block_start, p.keys.k_hole_len = Bq;
      if ((st = run_splits(&sp.du, p, sp.cache, nullptr, nullptr, cache, workspace, s))) return st;
    }
    // U queries: start from the cache and attend the block's keys only
    const blkattn_tensor kc = rows_from(k, block_start, eb), vc = rows_from(v, block_start, eb);
    blkattn_dims du1 = sp.du;
    du1.splits = 1;
    AttnParams p = attn_params(&du1, q, sp.cont);
    p.rows = rows_u;
    fill_keys(p.keys, &du1, nullptr, nullptr, nullptr, &kc, &vc, 0, (int32_t)Bq);
    p.init_o = cache->o, p.init_m = cache->m, p.init_l = cache->l;
    if ((st = run_splits(&du1, p, sp.cont, o, lse, nullptr, nullptr, s))) return st;
  }
  // C queries: every key of the sequence
  AttnParams p = attn_params(&sp.dc, q, sp.block);
  p.rows = rows_c;
  fill_keys(p.keys, &sp.dc, k, v, nullptr, nullptr, nullptr, N, 0);
  return run_splits(&sp.dc, p, sp.block, o, lse, nullptr, workspace, s);
}

int blkattn_prefix_mass(const blkattn_dims* d, const blkattn_tensor* q, const blkattn_tensor* k_pre,
                        const float* lse, float* mass, void* stream) {
  int st = check_dims(d);
  if (st) return st;
  const int eb = elt_bytes(d->dtype);
  if (d->batch == 0 || d->prefix_len == 0) return ok();
  if ((st = check_tensor(k_pre, "k_pre", eb, 1))) return st;
  if (mass == nullptr) return fail(BLKATTN_ERR_INVALID_ARG, "mass is NULL");
  if (reinterpret_cast<uintptr_t>(mass) % 4 != 0) return fail(BLKATTN_ERR_MISALIGNED, "mass is not 4-byte aligned");
  const int64_t groups = (int64_t)d->batch * d->kv_heads;
  hipStream_t s = (hipStream_t)stream;
  if (d->q_heads == 0 || d->block_len == 0) return ok();  // degenerate: no-op
  if ((st = check_tensor(q, "q", eb, 1))) return st;
  if (lse == nullptr) return fail(BLKATTN_ERR_INVALID_ARG, "lse is NULL");
  if (reinterpret_cast<uintptr_t>(lse) % 4 != 0) return fail(BLKATTN_ERR_MISALIGNED, "lse is not 4-byte aligned");
  const int64_t R = (int64_t)(d->q_heads / d->kv_heads) * d->block_len;
  if (R > INT32_MAX) return fail(BLKATTN_ERR_UNSUPPORTED, "too many query rows per kv head");
  MassParams p{};
  p.batch = d->batch, p.q_heads = d->q_heads, p.kv_heads = d->kv_heads, p.group = d->q_heads / d->kv_heads;
  p.head_dim = d->head_dim, p.block_len = d->block_len, p.dtype = d->dtype;
  p.q = q->data, p.q_sb = q->stride_b, p.q_sh = q->stride_h, p.q_st = q->stride_t;
  p.k = k_pre->data, p.k_sb = k_pre->stride_b, p.k_sh = k_pre->stride_h, p.k_st = k_pre->stride_t;
  p.n_keys = d->prefix_len;
  p.lse = lse, p.mass = mass;
  p.scale = d->scale;
  p.scale_log2 = (float)((double)d->scale * 1.4426950408889634);
  p.tiles = (int)((d->prefix_len + mass_tile_keys() - 1) / mass_tile_keys());
  int64_t splits = (kComputeUnits + groups - 1) / groups;
  if (splits > p.tiles) splits = p.tiles;
  if (splits < 1) splits = 1;
  p.splits = (int)splits;
  hipError_t e = launch_mass(p, s);
  if (e != hipSuccess) return fail(BLKATTN_ERR_HIP, "mass kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

int blkattn_select_retained(const blkattn_dims* d, const float* mass, int32_t* idx, void* workspace,
                            size_t workspace_bytes, void* stream) {
  int st = check_dims(d);
  if (st) return st;
  if (d->batch == 0 || d->n_keep == 0) return ok();
  if (d->n_keep > d->prefix_len)
    return fail(BLKATTN_ERR_INVALID_ARG, "n_keep (%d) exceeds prefix_len (%lld)", d->n_keep,
                (long long)d->prefix_len);
  if (d->prefix_len > INT32_MAX) return fail(BLKATTN_ERR_UNSUPPORTED, "prefix_len does not fit int32 indices");
  if (mass == nullptr || idx == nullptr) return fail(BLKATTN_ERR_INVALID_ARG, "mass or idx is NULL");
  if (reinterpret_cast<uintptr_t>(mass) % 4 != 0 || reinterpret_cast<uintptr_t>(idx) % 4 != 0)
    return fail(BLKATTN_ERR_MISALIGNED, "mass and idx must be 4-byte aligned");
  const int64_t groups = (int64_t)d->batch * d->kv_heads;
  const size_t need = select_plan(groups, d->prefix_len).ws_bytes;
  if (d->n_keep < d->prefix_len) {
    if (workspace == nullptr || workspace_bytes < need)
      return fail(BLKATTN_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                  workspace == nullptr ? (size_t)0 : workspace_bytes);
    if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
      return fail(BLKATTN_ERR_MISALIGNED, "workspace is not 16-byte aligned");
  }
  hipError_t e = launch_select(mass, idx, workspace, groups, d->prefix_len, d->n_keep, (hipStream_t)stream);
  if (e != hipSuccess) return fail(BLKATTN_ERR_HIP, "selection kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

int blkattn_gather_prefix(const blkattn_dims* d, const blkattn_tensor* k_full, const blkattn_tensor* v_full,
                          const int32_t* idx, const blkattn_tensor* k_out, const blkattn_tensor* v_out,
                          void* stream) {
  int st = check_dims(d);
  if (st) return st;
  const int eb = elt_bytes(d->dtype);
  if (d->batch == 0 || d->n_keep == 0) return ok();
  if (idx == nullptr) return fail(BLKATTN_ERR_INVALID_ARG, "idx is NULL");
  if ((st = check_idx(d, idx))) return st;
  if ((st = check_tensor(k_full, "k_full", eb, 1))) return st;
  if ((st = check_tensor(v_full, "v_full", eb, 1))) return st;
  if ((st = check_tensor(k_out, "k_out", eb, 1))) return st;
  if ((st = check_tensor(v_out, "v_out", eb, 1))) return st;
  GatherParams gp{};
  gp.batch = d->batch, gp.kv_heads = d->kv_heads, gp.head_dim = d->head_dim, gp.elt_bytes = eb;
  gp.p_rows = d->prefix_len, gp.n_keep = d->n_keep, gp.idx = idx;
  gp.k_full = k_full->data, gp.kf_sb = k_full->stride_b, gp.kf_sh = k_full->stride_h, gp.kf_st = k_full->stride_t;
  gp.v_full = v_full->data, gp.vf_sb = v_full->stride_b, gp.vf_sh = v_full->stride_h, gp.vf_st = v_full->stride_t;
  gp.k_out = k_out->data, gp.ko_sb = k_out->stride_b, gp.ko_sh = k_out->stride_h, gp.ko_st = k_out->stride_t;
  gp.v_out = v_out->data, gp.vo_sb = v_out->stride_b, gp.vo_sh = v_out->stride_h, gp.vo_st = v_out->stride_t;
  hipError_t e = launch_gather(gp, (hipStream_t)stream);
  if (e != hipSuccess) return fail(BLKATTN_ERR_HIP, "gather kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
