// C ABI: host-side validation (before any HIP call), launch planning and dispatch.
#include <math.h>
#include <stdint.h>
#include <mutex>
#include "kvb.h"
#include "kvb_launch.h"

namespace {

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

kvb_status check_pool(const kvb_pool* p) {
  if (!p) return KVB_ERR_NULL;
  if (!p->k || !p->v) return KVB_ERR_NULL;
  if (p->dtype != KVB_FP16 && p->dtype != KVB_BF16) return KVB_ERR_UNSUPPORTED;
  if (p->block_size != 16) return KVB_ERR_UNSUPPORTED;
  if (p->head_dim != 64 && p->head_dim != 96 && p->head_dim != 128) return KVB_ERR_UNSUPPORTED;
  if (p->num_kv_heads <= 0 || p->num_blocks <= 0) return KVB_ERR_INVALID;
  if (p->block_stride < (int64_t)p->num_kv_heads * 16 * p->head_dim) return KVB_ERR_INVALID;
  if (p->block_stride % 8 != 0) return KVB_ERR_INVALID;
  if (p->block_stride > 0x7fffffffLL) return KVB_ERR_INVALID;   // kernels take it as 32 bits
  if (!aligned16(p->k) || !aligned16(p->v)) return KVB_ERR_INVALID;
  return KVB_OK;
}

kvb_status check_pool_q8(const kvb_pool_q8* p, int bits = 8) {
  if (!p) return KVB_ERR_NULL;
  if (!p->k || !p->v || !p->v_scale || !p->k_scale) return KVB_ERR_NULL;
  if (p->block_size != 16) return KVB_ERR_UNSUPPORTED;
  if (p->head_dim != 64 && p->head_dim != 96 && p->head_dim != 128) return KVB_ERR_UNSUPPORTED;
  if (p->num_kv_heads <= 0 || p->num_blocks <= 0) return KVB_ERR_INVALID;
  if (p->block_stride < (int64_t)p->num_kv_heads * 16 * p->head_dim * bits / 8) return KVB_ERR_INVALID;
  if (p->block_stride % 16 != 0) return KVB_ERR_INVALID;
  if (p->block_stride > 0x7fffffffLL) return KVB_ERR_INVALID;
  if (!aligned16(p->k) || !aligned16(p->v) || !aligned16(p->v_scale) || !aligned16(p->k_scale))
    return KVB_ERR_INVALID;
  return KVB_OK;
}

kvb_status check_scale(float scale) {
  if (!isfinite(scale) || scale < 0.f) return KVB_ERR_INVALID;
  return KVB_OK;
}

kvb_status launch_status(hipError_t e) { return e == hipSuccess ? KVB_OK : KVB_ERR_LAUNCH; }

// Decode plan: the balanced stream form for batches it covers, else the split form.
struct DecodePlan {
  bool stream;
  int sb, ns;             // split form
  kvb::StreamPlan sp;     // stream form
  int64_t bytes;          // workspace
};
DecodePlan decode_plan_for(int batch, int hkv, int hq, int d, int max_ctx, int split_blocks) {
  DecodePlan r{};
  r.stream = kvb::decode_use_stream(batch);
  if (r.stream) {
    r.sp = kvb::decode_stream_plan(batch, hkv, hq, d, max_ctx, split_blocks);
    r.bytes = r.sp.bytes;
  } else {
    kvb::decode_plan(batch, hkv, hq, max_ctx, split_blocks, &r.sb, &r.ns);
    r.bytes = kvb::decode_ws_bytes(batch, hq, d, r.ns);
  }
  return r;
}
hipError_t launch_decode_plan(const DecodePlan& pl, const kvb_pool& p, const void* q, void* out,
                              const int32_t* ctx, const int32_t* bt, int bt_stride, int batch,
                              int hq, int max_ctx, float scale, void* ws, hipStream_t s) {
  if (pl.stream)
    return kvb::launch_decode_stream(p, 0, kvb::DecScales{nullptr, nullptr}, q, out, ctx, bt,
                                     bt_stride, batch, hq, max_ctx, pl.sp, scale, ws, s);
  return kvb::launch_decode(p, q, out, ctx, bt, bt_stride, batch, hq, max_ctx, pl.sb, pl.ns, scale,
                           ws, s);
}

}  // namespace

extern "C" {

const char* kvb_status_str(kvb_status s) {
  switch (s) {
    case KVB_OK: return "ok";
    case KVB_ERR_NULL: return "null pointer";
    case KVB_ERR_INVALID: return "invalid argument";
    case KVB_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVB_ERR_WORKSPACE: return "workspace missing or too small";
    case KVB_ERR_LAUNCH: return "kernel launch failed";
    case KVB_ERR_TOO_LARGE: return "needs more scratch than the static device buffer holds";
  }
  return "unknown status";
}

const char* kvb_version(void) { return "0.1.0"; }

kvb_status kvb_write_kv(const kvb_pool* pool, const void* k_new, const void* v_new,
                        const int64_t* slot_mapping, int32_t num_tokens, void* stream) {
  kvb_status st = check_pool(pool);
  if (st != KVB_OK) return st;
  if (num_tokens < 0) return KVB_ERR_INVALID;
  if (num_tokens == 0) return KVB_OK;
  if (!k_new || !v_new || !slot_mapping) return KVB_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new) || ((uintptr_t)slot_mapping & 7u)) return KVB_ERR_INVALID;
  return launch_status(kvb::launch_write_kv(*pool, k_new, v_new, slot_mapping, num_tokens,
                                            (hipStream_t)stream));
}

size_t kvb_paged_prefill_workspace_size(int32_t batch, int32_t num_q_heads, int32_t head_dim,
                                        int32_t total_q, int32_t max_prefix_len) {
  (void)head_dim; (void)max_prefix_len;
  return (size_t)kvb::prefill_plan_bytes(batch, num_q_heads, total_q);
}

}  // extern "C"

namespace {

// kvb_paged_prefill, with `slots` (NULL: none) the chunk's slot scatter fused in
kvb_status paged_prefill_impl(const kvb_pool* pool, const void* q, const void* k_new,
                              const void* v_new, void* out, const int64_t* slots, bool want_slots,
                              const int32_t* cu_q_lens, const int32_t* prefix_lens,
                              const int32_t* block_tables, int32_t block_table_stride, int32_t batch,
                              int32_t num_q_heads, int32_t total_q, int32_t max_q_len,
                              int32_t max_prefix_len, float scale, void* workspace,
                              size_t workspace_bytes, void* stream) {
  kvb_status st = check_pool(pool);
  if (st != KVB_OK) return st;
  if (batch < 0 || total_q < 0 || max_q_len < 0 || max_prefix_len < 0 || num_q_heads <= 0)
    return KVB_ERR_INVALID;
  if (num_q_heads % pool->num_kv_heads != 0) return KVB_ERR_INVALID;
  if ((st = check_scale(scale)) != KVB_OK) return st;
  if (batch == 0 || total_q == 0) return KVB_OK;
  if (!q || !k_new || !v_new || !out || !cu_q_lens || !prefix_lens || !block_tables)
    return KVB_ERR_NULL;
  if (want_slots && !slots) return KVB_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out) ||
      ((uintptr_t)cu_q_lens & 3u) || ((uintptr_t)prefix_lens & 3u) || ((uintptr_t)block_tables & 3u) ||
      ((uintptr_t)slots & 7u))
    return KVB_ERR_INVALID;
  if (max_q_len > total_q) return KVB_ERR_INVALID;
  if (block_table_stride < (max_prefix_len + 15) / 16 || block_table_stride < 0) return KVB_ERR_INVALID;
  // the workspace is optional (it holds the dispatch plan); one that is passed must be big enough
  const size_t need = kvb_paged_prefill_workspace_size(batch, num_q_heads, pool->head_dim, total_q,
                                                       max_prefix_len);
  if (workspace && workspace_bytes < need) return KVB_ERR_WORKSPACE;
  if (workspace && !aligned16(workspace)) return KVB_ERR_INVALID;
  if (max_q_len == 0) return KVB_OK;
  return launch_status(kvb::launch_prefill(*pool, q, k_new, v_new, out, cu_q_lens, prefix_lens,
                                           block_tables, block_table_stride, batch, num_q_heads,
                                           total_q, max_q_len, max_prefix_len, scale,
                                           need > 0 ? workspace : nullptr, (hipStream_t)stream,
                                           want_slots ? slots : nullptr));
}

}  // namespace

extern "C" {

kvb_status kvb_paged_prefill(const kvb_pool* pool, const void* q, const void* k_new,
                             const void* v_new, void* out, const int32_t* cu_q_lens,
                             const int32_t* prefix_lens, const int32_t* block_tables,
                             int32_t block_table_stride, int32_t batch, int32_t num_q_heads,
                             int32_t total_q, int32_t max_q_len, int32_t max_prefix_len,
                             float scale, void* workspace, size_t workspace_bytes, void* stream) {
  return paged_prefill_impl(pool, q, k_new, v_new, out, nullptr, false, cu_q_lens, prefix_lens,
                            block_tables, block_table_stride, batch, num_q_heads, total_q, max_q_len,
                            max_prefix_len, scale, workspace, workspace_bytes, stream);
}

kvb_status kvb_paged_prefill_write(const kvb_pool* pool, const void* q, const void* k_new,
                                   const void* v_new, void* out, const int64_t* slot_mapping,
                                   const int32_t* cu_q_lens, const int32_t* prefix_lens,
                                   const int32_t* block_tables, int32_t block_table_stride,
                                   int32_t batch, int32_t num_q_heads, int32_t total_q,
                                   int32_t max_q_len, int32_t max_prefix_len, float scale,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  return paged_prefill_impl(pool, q, k_new, v_new, out, slot_mapping, true, cu_q_lens, prefix_lens,
                            block_tables, block_table_stride, batch, num_q_heads, total_q, max_q_len,
                            max_prefix_len, scale, workspace, workspace_bytes, stream);
}

kvb_status kvb_paged_prefill_pooled(const kvb_pool* pool, const void* q, void* out,
                                    const int32_t* cu_q_lens, const int32_t* prefix_lens,
                                    const int32_t* block_tables, int32_t block_table_stride,
                                    int32_t batch, int32_t num_q_heads, int32_t total_q,
                                    int32_t max_q_len, int32_t max_prefix_len, float scale,
                                    void* stream) {
  kvb_status st = check_pool(pool);
  if (st != KVB_OK) return st;
  if (batch < 0 || total_q < 0 || max_q_len < 0 || max_prefix_len < 0 || num_q_heads <= 0)
    return KVB_ERR_INVALID;
  if (num_q_heads % pool->num_kv_heads != 0) return KVB_ERR_INVALID;
  if ((st = check_scale(scale)) != KVB_OK) return st;
  if (batch == 0 || total_q == 0) return KVB_OK;
  if (!q || !out || !cu_q_lens || !prefix_lens || !block_tables) return KVB_ERR_NULL;
  if (!aligned16(q) || !aligned16(out) || ((uintptr_t)cu_q_lens & 3u) ||
      ((uintptr_t)prefix_lens & 3u) || ((uintptr_t)block_tables & 3u))
    return KVB_ERR_INVALID;
  if (max_q_len > total_q) return KVB_ERR_INVALID;
  // each row must reach prefix_lens[b] + C_b tokens (not checkable on the host; keys past
  // block_table_stride * 16 are never read)
  if (block_table_stride < (max_prefix_len + 15) / 16 || block_table_stride < 0) return KVB_ERR_INVALID;
  if (max_q_len == 0) return KVB_OK;
  return launch_status(kvb::launch_prefill_pooled(*pool, q, out, cu_q_lens, prefix_lens,
                                                  block_tables, block_table_stride, batch,
                                                  num_q_heads, total_q, max_q_len, scale,
                                                  (hipStream_t)stream));
}

size_t kvb_paged_decode_workspace_size(int32_t batch, int32_t num_kv_heads, int32_t num_q_heads,
                                       int32_t head_dim, int32_t max_context_len,
                                       int32_t split_blocks) {
  // (every context empty, max_context_len 0: the plan still writes the zero rows, through
  // its header and merge, so it takes the same workspace as any other)
  if (batch <= 0 || num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % num_kv_heads ||
      max_context_len < 0 || split_blocks < 0)
    return 0;
  return (size_t)decode_plan_for(batch, num_kv_heads, num_q_heads, head_dim, max_context_len,
                                 split_blocks).bytes;
}

kvb_status kvb_paged_decode(const kvb_pool* pool, const void* q, void* out,
                            const int32_t* context_lens, const int32_t* block_tables,
                            int32_t block_table_stride, int32_t batch, int32_t num_q_heads,
                            int32_t max_context_len, int32_t split_blocks, float scale,
                            void* workspace, size_t workspace_bytes, void* stream) {
  kvb_status st = check_pool(pool);
  if (st != KVB_OK) return st;
  if (batch < 0 || num_q_heads <= 0 || max_context_len < 0 || split_blocks < 0)
    return KVB_ERR_INVALID;
  if (num_q_heads % pool->num_kv_heads != 0) return KVB_ERR_INVALID;
  if ((st = check_scale(scale)) != KVB_OK) return st;
  if (batch == 0) return KVB_OK;
  if (!q || !out || !context_lens || !block_tables) return KVB_ERR_NULL;
  if (!aligned16(q) || !aligned16(out) || ((uintptr_t)context_lens & 3u) ||
      ((uintptr_t)block_tables & 3u))
    return KVB_ERR_INVALID;
  if (block_table_stride < (max_context_len + 15) / 16 || block_table_stride <= 0)
    return KVB_ERR_INVALID;
  const DecodePlan pl = decode_plan_for(batch, pool->num_kv_heads, num_q_heads, pool->head_dim,
                                        max_context_len, split_blocks);
  const size_t need = (size_t)pl.bytes;
  if (need > 0 && (!workspace || workspace_bytes < need)) return KVB_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return KVB_ERR_INVALID;
  return launch_status(launch_decode_plan(pl, *pool, q, out, context_lens, block_tables,
                                          block_table_stride, batch, num_q_heads, max_context_len,
                                          scale, workspace, (hipStream_t)stream));
}

}  // extern "C"

// Scratch of kvb_paged_decode_noalloc: the split partials live in this file-scope device
// array instead of a caller workspace.  In host code `scratch` only names the symbol; its
// device address (one copy per GPU) comes from hipGetSymbolAddress, taken once per device
// with that device current and kept in scratch_dev[].
static __device__ __align__(256) unsigned char scratch[KVB_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_dev[kMaxDevices];

// Device address of the current device's scratch array (NULL if it cannot be obtained).
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    scratch_dev[dev] = ptr;
  }
  return scratch_dev[dev];
}

}  // namespace

extern "C" {

kvb_status kvb_paged_decode_noalloc(const kvb_pool* pool, const void* q, void* out,
                                    const int32_t* context_lens, const int32_t* block_tables,
                                    int32_t block_table_stride, int32_t batch, int32_t num_q_heads,
                                    int32_t max_context_len, int32_t split_blocks, float scale,
                                    void* stream) {
  kvb_status st = check_pool(pool);
  if (st != KVB_OK) return st;
  if (batch < 0 || num_q_heads <= 0 || max_context_len < 0 || split_blocks < 0)
    return KVB_ERR_INVALID;
  if (num_q_heads % pool->num_kv_heads != 0) return KVB_ERR_INVALID;
  if ((st = check_scale(scale)) != KVB_OK) return st;
  if (batch == 0) return KVB_OK;
  if (!q || !out || !context_lens || !block_tables) return KVB_ERR_NULL;
  if (!aligned16(q) || !aligned16(out) || ((uintptr_t)context_lens & 3u) ||
      ((uintptr_t)block_tables & 3u))
    return KVB_ERR_INVALID;
  if (block_table_stride < (max_context_len + 15) / 16 || block_table_stride <= 0)
    return KVB_ERR_INVALID;
  const DecodePlan pl = decode_plan_for(batch, pool->num_kv_heads, num_q_heads, pool->head_dim,
                                        max_context_len, split_blocks);
  if (pl.bytes > (int64_t)KVB_NOALLOC_SCRATCH_BYTES) return KVB_ERR_TOO_LARGE;
  void* ws = nullptr;
  if (pl.bytes > 0 && !(ws = scratch_address())) return KVB_ERR_LAUNCH;
  // the decode kernels write everything the merge reads (header and partial records)
  // before it runs: nothing needs clearing
  return launch_status(launch_decode_plan(pl, *pool, q, out, context_lens, block_tables,
                                          block_table_stride, batch, num_q_heads, max_context_len,
                                          scale, ws, (hipStream_t)stream));
}

// Plan of a cascade decode: the private splits, and the shared prefix either in group
// work-groups of the same launch (grouped) or in a separate pass of the prefill kernel
// (nks key splits of ks_tiles tiles; for the grouped form, nks splits of ks_tiles blocks).
struct CascadePlan {
  bool grouped;
  int sb, ns, nks, ks_tiles;
};
static CascadePlan cascade_plans(int batch, int hkv, int hq, int max_ctx, int shared_len,
                                 int split_blocks) {
  CascadePlan c{};
  kvb::decode_plan(batch, hkv, hq, max_ctx > shared_len ? max_ctx - shared_len : 0, split_blocks,
                   &c.sb, &c.ns);
  const int shared_eff = shared_len < max_ctx ? shared_len : max_ctx;
  c.grouped = kvb::cascade_use_grouped(batch, hkv, hq, shared_eff);
  if (c.grouped)
    kvb::decode_group_plan(shared_eff, c.sb, &c.ks_tiles, &c.nks);
  else
    kvb::cascade_plan(batch, hkv, hq, shared_eff, &c.nks, &c.ks_tiles);
  return c;
}

size_t kvb_paged_decode_cascade_workspace_size(int32_t batch, int32_t num_kv_heads,
                                               int32_t num_q_heads, int32_t head_dim,
                                               int32_t max_context_len, int32_t shared_len,
                                               int32_t split_blocks) {
  if (batch <= 0 || num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % num_kv_heads ||
      max_context_len < 0 || split_blocks < 0 || shared_len < 0 || shared_len % 16)
    return 0;
  const CascadePlan c = cascade_plans(batch, num_kv_heads, num_q_heads, max_context_len,
                                      shared_len, split_blocks);
  return (size_t)kvb::cascade_ws_bytes(batch, num_q_heads, head_dim, c.nks + c.ns);
}

kvb_status kvb_paged_decode_cascade(const kvb_pool* pool, const void* q, void* out,
                                    const int32_t* context_lens, const int32_t* block_tables,
                                    int32_t block_table_stride, const int32_t* shared_blocks,
                                    int32_t shared_len, int32_t batch, int32_t num_q_heads,
                                    int32_t max_context_len, int32_t split_blocks, float scale,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  kvb_status st = check_pool(pool);
  if (st != KVB_OK) return st;
  if (batch < 0 || num_q_heads <= 0 || max_context_len < 0 || split_blocks < 0)
    return KVB_ERR_INVALID;
  if (shared_len < 0 || shared_len % 16 != 0) return KVB_ERR_INVALID;
  if (num_q_heads % pool->num_kv_heads != 0) return KVB_ERR_INVALID;
  if ((st = check_scale(scale)) != KVB_OK) return st;
  if (batch == 0) return KVB_OK;
  if (!q || !out || !context_lens || !block_tables) return KVB_ERR_NULL;
  if (shared_len > 0 && !shared_blocks) return KVB_ERR_NULL;
  if (!aligned16(q) || !aligned16(out) || ((uintptr_t)context_lens & 3u) ||
      ((uintptr_t)block_tables & 3u) || ((uintptr_t)shared_blocks & 3u))
    return KVB_ERR_INVALID;
  if (block_table_stride < (max_context_len + 15) / 16 || block_table_stride <= 0)
    return KVB_ERR_INVALID;
  const CascadePlan c = cascade_plans(batch, pool->num_kv_heads, num_q_heads, max_context_len,
                                      shared_len, split_blocks);
  const size_t need = (size_t)kvb::cascade_ws_bytes(batch, num_q_heads, pool->head_dim, c.nks + c.ns);
  if (!workspace || workspace_bytes < need) return KVB_ERR_WORKSPACE;
  if (!aligned16(workspace)) return KVB_ERR_INVALID;
  if (c.grouped)
    return launch_status(kvb::launch_decode_grouped(*pool, q, out, context_lens, block_tables,
                                                    block_table_stride, shared_blocks, shared_len,
                                                    batch, num_q_heads, max_context_len, c.sb, c.ns,
                                                    c.ks_tiles, c.nks, scale, workspace,
                                                    (hipStream_t)stream));
  return launch_status(kvb::launch_decode_cascade(*pool, q, out, context_lens, block_tables,
                                                  block_table_stride, shared_blocks, shared_len,
                                                  batch, num_q_heads, max_context_len, c.sb, c.ns,
                                                  c.nks, c.ks_tiles, scale, workspace,
                                                  (hipStream_t)stream));
}

static kvb_status write_kv_quant(const kvb_pool_q8* pool, int bits, const void* k_new,
                                 const void* v_new, int32_t dtype, const int64_t* slot_mapping,
                                 int32_t num_tokens, void* stream) {
  kvb_status st = check_pool_q8(pool, bits);
  if (st != KVB_OK) return st;
  if (dtype != KVB_FP16 && dtype != KVB_BF16) return KVB_ERR_UNSUPPORTED;
  if (num_tokens < 0) return KVB_ERR_INVALID;
  if (num_tokens == 0) return KVB_OK;
  if (!k_new || !v_new || !slot_mapping) return KVB_ERR_NULL;
  if (!aligned16(k_new) || !aligned16(v_new) || ((uintptr_t)slot_mapping & 7u)) return KVB_ERR_INVALID;
  return launch_status(kvb::launch_write_kv_q8(*pool, bits, dtype, k_new, v_new, slot_mapping,
                                               num_tokens, (hipStream_t)stream));
}

kvb_status kvb_write_kv_q8(const kvb_pool_q8* pool, const void* k_new, const void* v_new,
                           int32_t dtype, const int64_t* slot_mapping, int32_t num_tokens,
                           void* stream) {
  return write_kv_quant(pool, 8, k_new, v_new, dtype, slot_mapping, num_tokens, stream);
}

kvb_status kvb_write_kv_q4(const kvb_pool_q4* pool, const void* k_new, const void* v_new,
                           int32_t dtype, const int64_t* slot_mapping, int32_t num_tokens,
                           void* stream) {
  return write_kv_quant(pool, 4, k_new, v_new, dtype, slot_mapping, num_tokens, stream);
}

static kvb_status decode_quant(const kvb_pool_q8* pool, int bits, int32_t dtype, const void* q,
                               void* out, const int32_t* context_lens, const int32_t* block_tables,
                               int32_t block_table_stride, int32_t batch, int32_t num_q_heads,
                               int32_t max_context_len, int32_t split_blocks, float scale,
                               void* workspace, size_t workspace_bytes, void* stream) {
  kvb_status st = check_pool_q8(pool, bits);
  if (st != KVB_OK) return st;
  if (dtype != KVB_FP16 && dtype != KVB_BF16) return KVB_ERR_UNSUPPORTED;
  if (batch < 0 || num_q_heads <= 0 || max_context_len < 0 || split_blocks < 0)
    return KVB_ERR_INVALID;
  if (num_q_heads % pool->num_kv_heads != 0) return KVB_ERR_INVALID;
  if ((st = check_scale(scale)) != KVB_OK) return st;
  if (batch == 0) return KVB_OK;
  if (!q || !out || !context_lens || !block_tables) return KVB_ERR_NULL;
  if (!aligned16(q) || !aligned16(out) || ((uintptr_t)context_lens & 3u) ||
      ((uintptr_t)block_tables & 3u))
    return KVB_ERR_INVALID;
  if (block_table_stride < (max_context_len + 15) / 16 || block_table_stride <= 0)
    return KVB_ERR_INVALID;
  const DecodePlan pl = decode_plan_for(batch, pool->num_kv_heads, num_q_heads, pool->head_dim,
                                        max_context_len, split_blocks);
  const size_t need = (size_t)pl.bytes;
  if (need > 0 && (!workspace || workspace_bytes < need)) return KVB_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return KVB_ERR_INVALID;
  if (pl.stream) {
    const kvb_pool p{pool->k, pool->v, pool->block_stride, pool->num_blocks, 16, pool->num_kv_heads,
                     pool->head_dim, dtype};
    return launch_status(kvb::launch_decode_stream(
        p, bits, kvb::DecScales{pool->k_scale, pool->v_scale}, q, out, context_lens, block_tables,
        block_table_stride, batch, num_q_heads, max_context_len, pl.sp, scale, workspace,
        (hipStream_t)stream));
  }
  return launch_status(kvb::launch_decode_q8(*pool, bits, dtype, q, out, context_lens, block_tables,
                                             block_table_stride, batch, num_q_heads,
                                             max_context_len, pl.sb, pl.ns, scale, workspace,
                                             (hipStream_t)stream));
}

kvb_status kvb_paged_decode_q8(const kvb_pool_q8* pool, int32_t dtype, const void* q, void* out,
                               const int32_t* context_lens, const int32_t* block_tables,
                               int32_t block_table_stride, int32_t batch, int32_t num_q_heads,
                               int32_t max_context_len, int32_t split_blocks, float scale,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return decode_quant(pool, 8, dtype, q, out, context_lens, block_tables, block_table_stride, batch,
                      num_q_heads, max_context_len, split_blocks, scale, workspace,
                      workspace_bytes, stream);
}

kvb_status kvb_paged_decode_q4(const kvb_pool_q4* pool, int32_t dtype, const void* q, void* out,
                               const int32_t* context_lens, const int32_t* block_tables,
                               int32_t block_table_stride, int32_t batch, int32_t num_q_heads,
                               int32_t max_context_len, int32_t split_blocks, float scale,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return decode_quant(pool, 4, dtype, q, out, context_lens, block_tables, block_table_stride, batch,
                      num_q_heads, max_context_len, split_blocks, scale, workspace,
                      workspace_bytes, stream);
}

size_t kvb_paged_prefill_q8_workspace_size(int32_t batch, int32_t num_kv_heads,
                                           int32_t num_q_heads, int32_t head_dim,
                                           int32_t total_q, int32_t max_prefix_len) {
  if (batch <= 0 || num_kv_heads <= 0 || num_q_heads <= 0 || total_q <= 0 || max_prefix_len < 0 ||
      (head_dim != 64 && head_dim != 96 && head_dim != 128))
    return 0;
  // the prefill's dispatch plan only: the codes are widened inside the prefill kernel
  return (size_t)kvb::prefill_plan_bytes(batch, num_q_heads, total_q);
}

static kvb_status prefill_quant(const kvb_pool_q8* pool, int bits, int32_t dtype, const void* q,
                                const void* k_new, const void* v_new, void* out,
                                const int32_t* cu_q_lens, const int32_t* prefix_lens,
                                const int32_t* block_tables, int32_t block_table_stride,
                                int32_t batch, int32_t num_q_heads, int32_t total_q,
                                int32_t max_q_len, int32_t max_prefix_len, float scale,
                                void* workspace, size_t workspace_bytes, void* stream) {
  kvb_status st = check_pool_q8(pool, bits);
  if (st != KVB_OK) return st;
  if (dtype != KVB_FP16 && dtype != KVB_BF16) return KVB_ERR_UNSUPPORTED;
  if (batch < 0 || total_q < 0 || max_q_len < 0 || max_prefix_len < 0 || num_q_heads <= 0)
    return KVB_ERR_INVALID;
  if (num_q_heads % pool->num_kv_heads != 0) return KVB_ERR_INVALID;
  if ((st = check_scale(scale)) != KVB_OK) return st;
  if (batch == 0 || total_q == 0) return KVB_OK;
  if (!q || !k_new || !v_new || !out || !cu_q_lens || !prefix_lens || !block_tables)
    return KVB_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_new) || !aligned16(v_new) || !aligned16(out) ||
      ((uintptr_t)cu_q_lens & 3u) || ((uintptr_t)prefix_lens & 3u) || ((uintptr_t)block_tables & 3u))
    return KVB_ERR_INVALID;
  if (max_q_len > total_q) return KVB_ERR_INVALID;
  if (block_table_stride < (max_prefix_len + 15) / 16 || block_table_stride < 0) return KVB_ERR_INVALID;
  const size_t need = kvb_paged_prefill_q8_workspace_size(batch, pool->num_kv_heads, num_q_heads,
                                                          pool->head_dim, total_q, max_prefix_len);
  if (workspace && workspace_bytes < need) return KVB_ERR_WORKSPACE;
  if (workspace && !aligned16(workspace)) return KVB_ERR_INVALID;
  if (max_q_len == 0) return KVB_OK;
  return launch_status(kvb::launch_prefill_quant(*pool, bits, dtype, q, k_new, v_new, out, cu_q_lens,
                                                 prefix_lens, block_tables, block_table_stride, batch,
                                                 num_q_heads, total_q, max_q_len, scale,
                                                 need > 0 ? workspace : nullptr, (hipStream_t)stream));
}

kvb_status kvb_paged_prefill_q8(const kvb_pool_q8* pool, int32_t dtype, const void* q,
                                const void* k_new, const void* v_new, void* out,
                                const int32_t* cu_q_lens, const int32_t* prefix_lens,
                                const int32_t* block_tables, int32_t block_table_stride,
                                int32_t batch, int32_t num_q_heads, int32_t total_q,
                                int32_t max_q_len, int32_t max_prefix_len, float scale,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_quant(pool, 8, dtype, q, k_new, v_new, out, cu_q_lens, prefix_lens, block_tables,
                       block_table_stride, batch, num_q_heads, total_q, max_q_len, max_prefix_len,
                       scale, workspace, workspace_bytes, stream);
}

kvb_status kvb_paged_prefill_q4(const kvb_pool_q4* pool, int32_t dtype, const void* q,
                                const void* k_new, const void* v_new, void* out,
                                const int32_t* cu_q_lens, const int32_t* prefix_lens,
                                const int32_t* block_tables, int32_t block_table_stride,
                                int32_t batch, int32_t num_q_heads, int32_t total_q,
                                int32_t max_q_len, int32_t max_prefix_len, float scale,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_quant(pool, 4, dtype, q, k_new, v_new, out, cu_q_lens, prefix_lens, block_tables,
                       block_table_stride, batch, num_q_heads, total_q, max_q_len, max_prefix_len,
                       scale, workspace, workspace_bytes, stream);
}

// Address the device uses for p: itself for device memory, the mapped address for pinned
// host memory; NULL for memory the device cannot address (e.g. pageable host memory).
static void* device_address(void* p) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();                 // clear the sticky error of an unknown pointer
    return nullptr;
  }
  if (a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged) return p;
  if (a.type == hipMemoryTypeHost) return a.devicePointer;
  return nullptr;
}

kvb_status kvb_copy_blocks(const kvb_pool* src, const kvb_pool* dst, const int32_t* src_ids,
                           const int32_t* dst_ids, int32_t n, void* stream) {
  kvb_status st = check_pool(src);
  if (st != KVB_OK) return st;
  if ((st = check_pool(dst)) != KVB_OK) return st;
  if (src->num_kv_heads != dst->num_kv_heads || src->head_dim != dst->head_dim ||
      src->dtype != dst->dtype)
    return KVB_ERR_INVALID;
  if (n < 0) return KVB_ERR_INVALID;
  if (n == 0) return KVB_OK;
  if (!src_ids || !dst_ids) return KVB_ERR_NULL;
  if (((uintptr_t)src_ids & 3u) || ((uintptr_t)dst_ids & 3u)) return KVB_ERR_INVALID;
  // either pool may live in pinned host memory (swap): use the addresses the device sees
  kvb_pool s = *src, d = *dst;
  s.k = device_address(s.k);
  s.v = device_address(s.v);
  d.k = device_address(d.k);
  d.v = device_address(d.v);
  if (!s.k || !s.v || !d.k || !d.v) return KVB_ERR_INVALID;
  return launch_status(kvb::launch_copy_blocks(s, d, src_ids, dst_ids, n, (hipStream_t)stream));
}

kvb_status kvb_gather_kv(const kvb_pool* pool, const int32_t* block_tables,
                         int32_t block_table_stride, const int32_t* seq_lens,
                         const int32_t* cu_seq_lens, void* k_out, void* v_out, int32_t batch,
                         int32_t max_len, void* stream) {
  kvb_status st = check_pool(pool);
  if (st != KVB_OK) return st;
  if (batch < 0 || max_len < 0) return KVB_ERR_INVALID;
  if (batch == 0 || max_len == 0) return KVB_OK;
  if (!block_tables || !seq_lens || !cu_seq_lens || !k_out || !v_out) return KVB_ERR_NULL;
  if (!aligned16(k_out) || !aligned16(v_out)) return KVB_ERR_INVALID;
  if (block_table_stride < (max_len + 15) / 16) return KVB_ERR_INVALID;
  return launch_status(kvb::launch_gather_kv(*pool, block_tables, block_table_stride, seq_lens,
                                             cu_seq_lens, k_out, v_out, batch, max_len,
                                             (hipStream_t)stream));
}

}  // extern "C"
