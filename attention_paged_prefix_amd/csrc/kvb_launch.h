// Host-side launchers of the gfx950 kernels (called by the C ABI after validation).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "kvb.h"

namespace kvb {

// Compute units of the current device (queried once per device, then cached).
inline int device_cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

hipError_t launch_write_kv(const kvb_pool& p, const void* kn, const void* vn, const int64_t* slots,
                           int num_tokens, hipStream_t s);
hipError_t launch_copy_blocks(const kvb_pool& src, const kvb_pool& dst, const int32_t* src_ids,
                              const int32_t* dst_ids, int n, hipStream_t s);
hipError_t launch_gather_kv(const kvb_pool& p, const int32_t* bt, int bt_stride,
                            const int32_t* seq_lens, const int32_t* cu, void* ko, void* vo,
                            int batch, int max_len, hipStream_t s);

// Decode: split planning and workspace layout (floats: partial outputs, then (max, sum) pairs).
int decode_heads_per_wg(int G);
void decode_plan(int batch, int hkv, int hq, int max_ctx, int split_blocks_req, int* split_blocks,
                 int* nsplit);
inline int64_t decode_ws_o_floats(int batch, int hq, int d, int nsplit) {
  return (int64_t)batch * hq * nsplit * d;
}
inline int64_t decode_ws_bytes(int batch, int hq, int d, int nsplit) {
  if (nsplit <= 1) return 0;
  return (decode_ws_o_floats(batch, hq, d, nsplit) + (int64_t)batch * hq * nsplit * 2) * 4;
}
hipError_t launch_decode(const kvb_pool& p, const void* q, void* out, const int32_t* ctx,
                         const int32_t* bt, int bt_stride, int batch, int hq, int max_ctx, int sb,
                         int ns, float scale, void* ws, hipStream_t s);

// Balanced stream decode (batches of up to 1024 sequences): the batch's blocks in equal
// ranges, one per wave of a grid sized to be resident, then a merge of the partial
// records.  Workspace: a header (range length, per-sequence block-count prefix sums),
// then (max, sum) pairs and partial outputs of `records` records of min(G, 16) heads.
struct StreamPlan {
  int span;          // blocks per wave range requested (0: balanced in the kernel)
  int64_t waves;     // waves in the grid (whole work-groups on every XCD)
  int64_t resident;  // waves the device holds at once (the balanced range length's divisor)
  int64_t records;   // partial records: waves + units
  int64_t bytes;     // workspace bytes
};
struct DecScales {   // per-channel K and per-token V scales of a quantised pool (else null)
  const float* k_scale;
  const float* v_scale;
};
bool decode_use_stream(int batch);
int64_t stream_hdr_bytes(int batch);
StreamPlan decode_stream_plan(int batch, int hkv, int hq, int d, int max_ctx, int split_blocks);
// bits: 0 for the 16-bit pool, else 8 or 4 (p describes the code planes, block_stride in bytes)
hipError_t launch_decode_stream(const kvb_pool& p, int bits, const DecScales& sc, const void* q,
                                void* out, const int32_t* ctx, const int32_t* bt, int bt_stride,
                                int batch, int hq, int max_ctx, const StreamPlan& sp, float scale,
                                void* ws, hipStream_t s);

// Quantised pools (bits = 8 or 4 per code; the 4-bit pool uses the same descriptor):
// quantising slot scatter and decode (workspace as launch_decode's).
hipError_t launch_write_kv_q8(const kvb_pool_q8& p, int bits, int dtype, const void* kn,
                              const void* vn, const int64_t* slots, int num_tokens, hipStream_t s);
hipError_t launch_decode_q8(const kvb_pool_q8& p, int bits, int dtype, const void* q, void* out,
                            const int32_t* ctx, const int32_t* bt, int bt_stride, int batch, int hq,
                            int max_ctx, int sb, int ns, float scale, void* ws, hipStream_t s);
// Prefill over the 8-bit or 4-bit pool: the prefill kernel stages each prefix block's
// codes in LDS and widens them there; the workspace holds only the dispatch plan
// (prefill_plan_bytes).
hipError_t launch_prefill_quant(const kvb_pool_q8& p, int bits, int dtype, const void* q,
                                const void* kn, const void* vn, void* out, const int32_t* cu,
                                const int32_t* plen, const int32_t* bt, int bt_stride, int batch,
                                int hq, int total_q, int max_q_len, float scale, void* plan_ws,
                                hipStream_t s);

// Cascade decode: the shared prefix pass (prefill kernel over all sequences' queries,
// key tiles split over `nks` work-groups of `ks_tiles` tiles, partials to slots 0..nks-1)
// and the private pass (decode split kernel from block `shared_len/16`, partials to
// slots nks..), then the merge over every slot.
void cascade_plan(int batch, int hkv, int hq, int shared_len, int* nks, int* ks_tiles);
hipError_t launch_cascade_shared(const kvb_pool& p, const void* q, const int32_t* ctx, int max_ctx,
                                 const int32_t* shared_blocks, int shared_len, int batch, int hq,
                                 float scale, int nks, int ks_tiles, float* ws_o, float* ws_ml,
                                 int ws_slots, hipStream_t s);
hipError_t launch_decode_cascade(const kvb_pool& p, const void* q, void* out, const int32_t* ctx,
                                 const int32_t* bt, int bt_stride, const int32_t* shared_blocks,
                                 int shared_len, int batch, int hq, int max_ctx, int sb, int ns,
                                 int nks, int ks_tiles, float scale, void* ws, hipStream_t s);
// Grouped cascade decode: the shared prefix in group work-groups of the split kernel's
// launch (16 / min(G, 16) sequences per work-group, `sh_nsplit` key splits of
// `sh_split_blocks` blocks, partials to slots 0..sh_nsplit-1), the private splits in the
// same launch, then the merge.  cascade_use_grouped picks it over the separate pass.
void decode_group_plan(int shared_len, int sb, int* sh_split_blocks, int* sh_nsplit);
bool cascade_use_grouped(int batch, int hkv, int hq, int shared_len);
hipError_t launch_decode_grouped(const kvb_pool& p, const void* q, void* out, const int32_t* ctx,
                                 const int32_t* bt, int bt_stride, const int32_t* shared_blocks,
                                 int shared_len, int batch, int hq, int max_ctx, int sb, int ns,
                                 int sh_sb, int sh_ns, float scale, void* ws, hipStream_t s);
inline int64_t cascade_ws_bytes(int batch, int hq, int d, int slots) {
  return ((int64_t)batch * hq * slots * d + (int64_t)batch * hq * slots * 2) * 4;
}

hipError_t launch_prefill_pooled(const kvb_pool& p, const void* q, void* out, const int32_t* cu,
                                 const int32_t* plen, const int32_t* bt, int bt_stride, int batch,
                                 int hq, int total_q, int max_q_len, float scale, hipStream_t s);
// Prefill: `plan_ws` (may be NULL) holds prefill_plan_bytes(...) bytes for the
// longest-first dispatch plan of a grid of several rounds; `slots` (may be NULL): also
// scatter the chunk's K/V into the pool at these slots in the same launch.
int64_t prefill_plan_bytes(int batch, int hq, int total_q);
hipError_t launch_prefill(const kvb_pool& p, const void* q, const void* kn, const void* vn, void* out,
                          const int32_t* cu, const int32_t* plen, const int32_t* bt, int bt_stride,
                          int batch, int hq, int total_q, int max_q_len, int max_prefix_len,
                          float scale, void* plan_ws, hipStream_t s, const int64_t* slots = nullptr);

}  // namespace kvb
