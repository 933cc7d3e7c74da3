// Slot scatter (write new K/V into pool slots) and the block-table gather used by
// the indexing tests.  Both are pure 16-byte copies: HBM-bound, bit-exact.
//
// Slot scatter follows kvstream 0.1.0, "Why KVStream?" (streaming KV allocation, one
// slot per token); the gather follows its "Request lifecycle" step 3 (a block table
// maps a sequence onto possibly shared pool pages).
#include "kvb_device.h"
#include "kvb_launch.h"

namespace kvb {

// One thread per 16-byte chunk of one (token, kv head) row, for K and for V.
// Chunks per row = head_dim/8; consecutive threads cover consecutive chunks of a
// row, so both the read of k_new and the write into the pool are coalesced.
__global__ void __launch_bounds__(256)
write_kv_kernel(uint16_t* __restrict__ kp, uint16_t* __restrict__ vp, int64_t block_stride,
                int64_t pool_slots, const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn,
                const int64_t* __restrict__ slots, int num_tokens, int hkv, int head_dim) {
  const int cpr = head_dim >> 3;                       // chunks per (token, head) row
  const int64_t per_tok = (int64_t)hkv * cpr;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= per_tok * num_tokens) return;
  const int t = (int)(idx / per_tok);
  const int rem = (int)(idx - (int64_t)t * per_tok);
  const int h = rem / cpr, c = rem - h * cpr;
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= pool_slots) return;
  const int64_t blk = slot >> 4;
  const int row = (int)(slot & 15);
  const int64_t dst = blk * block_stride + ((int64_t)(h * kBlock + row)) * head_dim + c * 8;
  const int64_t src = ((int64_t)t * hkv + h) * head_dim + c * 8;
  const uint4 kv = *reinterpret_cast<const uint4*>(kn + src);
  const uint4 vv = *reinterpret_cast<const uint4*>(vn + src);
  *reinterpret_cast<uint4*>(kp + dst) = kv;
  *reinterpret_cast<uint4*>(vp + dst) = vv;
}

// grid: (ceil(max_len * hkv * cpr / 256), batch)
__global__ void __launch_bounds__(256)
gather_kv_kernel(const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
                 int64_t block_stride, int num_blocks, const int32_t* __restrict__ bt,
                 int bt_stride, const int32_t* __restrict__ seq_lens,
                 const int32_t* __restrict__ cu, uint16_t* __restrict__ ko,
                 uint16_t* __restrict__ vo, int hkv, int head_dim) {
  const int b = blockIdx.y;
  const int cpr = head_dim >> 3;
  const int per_tok = hkv * cpr;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int n = seq_lens[b];
  if (idx >= (int64_t)per_tok * n) return;
  const int j = (int)(idx / per_tok);
  const int rem = (int)(idx - (int64_t)j * per_tok);
  const int h = rem / cpr, c = rem - h * cpr;
  const int blk = bt[(int64_t)b * bt_stride + (j >> 4)];
  if (blk < 0 || blk >= num_blocks) return;
  const int64_t src = (int64_t)blk * block_stride + ((int64_t)(h * kBlock + (j & 15))) * head_dim + c * 8;
  const int64_t dst = ((int64_t)(cu[b] + j) * hkv + h) * head_dim + c * 8;
  *reinterpret_cast<uint4*>(ko + dst) = *reinterpret_cast<const uint4*>(kp + src);
  *reinterpret_cast<uint4*>(vo + dst) = *reinterpret_cast<const uint4*>(vp + src);
}

// Whole-block copies between two pools of the same shape (kvboost 0.6.0, "CPU paged
// attention": shared prefixes share physical blocks copy-on-write; kvstream 0.1.0, "Why
// KVStream?": sequences spilled to a CPU page pool).  One work-group per (pair, K or V
// part); the part of a block, num_kv_heads x 16 x head_dim, is contiguous.  Pairs whose
// source or destination id is outside its pool are skipped.
__global__ void __launch_bounds__(256)
copy_blocks_kernel(const uint16_t* __restrict__ sk, const uint16_t* __restrict__ sv, int64_t s_stride,
                   int s_nb, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int64_t d_stride,
                   int d_nb, const int32_t* __restrict__ src_ids, const int32_t* __restrict__ dst_ids,
                   int64_t chunks) {
  const int i = blockIdx.x;
  const int sb = src_ids[i], db = dst_ids[i];
  if (sb < 0 || sb >= s_nb || db < 0 || db >= d_nb) return;
  const uint4* src = reinterpret_cast<const uint4*>((blockIdx.y ? sv : sk) + (int64_t)sb * s_stride);
  uint4* dst = reinterpret_cast<uint4*>((blockIdx.y ? dv : dk) + (int64_t)db * d_stride);
  for (int64_t c = threadIdx.x; c < chunks; c += 256) dst[c] = src[c];
}

hipError_t launch_copy_blocks(const kvb_pool& src, const kvb_pool& dst, const int32_t* src_ids,
                              const int32_t* dst_ids, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t chunks = (int64_t)src.num_kv_heads * kBlock * src.head_dim / 8;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)n, 2), dim3(256), 0, s,
                     (const uint16_t*)src.k, (const uint16_t*)src.v, src.block_stride, src.num_blocks,
                     (uint16_t*)dst.k, (uint16_t*)dst.v, dst.block_stride, dst.num_blocks, src_ids,
                     dst_ids, chunks);
  return hipGetLastError();
}

hipError_t launch_write_kv(const kvb_pool& p, const void* kn, const void* vn, const int64_t* slots,
                           int num_tokens, hipStream_t s) {
  const int64_t total = (int64_t)num_tokens * p.num_kv_heads * (p.head_dim / 8);
  const int64_t grid = (total + 255) / 256;
  hipLaunchKernelGGL(write_kv_kernel, dim3((unsigned)grid), dim3(256), 0, s,
                     (uint16_t*)p.k, (uint16_t*)p.v, p.block_stride, (int64_t)p.num_blocks * kBlock,
                     (const uint16_t*)kn, (const uint16_t*)vn, slots, num_tokens, p.num_kv_heads,
                     p.head_dim);
  return hipGetLastError();
}

hipError_t launch_gather_kv(const kvb_pool& p, const int32_t* bt, int bt_stride,
                            const int32_t* seq_lens, const int32_t* cu, void* ko, void* vo,
                            int batch, int max_len, hipStream_t s) {
  const int64_t per_seq = (int64_t)max_len * p.num_kv_heads * (p.head_dim / 8);
  const int64_t gx = (per_seq + 255) / 256;
  hipLaunchKernelGGL(gather_kv_kernel, dim3((unsigned)gx, (unsigned)batch), dim3(256), 0, s,
                     (const uint16_t*)p.k, (const uint16_t*)p.v, p.block_stride, p.num_blocks, bt,
                     bt_stride, seq_lens, cu, (uint16_t*)ko, (uint16_t*)vo, p.num_kv_heads,
                     p.head_dim);
  return hipGetLastError();
}

}  // namespace kvb
