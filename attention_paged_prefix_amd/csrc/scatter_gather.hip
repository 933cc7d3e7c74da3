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
