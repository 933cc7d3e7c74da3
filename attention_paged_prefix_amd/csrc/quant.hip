// Quantising slot scatter into the 8-bit and 4-bit K/V pools.
//
// The pages keep cached K at per-channel scales and V at per-token scales, at 8 bits or
// 4 (kvboost 0.6.0, "Optional: KV quantization").  K uses the pool's scale of each
// (KV head, channel); V gets one scale per (token, KV head), max |v| / M, computed here,
// with M = 127 (8 bits) or 7 (4 bits).  A code is rint(x / s) in float32 (IEEE division,
// half to even) clamped to [-M, M], and 0 at a zero scale.  4-bit codes are stored two
// per byte, the even channel in the low nibble.
#include "kvb_device.h"
#include "kvb_launch.h"

namespace kvb {

template <int M>
__device__ inline uint32_t quant_code(float x, float s) {
  if (s == 0.f) return 0;
  const float r = fminf(fmaxf(rintf(__fdiv_rn(x, s)), -(float)M), (float)M);
  return (uint32_t)(int)r & (M > 7 ? 0xffu : 0xfu);
}

// One wave per (token, KV head); lane l codes channels 2l and 2l+1 (l < D/2): two bytes
// at 8 bits, one byte (two nibbles) at 4.
template <typename T, int D, int BITS>
__global__ void __launch_bounds__(256)
write_kv_q8_kernel(uint8_t* __restrict__ kp, uint8_t* __restrict__ vp, float* __restrict__ v_scale,
                   const float* __restrict__ k_scale, int64_t block_stride, int64_t pool_slots,
                   const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn,
                   const int64_t* __restrict__ slots, int num_tokens, int hkv) {
  const int lane = threadIdx.x & 63;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= (int64_t)num_tokens * hkv) return;
  const int t = (int)(wid / hkv);
  const int h = (int)(wid - (int64_t)t * hkv);
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= pool_slots) return;
  const int64_t blk = slot >> 4;
  const int row = (int)(slot & 15);
  const bool act = 2 * lane < D;
  const int64_t src = ((int64_t)t * hkv + h) * D + 2 * lane;
  uint32_t kw = 0, vw = 0;
  if (act) {
    kw = *reinterpret_cast<const uint32_t*>(kn + src);
    vw = *reinterpret_cast<const uint32_t*>(vn + src);
  }
  const float v0 = lo_f32<T>(vw), v1 = hi_f32<T>(vw);
  float a = fmaxf(fabsf(v0), fabsf(v1));              // 0 on lanes past the row
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) a = fmaxf(a, __shfl_xor(a, m, 64));
  constexpr int M = BITS == 8 ? 127 : 7;
  const float s = __fdiv_rn(a, (float)M);
  if (act) {
    const float2 ks = *reinterpret_cast<const float2*>(k_scale + h * D + 2 * lane);
    const int64_t dst = blk * block_stride + ((int64_t)(h * kBlock + row) * D + 2 * lane) * BITS / 8;
    const uint32_t kc = quant_code<M>(lo_f32<T>(kw), ks.x) | (quant_code<M>(hi_f32<T>(kw), ks.y) << BITS);
    const uint32_t vc = quant_code<M>(v0, s) | (quant_code<M>(v1, s) << BITS);
    if constexpr (BITS == 8) {
      *reinterpret_cast<uint16_t*>(kp + dst) = (uint16_t)kc;
      *reinterpret_cast<uint16_t*>(vp + dst) = (uint16_t)vc;
    } else {
      kp[dst] = (uint8_t)kc;
      vp[dst] = (uint8_t)vc;
    }
  }
  if (lane == 0) v_scale[(blk * hkv + h) * kBlock + row] = s;
}

hipError_t launch_write_kv_q8(const kvb_pool_q8& p, int bits, int dtype, const void* kn,
                              const void* vn, const int64_t* slots, int num_tokens, hipStream_t s) {
  const int64_t waves = (int64_t)num_tokens * p.num_kv_heads;
  if (waves == 0) return hipSuccess;
  const unsigned grid = (unsigned)((waves + 3) / 4);
#define KVB_WQ8(TT, DD)                                                                           \
  if (bits == 4) KVB_WQ(TT, DD, 4); else KVB_WQ(TT, DD, 8)
#define KVB_WQ(TT, DD, BB)                                                                        \
  hipLaunchKernelGGL((write_kv_q8_kernel<TT, DD, BB>), dim3(grid), dim3(256), 0, s, (uint8_t*)p.k, \
                     (uint8_t*)p.v, p.v_scale, p.k_scale, p.block_stride,                          \
                     (int64_t)p.num_blocks * kBlock, (const uint16_t*)kn, (const uint16_t*)vn,     \
                     slots, num_tokens, p.num_kv_heads)
  const bool bf = dtype == KVB_BF16;
  switch (p.head_dim) {
    case 64:  if (bf) KVB_WQ8(BF16, 64); else KVB_WQ8(F16, 64); break;
    case 96:  if (bf) KVB_WQ8(BF16, 96); else KVB_WQ8(F16, 96); break;
    default:  if (bf) KVB_WQ8(BF16, 128); else KVB_WQ8(F16, 128); break;
  }
#undef KVB_WQ
#undef KVB_WQ8
  return hipGetLastError();
}

}  // namespace kvb
