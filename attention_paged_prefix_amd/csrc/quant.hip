// Quantising slot scatter into the 8-bit and 4-bit K/V pools, and the widening gather of
// prefill over them.
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

// Prefill over the 8-bit pool.  The prefill kernel stages 16-bit tiles straight from the
// pool into LDS, so the 8-bit prefix is first widened: each sequence's prefix blocks go,
// as 16-bit values (K code x channel scale, V code x token scale, rounded to nearest even),
// into a staging pool in the workspace — staged block b * nbp + j holds logical block j of
// sequence b — with a block table to match (-1 past the prefix or for an out-of-pool id).
// The 16-bit prefill then runs on that pool.  Grid (nbp, batch), 256 threads; each thread
// widens 16-byte chunks (128/BITS codes) of the block's K and V.
template <typename T, int D, int BITS>
__global__ void __launch_bounds__(256)
dequant_gather_kernel(const uint8_t* __restrict__ kp, const uint8_t* __restrict__ vp,
                      const float* __restrict__ v_scale, const float* __restrict__ k_scale,
                      int64_t block_stride, int num_blocks, const int32_t* __restrict__ bt,
                      int bt_stride, const int32_t* __restrict__ plen, int hkv, int nbp,
                      uint16_t* __restrict__ sk, uint16_t* __restrict__ sv,
                      int32_t* __restrict__ stab) {
  const int j = blockIdx.x, b = blockIdx.y;
  const int P = min(max(plen[b], 0), bt_stride * kBlock);
  const int64_t sidx = (int64_t)b * nbp + j;
  int pb = -1;
  if (j < (P + kBlock - 1) / kBlock) {
    pb = bt[(int64_t)b * bt_stride + j];
    if (pb < 0 || pb >= num_blocks) pb = -1;
  }
  if (threadIdx.x == 0) stab[sidx] = pb >= 0 ? (int32_t)sidx : -1;
  if (pb < 0) return;
  constexpr int CPC = 128 / BITS;                      // codes per 16-byte chunk
  const int chunks = hkv * kBlock * D / CPC;
  const uint8_t* kb = kp + (int64_t)pb * block_stride;
  const uint8_t* vb = vp + (int64_t)pb * block_stride;
  uint16_t* dk = sk + sidx * ((int64_t)hkv * kBlock * D);
  uint16_t* dv = sv + sidx * ((int64_t)hkv * kBlock * D);
  for (int c = threadIdx.x; c < chunks; c += 256) {
    const int e0 = c * CPC;                             // (h * 16 + row) * D + col
    const int h = e0 / (kBlock * D);
    const int row = (e0 - h * kBlock * D) / D;
    const int col = e0 - (h * kBlock + row) * D;
    const uint4 kc = *reinterpret_cast<const uint4*>(kb + (int64_t)c * 16);
    const uint4 vc = *reinterpret_cast<const uint4*>(vb + (int64_t)c * 16);
    const float vs = v_scale[((int64_t)pb * hkv + h) * kBlock + row];
    const float* ks = k_scale + h * D + col;
    const uint32_t kw[4] = {kc.x, kc.y, kc.z, kc.w}, vw[4] = {vc.x, vc.y, vc.z, vc.w};
    constexpr int PER = 32 / BITS;                      // codes per dword
    uint32_t ko[CPC / 2], vo[CPC / 2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int32_t xk = (int32_t)kw[i], xv = (int32_t)vw[i];
#pragma unroll
      for (int k = 0; k < PER; k += 2) {
        const int e = PER * i + k;                      // code index within the chunk
        const float k0 = (float)((xk << (32 - BITS * (k + 1))) >> (32 - BITS));
        const float k1 = (float)((xk << (32 - BITS * (k + 2))) >> (32 - BITS));
        const float v0 = (float)((xv << (32 - BITS * (k + 1))) >> (32 - BITS));
        const float v1 = (float)((xv << (32 - BITS * (k + 2))) >> (32 - BITS));
        ko[e / 2] = pack2<T>(k0 * ks[e], k1 * ks[e + 1]);
        vo[e / 2] = pack2<T>(v0 * vs, v1 * vs);
      }
    }
#pragma unroll
    for (int q = 0; q < CPC / 8; ++q) {
      *reinterpret_cast<uint4*>(dk + e0 + 8 * q) = make_uint4(ko[4 * q], ko[4 * q + 1], ko[4 * q + 2], ko[4 * q + 3]);
      *reinterpret_cast<uint4*>(dv + e0 + 8 * q) = make_uint4(vo[4 * q], vo[4 * q + 1], vo[4 * q + 2], vo[4 * q + 3]);
    }
  }
}

// Workspace of prefill over the 8-bit pool: staged K, staged V, staged block table, then
// the dispatch plan of the 16-bit prefill (each part 256-byte aligned).
static int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }
static int64_t staged_blocks(int batch, int max_prefix_len) {
  return (int64_t)batch * std::max(1, (max_prefix_len + kBlock - 1) / kBlock);
}

int64_t prefill_q8_ws_bytes(int batch, int hkv, int hq, int d, int total_q, int max_prefix_len) {
  if (batch <= 0 || hkv <= 0 || hq <= 0 || total_q <= 0) return 0;
  const int64_t nb = staged_blocks(batch, max_prefix_len);
  const int64_t stage = align256(nb * hkv * kBlock * d * 2);
  return 2 * stage + align256(nb * 4) + prefill_plan_bytes(batch, hq, total_q);
}

hipError_t launch_prefill_q8(const kvb_pool_q8& p, int bits, int dtype, const void* q, const void* kn,
                             const void* vn, void* out, const int32_t* cu, const int32_t* plen,
                             const int32_t* bt, int bt_stride, int batch, int hq, int total_q,
                             int max_q_len, int max_prefix_len, float scale, void* ws,
                             hipStream_t s) {
  const int nbp = std::max(1, (max_prefix_len + kBlock - 1) / kBlock);
  const int64_t nb = staged_blocks(batch, max_prefix_len);
  const int64_t stage = align256(nb * p.num_kv_heads * kBlock * p.head_dim * 2);
  uint8_t* base = (uint8_t*)ws;
  uint16_t* sk = (uint16_t*)base;
  uint16_t* sv = (uint16_t*)(base + stage);
  int32_t* stab = (int32_t*)(base + 2 * stage);
  void* plan = base + 2 * stage + align256(nb * 4);
  const dim3 grid((unsigned)nbp, (unsigned)batch);
#define KVB_DG(TT, DD)                                                                            \
  if (bits == 4) KVB_DGB(TT, DD, 4); else KVB_DGB(TT, DD, 8)
#define KVB_DGB(TT, DD, BB)                                                                       \
  hipLaunchKernelGGL((dequant_gather_kernel<TT, DD, BB>), grid, dim3(256), 0, s, (const uint8_t*)p.k, \
                     (const uint8_t*)p.v, p.v_scale, p.k_scale, p.block_stride, p.num_blocks, bt,   \
                     bt_stride, plen, p.num_kv_heads, nbp, sk, sv, stab)
  const bool bf = dtype == KVB_BF16;
  switch (p.head_dim) {
    case 64:  if (bf) KVB_DG(BF16, 64); else KVB_DG(F16, 64); break;
    case 96:  if (bf) KVB_DG(BF16, 96); else KVB_DG(F16, 96); break;
    default:  if (bf) KVB_DG(BF16, 128); else KVB_DG(F16, 128); break;
  }
#undef KVB_DGB
#undef KVB_DG
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const kvb_pool staged{sk, sv, (int64_t)p.num_kv_heads * kBlock * p.head_dim, (int32_t)nb, kBlock,
                        p.num_kv_heads, p.head_dim, dtype};
  return launch_prefill(staged, q, kn, vn, out, cu, plen, stab, nbp, batch, hq, total_q, max_q_len,
                        max_prefix_len, scale, plan, s);
}

}  // namespace kvb
