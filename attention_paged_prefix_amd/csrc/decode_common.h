// Device-side pieces shared by the split decode (decode.hip) and the balanced stream
// decode (decode_stream.hip): tile constants, the register staging of one step (two
// 16-token blocks) of K/V, and the widening of 8- and 4-bit codes.
#pragma once
#include <type_traits>

#include "kvb_device.h"

namespace kvb {

// 16 bytes per lane with the non-temporal (streaming) cache policy (operand 2 = nt).
__device__ inline uint4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 2));
}

constexpr int kDecWaves = 4;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kMaxSplitBlocks = 256;
constexpr int kDecHeads = 16;               // query heads per work-group (MFMA N)
constexpr float kRescaleThreshold = 8.0f;   // log2 units
constexpr float kNegBig = -1.0e30f;

template <int D> struct DecStep {
  static constexpr int VCH = D / 32;        // 16-byte chunks per lane per block, K and V
  uint4 k[2][VCH];
  uint4 v[2][VCH];
  int rows[2];                              // valid key rows of each block (0..16)
  int pos[2];                               // position of each block's first key
};

// A quantised pool's step (QB bits per code): a 16-byte chunk holds 128/QB codes of one
// key row, a block's K (or V) is CH = D*QB/8 chunks, NCH per lane; vsc holds the V scale
// of the key row each of the lane's V chunks belongs to.
template <int D, int QB> struct DecStepQ {
  static constexpr int CH = D * QB / 8;          // chunks per block (K or V)
  static constexpr int CPRQ = D * QB / 128;      // chunks per key row
  static constexpr int NCH = (CH + 63) / 64;
  uint4 k[2][NCH];
  uint4 v[2][NCH];
  float vsc[2][NCH];
  int rows[2];
  int pos[2];
};

// Scales of the 8-bit pool (ignored by the 16-bit forms): the per-channel K scales
// [Hkv][D] and the per-token V scales [block][Hkv][16].
struct DecQ8 {
  const float* k_scale;
  const float* v_scale;
};

// 16 int8 codes -> 16 values code * s of T in two 16-byte halves (s = 1: exact, since
// |code| <= 127 fits the 8-bit significand of bf16 and the 11-bit one of fp16; otherwise
// rounded to nearest even like any 16-bit value).
template <typename T>
__device__ inline void codes_to(uint4 c, float s, uint4& lo, uint4& hi) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int32_t x = (int32_t)w[i];
    o[2 * i] = pack2<T>((float)((x << 24) >> 24) * s, (float)((x << 16) >> 24) * s);
    o[2 * i + 1] = pack2<T>((float)((x << 8) >> 24) * s, (float)(x >> 24) * s);
  }
  lo = make_uint4(o[0], o[1], o[2], o[3]);
  hi = make_uint4(o[4], o[5], o[6], o[7]);
}

// 32 4-bit codes (two per byte, the even channel in the low nibble, 4-bit two's
// complement) -> 32 values code * s of T in four 16-byte quarters (s = 1: exact).
template <typename T>
__device__ inline void nibbles_to(uint4 c, float s, uint4 (&o4)[4]) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
  uint32_t o[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int32_t x = (int32_t)w[i];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      o[4 * i + k] = pack2<T>((float)((x << (28 - 8 * k)) >> 28) * s, (float)((x << (24 - 8 * k)) >> 28) * s);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) o4[q] = make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
}

// Merge kernels: one wave per (sequence, query head) row, four rows per work-group,
// partials taken eight at a time.
constexpr int kMergeRows = 4;
constexpr int kMergeBatch = 8;

}  // namespace kvb
