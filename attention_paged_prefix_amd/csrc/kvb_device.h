// Device-side helpers shared by the gfx950 kernels: 16-bit element types,
// vector types for MFMA operands, cross-lane reductions and the XCD-aware
// work-group remap.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvb {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(2 * sizeof(_Float16)))) _Float16 f16x2;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kBlock = 16;        // tokens per physical block
constexpr int kNumXcd = 8;        // MI355X: 8 XCDs, work-groups dealt round-robin

// Element type tags.  Storage is always the raw 16-bit payload.
struct F16 {
  static constexpr int id = 0;
  __device__ static inline float to_f32(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
  }
  __device__ static inline uint16_t from_f32(float f) {   // round to nearest even
    return __builtin_bit_cast(uint16_t, (_Float16)f);
  }
  // 32x32x16 MFMA with 16-bit operands passed as 8 x 16-bit lanes.
  __device__ static inline f32x16 mfma32(s16x8 a, s16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static inline f32x4 mfma16(s16x8 a, s16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static constexpr uint32_t kOnePair = 0x3C003C00u;   // (1.0, 1.0)
  // a.x*b.x + a.y*b.y + c (fp32 accumulate)
  __device__ static inline float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b),
                                  c, false);
  }
};

struct BF16 {
  static constexpr int id = 1;
  __device__ static inline float to_f32(uint16_t b) {
    return __builtin_bit_cast(float, (uint32_t)b << 16);
  }
  __device__ static inline uint16_t from_f32(float f) {   // round to nearest even
    return __builtin_bit_cast(uint16_t, (__bf16)f);
  }
  __device__ static inline f32x16 mfma32(s16x8 a, s16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline f32x4 mfma16(s16x8 a, s16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static constexpr uint32_t kOnePair = 0x3F803F80u;   // (1.0, 1.0)
  __device__ static inline float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
  }
};

// Low / high 16-bit halves of a packed pair, as fp32.
template <typename T> __device__ inline float lo_f32(uint32_t w) { return T::to_f32((uint16_t)(w & 0xffffu)); }
template <typename T> __device__ inline float hi_f32(uint32_t w) { return T::to_f32((uint16_t)(w >> 16)); }
template <> __device__ inline float lo_f32<BF16>(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
template <> __device__ inline float hi_f32<BF16>(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Two fp32 values rounded (nearest even) into one packed 16-bit pair (v_cvt_pk_*_f32).
template <typename T> __device__ inline uint32_t pack2(float a, float b);
template <> __device__ inline uint32_t pack2<F16>(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){a, b}, f16x2v));
}
template <> __device__ inline uint32_t pack2<BF16>(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){a, b}, bf16x2v));
}

// gfx950 LDS transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane t
// receives element t%4 of the 4 x 16-bit values addressed by lanes t/4, t/4+4, t/4+8 and
// t/4+12 of its group, in that order.  With source lane s pointing at row (r0 + s/4),
// columns (c0 + 4*(s%4)) .. +3 of a row-major 16-bit matrix, lane t receives column
// c0 + t of rows r0 .. r0+3.
// The restrict-qualified pointer gives the read alias-scope information once inlined.
// Without it the compiler waits for every outstanding LDS-direct buffer load before the
// read, including loads into a different LDS buffer; callers that read memory filled by
// LDS-direct loads must therefore wait for those loads themselves (s_waitcnt + barrier).
__device__ __attribute__((always_inline)) inline s16x4 lds_read_tr16(const uint16_t* __restrict__ p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

// DPP quad permutations (within groups of 4 lanes): lane ^ 1 and lane ^ 2.
__device__ inline float quad_xor1(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
}
__device__ inline float quad_xor2(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
}

__device__ inline float xor_lane(float x, int mask) { return __shfl_xor(x, mask, 64); }
// x of lane l ^ 16: ds_swizzle in bit-mask mode (and 0x1f, or 0, xor 0x10 within each
// 32-lane group), which needs no lane-address register, unlike a permute.
__device__ inline float xor16(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401f));
}

// Both halves of a wave exchanged (lane l <-> lane l^32) with gfx950's v_permlane32_swap,
// which swaps lanes 32..63 of its first operand with lanes 0..31 of its second.  With x in
// both operands, the pair then holds (x[l], x[l^32]) in some order in every lane, so
// max/sum of the pair is the reduction over the two halves.  Written as (non-volatile)
// inline assembly: the compiler folds the intrinsic's two results into one when both
// inputs are the same value.  The s_nop covers the VALU-write -> permlane-read hazard.
__device__ inline void half_swap(float x, float& a, float& b) {
  a = x;
  b = x;
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ inline float halves_max(float x) {
  float a, b;
  half_swap(x, a, b);
  return fmaxf(a, b);
}
__device__ inline float halves_sum(float x) {
  float a, b;
  half_swap(x, a, b);
  return a + b;
}

// Instruction classes for __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedValu = 0x002;
constexpr int kSchedMfma = 0x008;
constexpr int kSchedVmem = 0x010;
constexpr int kSchedDsRead = 0x100;

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Raw buffer resources (gfx9 family dword3).  Loads at byte offsets >= num_records
// return zero without touching memory, which gives branch-free zero fill for masked
// rows and keeps every load unconditional (so the compiler can count outstanding
// loads exactly instead of waiting for all of them).
constexpr int kBufDword3 = 0x00020000;
// The fields are forced into scalar registers (readfirstlane): callers pass wave-uniform
// values, and a resource the compiler cannot prove uniform becomes a waterfall loop.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t num_bytes) {
  const uint64_t a = (uint64_t)base;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  const int n = __builtin_amdgcn_readfirstlane((int)num_bytes);
  void* p = (void*)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, n, kBufDword3);
}
__device__ inline uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0));
}
constexpr uint32_t kOobOffset = 0x7ffffff0u;   // beyond any num_records used here
// One dword into a vector register (the same value in every lane for a uniform offset).
__device__ inline uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)byte_off, 0, 0);
}

__device__ inline int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Placed inside a rarely taken branch so the compiler keeps the branch instead of
// speculating the block into selects that would then run on every iteration.
__device__ inline void keep_branch() { asm volatile("" ::: "memory"); }

// 16 bytes per lane from a buffer straight into LDS: lane L's bytes land at
// lds + 16*L (the LDS base must be wave-uniform).  Out-of-range lanes write zeros.
typedef __attribute__((address_space(3))) void lds_void_t;
__device__ inline void buf_load16_lds(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(lds), 16, (int)byte_off, 0, 0, 0);
}

// XCD-aware remap: hardware deals consecutive work-group ids round-robin over the
// XCDs; give each XCD a contiguous range of logical ids so neighbouring logical
// work (same sequence / KV head) shares that XCD's L2.  `padded` is a multiple of 8.
__device__ inline int xcd_logical_id(int hw_id, int padded) {
  int per = padded / kNumXcd;
  return (hw_id % kNumXcd) * per + hw_id / kNumXcd;
}

}  // namespace kvb
