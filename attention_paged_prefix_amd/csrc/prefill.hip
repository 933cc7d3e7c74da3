// Paged prefill: the rows of a new chunk attend to the sequence's cached prefix, read
// from the block pool through its block table, and causally to the chunk's own K/V.
//
// What is computed follows kvboost 0.6.0, "How it works" steps 3 and 5 (cached prefix
// plus live suffix in one forward pass) and "Flash Attention (CUDA)" (tiled attention
// with online softmax; fp16/bf16; head dims 64/96/128; causal masking that skips
// future K/V tiles).  That page's CUDA kernel is prior art; this kernel is laid out for
// CDNA4 (gfx950):
//
//  * Work-group = 4 waves = 128 "virtual rows" of one (sequence, KV head).  Virtual
//    row v = i*G + g packs chunk row i and query head kvh*G + g, so the G query heads
//    that share a KV head share every K/V tile staged in LDS (GQA packing; works for
//    any G, including 5).
//  * K/V tiles of 64 keys = four 16-token blocks.  A prefix tile gathers its four
//    (block, kv-head) runs of 16 x head_dim through the block table; a self tile reads
//    k_new/v_new.  The next tile is loaded into registers while the current one is
//    used (register double buffering), then written to LDS.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16 (A = K from
//    LDS, B = Q held in registers for the whole kernel).  Each lane then owns one query
//    row, so the row max needs a single cross-lane step and the row sum none.
//  * The output is accumulated transposed, O^T += V^T P^T: the score accumulators are
//    already laid out as the B operand, and V is stored in LDS transposed with keys
//    permuted inside every 16-key group to match that layout (one 16-byte LDS read per
//    A operand).
//  * Online softmax in the exp2 domain with scale*log2(e) folded in.  Only tiles that
//    cross the causal diagonal or the end of the keys are masked; tiles entirely in the
//    future of every row of the work-group are never visited.
#include "kvb_device.h"
#include "kvb_launch.h"

namespace kvb {

constexpr int kPfWaves = 4;
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kBM = 32 * kPfWaves;      // virtual rows per work-group
constexpr int kKT = 64;                 // keys per tile
constexpr int kVPad = 8;                // elements of padding per V^T row
constexpr float kPfNegBig = -1.0e30f;

// Position of key k (0..15) inside its 16-key group in the transposed V tile: lane half
// h of the PV MFMA reads keys {4h..4h+3, 8+4h..8+4h+3} as 8 consecutive elements.
__device__ inline int vt_group_pos(int q4) { return ((q4 & 1) << 3) | ((q4 >> 1) << 2); }

template <typename T, int D>
__global__ void __launch_bounds__(kPfThreads, 2)
prefill_kernel(const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
               int64_t block_stride, int num_blocks, const uint16_t* __restrict__ q,
               const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn,
               uint16_t* __restrict__ out, const int32_t* __restrict__ cu,
               const int32_t* __restrict__ plen, const int32_t* __restrict__ bt, int bt_stride,
               int hq, int hkv, int total_q, int max_tiles, float c_log2, int padded, int real) {
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int NK = kKT * CPR / kPfThreads; // K chunks per thread per tile
  constexpr int KS = D + 8;                  // K row stride in LDS (elements)
  constexpr int VS = kKT + kVPad;            // V^T row stride in LDS (elements)
  constexpr int NKK = D / 16;                // MFMA k-steps over head_dim
  constexpr int NDB = D / 32;                // 32-wide d blocks of the output

  __shared__ __attribute__((aligned(16))) uint16_t sK[kKT * KS];
  __shared__ __attribute__((aligned(16))) uint16_t sV[D * VS];

  const int lid = xcd_logical_id(blockIdx.x, padded);
  if (lid >= real) return;
  int r = lid;
  const int tile = r % max_tiles; r /= max_tiles;
  const int kvh = r % hkv;
  const int b = r / hkv;
  const int G = hq / hkv;
  const int cu_b = min(max(cu[b], 0), total_q);
  const int C = max(0, min(cu[b + 1], total_q) - cu_b);
  const int nrows = C * G;
  const int v0 = tile * kBM;
  if (v0 >= nrows) return;
  int P = plen[b];
  P = max(0, min(P, bt_stride * kBlock));

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int lr = lane & 31, hf = lane >> 5;

  // this lane's query row
  const int v = v0 + 32 * w + lr;
  const bool rvalid = v < nrows;
  const int i_row = rvalid ? v / G : C;
  const int g_row = rvalid ? v - (v / G) * G : 0;
  const bool wave_active = v0 + 32 * w < nrows;

  s16x8 qreg[NKK];
  {
    const uint16_t* qrow = q + ((int64_t)(cu_b + i_row) * hq + kvh * G + g_row) * D + 8 * hf;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      if (rvalid) qreg[kk] = *reinterpret_cast<const s16x8*>(qrow + 16 * kk);
      else qreg[kk] = s16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }

  const int last_row = min(nrows, v0 + kBM) - 1;
  const int self_n = last_row / G + 1;       // chunk keys needed by this work-group
  const int i_first = v0 / G;
  const int n_pre = (P + kKT - 1) / kKT;
  const int n_self = (self_n + kKT - 1) / kKT;
  const int total = n_pre + n_self;

  f32x16 o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) o[i] = f32x16{};
  float m_run = kPfNegBig, l_run = 0.f;

  uint4 kreg[NK];
  uint4 vreg[4];
  const int vkg = tid & 15, vcc = tid >> 4;  // V loader: key group (4 keys), d chunk
  const int64_t bt_row = (int64_t)b * bt_stride;
  const int64_t head_off = (int64_t)kvh * kBlock * D;

  auto load_tile = [&](int t) {
    const bool pre = t < n_pre;
    const int base = pre ? t * kKT : (t - n_pre) * kKT;
    const int count = pre ? min(kKT, P - base) : min(kKT, self_n - base);
    int blk4[4] = {-1, -1, -1, -1};
    if (pre) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i * kBlock < count) {
          const int pb = bt[bt_row + (base >> 4) + i];
          blk4[i] = (pb >= 0 && pb < num_blocks) ? pb : -1;
        }
      }
    }
#pragma unroll
    for (int jj = 0; jj < NK; ++jj) {
      const int c = tid + kPfThreads * jj;
      const int row = c / CPR, col = c - (c / CPR) * CPR;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (row < count) {
        if (pre) {
          const int pb = blk4[row >> 4];
          if (pb >= 0)
            val = *reinterpret_cast<const uint4*>(kp + (int64_t)pb * block_stride + head_off +
                                                  (row & 15) * D + col * 8);
        } else {
          val = *reinterpret_cast<const uint4*>(kn + ((int64_t)(cu_b + base + row) * hkv + kvh) * D + col * 8);
        }
      }
      kreg[jj] = val;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 4 * vkg + e;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (vcc < CPR && row < count) {
        if (pre) {
          const int pb = blk4[row >> 4];
          if (pb >= 0)
            val = *reinterpret_cast<const uint4*>(vp + (int64_t)pb * block_stride + head_off +
                                                  (row & 15) * D + vcc * 8);
        } else {
          val = *reinterpret_cast<const uint4*>(vn + ((int64_t)(cu_b + base + row) * hkv + kvh) * D + vcc * 8);
        }
      }
      vreg[e] = val;
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int jj = 0; jj < NK; ++jj) {
      const int c = tid + kPfThreads * jj;
      const int row = c / CPR, col = c - (c / CPR) * CPR;
      *reinterpret_cast<uint4*>(&sK[row * KS + col * 8]) = kreg[jj];
    }
    if (vcc < CPR) {
      // keys 4*vkg .. 4*vkg+3, d = 8*vcc .. 8*vcc+7  ->  V^T rows d, 4 consecutive positions
      const int pos = (vkg >> 2) * 16 + vt_group_pos(vkg & 3);
      const uint32_t w0[4] = {vreg[0].x, vreg[0].y, vreg[0].z, vreg[0].w};
      const uint32_t w1[4] = {vreg[1].x, vreg[1].y, vreg[1].z, vreg[1].w};
      const uint32_t w2[4] = {vreg[2].x, vreg[2].y, vreg[2].z, vreg[2].w};
      const uint32_t w3[4] = {vreg[3].x, vreg[3].y, vreg[3].z, vreg[3].w};
#pragma unroll
      for (int pi = 0; pi < 4; ++pi) {
        // element 2*pi (low halves) and 2*pi+1 (high halves)
        uint2 lo, hi;
        lo.x = __builtin_amdgcn_perm(w1[pi], w0[pi], 0x05040100u);
        lo.y = __builtin_amdgcn_perm(w3[pi], w2[pi], 0x05040100u);
        hi.x = __builtin_amdgcn_perm(w1[pi], w0[pi], 0x07060302u);
        hi.y = __builtin_amdgcn_perm(w3[pi], w2[pi], 0x07060302u);
        *reinterpret_cast<uint2*>(&sV[(vcc * 8 + 2 * pi) * VS + pos]) = lo;
        *reinterpret_cast<uint2*>(&sV[(vcc * 8 + 2 * pi + 1) * VS + pos]) = hi;
      }
    }
  };

  if (total > 0) load_tile(0);
  for (int t = 0; t < total; ++t) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (t + 1 < total) load_tile(t + 1);
    if (!wave_active) continue;

    const bool pre = t < n_pre;
    const int base = pre ? t * kKT : (t - n_pre) * kKT;
    const int count = pre ? min(kKT, P - base) : min(kKT, self_n - base);
    const bool need_mask = (count < kKT) || (!pre && base + kKT - 1 > i_first);

    // S^T = K Q^T for two 32-key halves
    f32x16 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      s[mb] = f32x16{};
      const uint16_t* krow = &sK[(32 * mb + lr) * KS + 8 * hf];
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const s16x8 a = *reinterpret_cast<const s16x8*>(krow + 16 * kk);
        s[mb] = T::mfma32(a, qreg[kk], s[mb]);
      }
    }

    // scale, mask, row max
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        float tv = s[mb][rr] * c_log2;
        if (need_mask) {
          const int kl = 32 * mb + (rr >> 2) * 8 + hf * 4 + (rr & 3);
          const bool ok = kl < count && (pre || base + kl <= i_row);
          tv = ok ? tv : -INFINITY;
        }
        s[mb][rr] = tv;
        mx = fmaxf(mx, tv);
      }
    mx = fmaxf(mx, xor_lane(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;

    // probabilities, packed as the B operand of the PV product
    s16x8 pk[4];
    float psum = 0.f;
#pragma unroll
    for (int kp4 = 0; kp4 < 4; ++kp4) {
      const int mb = kp4 >> 1, r0 = (kp4 & 1) * 8;
      uint32_t pw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = fast_exp2(s[mb][r0 + 2 * e] - m_new);
        const float p1 = fast_exp2(s[mb][r0 + 2 * e + 1] - m_new);
        psum += p0 + p1;
        pw[e] = pack2<T>(p0, p1);
      }
      uint4 u = make_uint4(pw[0], pw[1], pw[2], pw[3]);
      pk[kp4] = __builtin_bit_cast(s16x8, u);
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) o[db][rr] *= alpha;

    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const uint16_t* vrow = &sV[(32 * db + lr) * VS + 8 * hf];
#pragma unroll
      for (int kp4 = 0; kp4 < 4; ++kp4) {
        const s16x8 a = *reinterpret_cast<const s16x8*>(vrow + 16 * kp4);
        o[db] = T::mfma32(a, pk[kp4], o[db]);
      }
    }
  }

  // epilogue: normalise and store (lane owns one query row, d in runs of 4)
  const float l_tot = l_run + xor_lane(l_run, 32);
  if (!rvalid) return;
  const float inv = 1.0f / l_tot;
  uint16_t* orow = out + ((int64_t)(cu_b + i_row) * hq + kvh * G + g_row) * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = 32 * db + r4 * 8 + hf * 4;
      uint2 u;
      u.x = pack2<T>(o[db][4 * r4 + 0] * inv, o[db][4 * r4 + 1] * inv);
      u.y = pack2<T>(o[db][4 * r4 + 2] * inv, o[db][4 * r4 + 3] * inv);
      *reinterpret_cast<uint2*>(orow + d) = u;
    }
}

template <typename T, int D>
static hipError_t launch_prefill_t(const kvb_pool& p, const void* q, const void* kn, const void* vn,
                                   void* out, const int32_t* cu, const int32_t* plen,
                                   const int32_t* bt, int bt_stride, int batch, int hq,
                                   int total_q, int max_q_len, float scale, hipStream_t s) {
  const int G = hq / p.num_kv_heads;
  const long long rows = (long long)max_q_len * G;
  const int max_tiles = (int)((rows + kBM - 1) / kBM);
  const long long real = (long long)batch * p.num_kv_heads * max_tiles;
  if (real == 0) return hipSuccess;
  const long long padded = (real + kNumXcd - 1) / kNumXcd * kNumXcd;
  const float c = scale * 1.4426950408889634f;
  hipLaunchKernelGGL((prefill_kernel<T, D>), dim3((unsigned)padded), dim3(kPfThreads), 0, s,
                     (const uint16_t*)p.k, (const uint16_t*)p.v, p.block_stride, p.num_blocks,
                     (const uint16_t*)q, (const uint16_t*)kn, (const uint16_t*)vn, (uint16_t*)out,
                     cu, plen, bt, bt_stride, hq, p.num_kv_heads, total_q, max_tiles, c, (int)padded,
                     (int)real);
  return hipGetLastError();
}

hipError_t launch_prefill(const kvb_pool& p, const void* q, const void* kn, const void* vn, void* out,
                          const int32_t* cu, const int32_t* plen, const int32_t* bt, int bt_stride,
                          int batch, int hq, int total_q, int max_q_len, int max_prefix_len,
                          float scale, hipStream_t s) {
  (void)max_prefix_len;
  const bool bf = p.dtype == KVB_BF16;
  switch (p.head_dim) {
    case 64:  return bf ? launch_prefill_t<BF16, 64>(p, q, kn, vn, out, cu, plen, bt, bt_stride, batch, hq, total_q, max_q_len, scale, s)
                        : launch_prefill_t<F16, 64>(p, q, kn, vn, out, cu, plen, bt, bt_stride, batch, hq, total_q, max_q_len, scale, s);
    case 96:  return bf ? launch_prefill_t<BF16, 96>(p, q, kn, vn, out, cu, plen, bt, bt_stride, batch, hq, total_q, max_q_len, scale, s)
                        : launch_prefill_t<F16, 96>(p, q, kn, vn, out, cu, plen, bt, bt_stride, batch, hq, total_q, max_q_len, scale, s);
    default:  return bf ? launch_prefill_t<BF16, 128>(p, q, kn, vn, out, cu, plen, bt, bt_stride, batch, hq, total_q, max_q_len, scale, s)
                        : launch_prefill_t<F16, 128>(p, q, kn, vn, out, cu, plen, bt, bt_stride, batch, hq, total_q, max_q_len, scale, s);
  }
}

}  // namespace kvb
