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
//  * K/V tiles of 64 keys = four 16-token blocks.  Each block (or each 16-row group of
//    the chunk's own K/V) is read through a buffer resource sized to its valid rows:
//    one 16-byte load per thread, rows past the end read as zero with no memory
//    traffic, and every load is unconditional so it overlaps the previous tile's math.
//  * LDS is double buffered: tile t+1 is loaded into registers while tile t is used,
//    then stored to the other buffer; one barrier per tile.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16 (A = K rows
//    from LDS, B = Q held in registers for the whole kernel).  Each lane then owns one
//    query row, so the row max needs one cross-lane step and the row sum none.
//  * The output is accumulated transposed, O^T += V^T P^T: the score accumulators are
//    already the B operand, and V stays in its natural row-major layout in LDS and is
//    read transposed with ds_read_b64_tr_b16.
//  * Online softmax in the exp2 domain with scale*log2(e) folded into one FMA; the
//    running max only moves (and the output is only rescaled) when a score exceeds it
//    by more than 2^8.  Only tiles crossing the causal diagonal or the end of the keys
//    are masked; tiles entirely in the future of every row are never visited.
#include "kvb_device.h"
#include "kvb_launch.h"

namespace kvb {

constexpr int kPfWaves = 4;
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kBM = 32 * kPfWaves;      // virtual rows per work-group
constexpr int kKT = 64;                 // keys per tile
constexpr float kPfNegBig = -1.0e30f;
constexpr float kPfRescale = 8.0f;      // log2 units

template <int D> struct PfLayout {
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int KS = D + 8;                  // K row stride: rows 4 banks apart
  static constexpr int VS = D == 128 ? 160 : 96;    // V row stride: rows 16 banks apart
  static constexpr int KBUF = kKT * KS;
  static constexpr int VBUF = kKT * VS;
  static constexpr int BUF = KBUF + VBUF;           // elements per LDS buffer
};

template <typename T, int D>
__global__ void __launch_bounds__(kPfThreads, 2)
prefill_kernel(const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
               int64_t block_stride, int num_blocks, const uint16_t* __restrict__ q,
               const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn,
               uint16_t* __restrict__ out, const int32_t* __restrict__ cu,
               const int32_t* __restrict__ plen, const int32_t* __restrict__ bt, int bt_stride,
               int batch, int hq, int hkv, int total_q, int max_tiles, float c_log2, int padded,
               int real) {
  using L = PfLayout<D>;
  constexpr int CPR = L::CPR, KS = L::KS, VS = L::VS;
  constexpr int NKK = D / 16;                // MFMA k-steps over head_dim
  constexpr int NDB = D / 32;                // 32-wide d blocks of the output

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * L::BUF];

  const int lid = xcd_logical_id(blockIdx.x, padded);
  if (lid >= real) return;
  // logical id -> (kvh, b, tile), tile fastest and KV head slowest
  int r = lid;
  const int tile = r % max_tiles; r /= max_tiles;
  const int b = r % batch;
  const int kvh = r / batch;
  const int G = hq / hkv;
  const int cu_b = min(max(cu[b], 0), total_q);
  const int C = max(0, min(cu[b + 1], total_q) - cu_b);
  const int nrows = C * G;
  const int v0 = tile * kBM;
  if (v0 >= nrows) return;
  const int P = max(0, min(plen[b], bt_stride * kBlock));

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = uniform(tid >> 6);
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

  // loader geometry: thread tid covers row tid/CPR, chunk tid%CPR of each 16-row group
  const bool ld_on = tid < kBlock * CPR;
  const int ld_row = ld_on ? tid / CPR : 0;
  const int ld_col = ld_on ? tid - ld_row * CPR : 0;
  const int32_t* bt_row = bt + (int64_t)b * bt_stride;
  const int64_t head_off = (int64_t)kvh * kBlock * D;
  const uint16_t* kbase = kp + head_off;                          // + block * block_stride
  const uint16_t* vbase = vp + head_off;
  const uint16_t* knb = kn + ((int64_t)cu_b * hkv + kvh) * D;     // + row * hkv * D
  const uint16_t* vnb = vn + ((int64_t)cu_b * hkv + kvh) * D;
  const uint32_t pool_off = ld_on ? (uint32_t)(ld_row * D + ld_col * 8) * 2 : kOobOffset;
  const uint32_t self_off = ld_on ? (uint32_t)(ld_row * hkv * D + ld_col * 8) * 2 : kOobOffset;
  const uint32_t self_row_bytes = (uint32_t)(hkv * D * 2);

  // block ids of prefix tile t (uniform scalar loads); -1 past the prefix or out of pool
  auto tile_blocks = [&](int t, int* ids) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = t * 4 + i;
      int pb = -1;
      if (j * kBlock < P) pb = bt_row[j];
      ids[i] = (pb >= 0 && pb < num_blocks) ? pb : -1;
    }
  };

  // Tile t (prefix tiles first, then the chunk's own tiles) into registers.  Branch
  // free: both sources are described by (base pointer, valid bytes, lane offset) and
  // selected with uniform conditions; past the last tile every size is zero.
  uint4 kreg[4], vreg[4];
  auto load_tile = [&](int t, const int* ids) {
    const bool pre = t < n_pre;
    const int u = t - n_pre;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pb = ids[i];
      const int rows_pre = max(0, min(kBlock, P - (t * kKT + kBlock * i)));
      const int row0 = u * kKT + kBlock * i;
      const int rows_self = max(0, min(kBlock, self_n - row0));
      const int64_t pre_off = (int64_t)(pb >= 0 ? pb : 0) * block_stride;
      const int64_t self_row = (int64_t)(pre ? 0 : min(row0, C)) * hkv * D;
      const uint16_t* kb = pre ? kbase + pre_off : knb + self_row;
      const uint16_t* vb = pre ? vbase + pre_off : vnb + self_row;
      const uint32_t nb = pre ? (pb >= 0 ? (uint32_t)(rows_pre * D * 2) : 0u)
                              : (rows_self > 0 ? (uint32_t)(rows_self - 1) * self_row_bytes + D * 2 : 0u);
      const uint32_t off = pre ? pool_off : self_off;
      kreg[i] = buf_load16(make_rsrc(kb, nb), off);
      vreg[i] = buf_load16(make_rsrc(vb, nb), off);
    }
  };

  auto store_tile = [&](int buf) {
    if (ld_on) {
      uint16_t* sk = smem + buf * L::BUF;
      uint16_t* sv = sk + L::KBUF;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = kBlock * i + ld_row;
        *reinterpret_cast<uint4*>(sk + row * KS + ld_col * 8) = kreg[i];
        *reinterpret_cast<uint4*>(sv + row * VS + ld_col * 8) = vreg[i];
      }
    }
  };

  // tr-read source address of this lane inside a V tile: rows 4*hf + (l%16)/4 (+8),
  // columns 16*((l/16)%2) + 4*(l%4) (+32 per d block, +16 rows per 16-key step)
  const int tr_base = (4 * hf + ((lane & 15) >> 2)) * VS + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int k_base = lr * KS + 8 * hf;

  auto compute = [&](int t, int buf) {
    const uint16_t* sk = smem + buf * L::BUF;
    const uint16_t* sv = sk + L::KBUF;
    const bool pre = t < n_pre;
    const int base = pre ? t * kKT : (t - n_pre) * kKT;
    const int count = pre ? min(kKT, P - base) : min(kKT, self_n - base);
    const bool need_mask = (count < kKT) || (!pre && base + kKT - 1 > i_first);

    // S^T = K Q^T for two 32-key halves; the two accumulation chains are interleaved
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const s16x8 a0 = *reinterpret_cast<const s16x8*>(sk + k_base + 16 * kk);
      const s16x8 a1 = *reinterpret_cast<const s16x8*>(sk + k_base + 32 * KS + 16 * kk);
      s0 = T::mfma32(a0, qreg[kk], s0);
      s1 = T::mfma32(a1, qreg[kk], s1);
    }
    if (need_mask) {
      // key kl of the tile is visible to this lane's row iff kl < lim
      const int lim = pre ? count : min(count, i_row - base + 1);
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const int kl = (rr >> 2) * 8 + hf * 4 + (rr & 3);
        s0[rr] = kl < lim ? s0[rr] : -INFINITY;
        s1[rr] = kl + 32 < lim ? s1[rr] : -INFINITY;
      }
    }
    float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
    for (int rr = 1; rr < 16; ++rr) mx = fmaxf(mx, fmaxf(s0[rr], s1[rr]));
    mx = fmaxf(mx, xor_lane(mx, 32)) * c_log2;
    if (__any(mx > m_run + kPfRescale)) {
      const float mn = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - mn);
      m_run = mn;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) o[db][rr] *= alpha;
    }
    // probabilities, packed as the B operand of the PV product; the row sum adds the
    // rounded values (the ones PV uses) two at a time with a dot product against (1, 1)
    s16x8 pk[4];
    float ls = l_run;
#pragma unroll
    for (int kp4 = 0; kp4 < 4; ++kp4) {
      const f32x16& sv4 = (kp4 >> 1) ? s1 : s0;
      const int r0 = (kp4 & 1) * 8;
      uint32_t pw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = fast_exp2(fmaf(sv4[r0 + 2 * e], c_log2, -m_run));
        const float p1 = fast_exp2(fmaf(sv4[r0 + 2 * e + 1], c_log2, -m_run));
        pw[e] = pack2<T>(p0, p1);
        ls = T::dot2(pw[e], T::kOnePair, ls);
      }
      pk[kp4] = __builtin_bit_cast(s16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
    }
    l_run = ls;
    // O^T += V^T P^T; all eight transposed reads of a d block are issued before its MFMAs
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      s16x8 a[4];
#pragma unroll
      for (int kp4 = 0; kp4 < 4; ++kp4) {
        const uint16_t* src = sv + tr_base + 16 * kp4 * VS + 32 * db;
        const s16x4 lo = lds_read_tr16(src);
        const s16x4 hi = lds_read_tr16(src + 8 * VS);
        a[kp4] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int kp4 = 0; kp4 < 4; ++kp4) o[db] = T::mfma32(a[kp4], pk[kp4], o[db]);
    }
  };

  int ids[4];
  tile_blocks(0, ids);
  load_tile(0, ids);
  store_tile(0);
  tile_blocks(1, ids);
  __syncthreads();
  for (int t = 0; t < total; ++t) {
    load_tile(t + 1, ids);                  // in flight during this tile's math
    tile_blocks(t + 2, ids);
    if (wave_active) compute(t, t & 1);
    store_tile((t + 1) & 1);
    __syncthreads();
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
  // scale 0 (all scores equal) is kept positive so masked -inf scores stay -inf
  const float c = fmaxf(scale * 1.4426950408889634f, 1e-30f);
  hipLaunchKernelGGL((prefill_kernel<T, D>), dim3((unsigned)padded), dim3(kPfThreads), 0, s,
                     (const uint16_t*)p.k, (const uint16_t*)p.v, p.block_stride, p.num_blocks,
                     (const uint16_t*)q, (const uint16_t*)kn, (const uint16_t*)vn, (uint16_t*)out,
                     cu, plen, bt, bt_stride, batch, hq, p.num_kv_heads, total_q, max_tiles, c,
                     (int)padded, (int)real);
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
