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

constexpr int kRowWaves = 4;             // waves along the rows (32 rows each)
constexpr int kRowBlocks = 1;            // 32-row MFMA blocks per wave
constexpr int kBM = 32 * kRowBlocks * kRowWaves;  // virtual rows per work-group
constexpr int kKT = 64;                  // keys per tile
constexpr float kPfNegBig = -1.0e30f;
constexpr float kPfRescale = 8.0f;       // log2 units

// LDS tile = K rows then V rows, 64 x D each, unpadded.  Tiles are written by
// LDS-direct buffer loads (16 bytes per lane, lanes contiguous), so rows cannot be
// padded; instead the 16-byte chunks of a row are permuted so that the two read
// patterns are bank-conflict free:
//   K: the MFMA A operand reads one chunk from 16 consecutive rows per 16 lanes;
//   V: the transpose read reads four 32-byte row pieces (4 rows x 4 chunks) per 32 lanes.
// The permutation of a row depends only on row bits that are the same for every row a
// given lane reads, so read addresses are precomputed per lane.
template <int D> struct PfLayout {
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int TILE = 2 * kKT * D;          // elements: K then V
  __device__ static int posK(int r, int c) {
    if constexpr (D == 128) return c ^ (r & 15);
    else if constexpr (D == 96) return (c + ((r >> 2) & 3)) % 12;
    else return c ^ ((r >> 1) & 7);
  }
  __device__ static int invK(int r, int p) {
    if constexpr (D == 128) return p ^ (r & 15);
    else if constexpr (D == 96) return (p + 12 - ((r >> 2) & 3)) % 12;
    else return p ^ ((r >> 1) & 7);
  }
  __device__ static int posV(int r, int c) {
    if constexpr (D == 128) return ((((c >> 2) + r) & 3) << 2) | (c & 3);
    else if constexpr (D == 96) return (c + ((r >> 2) & 3)) % 12;
    else return ((((c >> 2) + (r >> 1)) & 1) << 2) | (c & 3);
  }
  __device__ static int invV(int r, int p) {
    if constexpr (D == 128) return ((((p >> 2) - r) & 3) << 2) | (p & 3);
    else if constexpr (D == 96) return (p + 12 - ((r >> 2) & 3)) % 12;
    else return ((((p >> 2) - (r >> 1)) & 1) << 2) | (p & 3);
  }
};

// Work-group = 4 * KS waves.  Wave w handles the 32 virtual rows 32*(w & 3) .. +31 of
// the work-group's 128 and the key tiles t with t % KS == (w >> 2).  With KS = 2 (small
// grids: 8 waves, one work-group per CU) the two waves of a row group split the keys
// and merge their (output, max, sum) through LDS at the end; with KS = 1 (large grids)
// two independent 4-wave work-groups share a CU and drift out of phase, so one group's
// softmax overlaps the other's MFMAs.  A stage holds KS tiles; stages are double
// buffered in LDS.
template <typename T, int D, int KS>
__global__ void __launch_bounds__(256 * KS, 2 / KS)
prefill_kernel(const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
               int64_t block_stride, int num_blocks, const uint16_t* __restrict__ q,
               const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn,
               uint16_t* __restrict__ out, const int32_t* __restrict__ cu,
               const int32_t* __restrict__ plen, const int32_t* __restrict__ bt, int bt_stride,
               int batch, int hq, int hkv, int total_q, int max_tiles, float c_log2, int padded,
               int real) {
  using L = PfLayout<D>;
  constexpr int CPR = L::CPR;
  constexpr int NKK = D / 16;                // MFMA k-steps over head_dim
  constexpr int NDB = D / 32;                // 32-wide d blocks of the output
  constexpr int NLD = CPR / 4;               // 1 KiB load instructions per 16-row block
  constexpr int VOFF = kKT * D;              // V rows follow K rows in a tile

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * KS * L::TILE];  // [key part][stage]

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
  const int rw = w & (kRowWaves - 1), kh = w / kRowWaves;   // row group, key part

  // this lane's two query rows
  int i_row[kRowBlocks], g_row[kRowBlocks];
  bool rvalid[kRowBlocks];
  s16x8 qreg[kRowBlocks][NKK];
#pragma unroll
  for (int j = 0; j < kRowBlocks; ++j) {
    const int v = v0 + 32 * kRowBlocks * rw + 32 * j + lr;
    rvalid[j] = v < nrows;
    i_row[j] = rvalid[j] ? v / G : C;
    g_row[j] = rvalid[j] ? v - (v / G) * G : 0;
    const uint16_t* qrow = q + ((int64_t)(cu_b + i_row[j]) * hq + kvh * G + g_row[j]) * D + 8 * hf;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      if (rvalid[j]) qreg[j][kk] = *reinterpret_cast<const s16x8*>(qrow + 16 * kk);
      else qreg[j][kk] = s16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  const bool wave_active = v0 + 32 * kRowBlocks * rw < nrows;

  const int last_row = min(nrows, v0 + kBM) - 1;
  const int self_n = last_row / G + 1;       // chunk keys needed by this work-group
  const int i_first = v0 / G;
  const int n_pre = (P + kKT - 1) / kKT;
  const int n_self = (self_n + kKT - 1) / kKT;
  const int total = n_pre + n_self;
  const int nstage = (total + KS - 1) / KS;

  f32x16 o[kRowBlocks][NDB];
#pragma unroll
  for (int j = 0; j < kRowBlocks; ++j)
#pragma unroll
    for (int i = 0; i < NDB; ++i) o[j][i] = f32x16{};
  float m_run[kRowBlocks], l_run[kRowBlocks];
#pragma unroll
  for (int j = 0; j < kRowBlocks; ++j) { m_run[j] = kPfNegBig; l_run[j] = 0.f; }

  // ---- loader: waves 4k..4k+3 stage tile k of a stage; within a tile wave (w & 3)
  // loads block (w & 3).  Instruction m of a block fills LDS chunks
  // 64m..64m+63 of that block; lane L's chunk holds row (64m+L)/CPR, logical chunk
  // inv(row, (64m+L)%CPR).
  const int ld_tile = w / kRowWaves, ld_blk = w & (kRowWaves - 1);
  // byte offset of lane's chunk = row * (source row pitch) + column bytes; the pitch is
  // D*2 in the pool and hkv*D*2 in the chunk's own K/V, chosen per tile (uniform)
  uint32_t ld_row[NLD], ld_colK[NLD], ld_colV[NLD];
#pragma unroll
  for (int m = 0; m < NLD; ++m) {
    const int pos = 64 * m + lane;
    const int rb = pos / CPR, cp = pos - (pos / CPR) * CPR;
    ld_row[m] = (uint32_t)rb;
    ld_colK[m] = (uint32_t)L::invK(rb, cp) * 16;
    ld_colV[m] = (uint32_t)L::invV(rb, cp) * 16;
  }
  const int32_t* bt_row = bt + (int64_t)b * bt_stride;
  const int64_t head_off = (int64_t)kvh * kBlock * D;
  const uint16_t* kbase = kp + head_off;                          // + block * block_stride
  const uint16_t* vbase = vp + head_off;
  const uint16_t* knb = kn + ((int64_t)cu_b * hkv + kvh) * D;     // + row * hkv * D
  const uint16_t* vnb = vn + ((int64_t)cu_b * hkv + kvh) * D;
  const uint32_t self_row_bytes = (uint32_t)(hkv * D * 2);

  // block id of this wave's block of prefix tile t (uniform scalar load)
  auto tile_blocks = [&](int t, int* ids) {
    const int jb = t * 4 + ld_blk;
    int pb = -1;
    if (t < n_pre && jb * kBlock < P) pb = bt_row[jb];
    ids[0] = (pb >= 0 && pb < num_blocks) ? pb : -1;
  };

  // Tile t (prefix tiles first, then the chunk's own tiles) straight into LDS buffer
  // (ld_tile, stage).  Sources are (base, valid bytes, lane offset) selected with uniform
  // conditions; rows past the end read as zero; past the last tile every size is zero.
  auto load_tile = [&](int t, const int* ids, int stage) {
    const bool pre = t < n_pre;
    const int tu = t - n_pre;
    uint16_t* dst = smem + (ld_tile * 2 + stage) * L::TILE;
    {
      const int i = ld_blk;
      const int pb = ids[0];
      const int rows_pre = max(0, min(kBlock, P - (t * kKT + kBlock * i)));
      const int row0 = tu * kKT + kBlock * i;
      const int rows_self = t < total ? max(0, min(kBlock, self_n - row0)) : 0;
      const int64_t pre_off = (int64_t)(pb >= 0 ? pb : 0) * block_stride;
      const int64_t self_row = (int64_t)(pre ? 0 : min(max(row0, 0), C)) * hkv * D;
      const uint16_t* kb = pre ? kbase + pre_off : knb + self_row;
      const uint16_t* vb = pre ? vbase + pre_off : vnb + self_row;
      const uint32_t nb = pre ? (pb >= 0 ? (uint32_t)(rows_pre * D * 2) : 0u)
                              : (rows_self > 0 ? (uint32_t)(rows_self - 1) * self_row_bytes + D * 2 : 0u);
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, nb), rv = make_rsrc(vb, nb);
      const uint32_t pitch = uniform(pre ? D * 2 : (int)self_row_bytes);
#pragma unroll
      for (int m = 0; m < NLD; ++m) {
        uint16_t* dk = dst + (kBlock * i * CPR + 64 * m) * 8;
        const uint32_t rowoff = ld_row[m] * pitch;
        buf_load16_lds(rk, rowoff + ld_colK[m], dk);
        buf_load16_lds(rv, rowoff + ld_colV[m], dk + VOFF);
      }
    }
  };

  // ---- per-lane LDS read addresses (elements, relative to a tile)
  // K operand of row block mb: row 32*mb + lr, logical chunk 2*kk + hf (mb adds 32 rows)
  int kaddr[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) kaddr[kk] = (lr * CPR + L::posK(lr, 2 * kk + hf)) * 8;
  // V transpose-read source: rows 16*kp4 + 4*hf + (l%16)/4 (+8 for the high half),
  // columns 32*db + 16*((l/16)%2) + 4*(l%4), i.e. chunk 4*db + 2*((l/16)%2) + (l%4)/2
  int vaddr[NDB][2];
  {
    const int s4 = (lane & 15) >> 2;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int hi = 0; hi < 2; ++hi) {
        const int row = 4 * hf + s4 + 8 * hi;
        const int c = 4 * db + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
        vaddr[db][hi] = VOFF + (row * CPR + L::posV(row, c)) * 8 + 4 * (lane & 1);
      }
  }

  auto compute = [&](int t, const uint16_t* sk) {
    const bool pre = t < n_pre;
    const int base = pre ? t * kKT : (t - n_pre) * kKT;
    const int count = pre ? min(kKT, P - base) : min(kKT, self_n - base);
    const bool need_mask = (count < kKT) || (!pre && base + kKT - 1 > i_first);

    // S^T = K Q^T: each K operand read feeds both row blocks
    f32x16 s[kRowBlocks][2];
#pragma unroll
    for (int j = 0; j < kRowBlocks; ++j) { s[j][0] = f32x16{}; s[j][1] = f32x16{}; }
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const s16x8 a0 = *reinterpret_cast<const s16x8*>(sk + kaddr[kk]);
      const s16x8 a1 = *reinterpret_cast<const s16x8*>(sk + kaddr[kk] + 32 * D);
#pragma unroll
      for (int j = 0; j < kRowBlocks; ++j) {
        s[j][0] = T::mfma32(a0, qreg[j][kk], s[j][0]);
        s[j][1] = T::mfma32(a1, qreg[j][kk], s[j][1]);
      }
    }
    if (need_mask) {
      keep_branch();
#pragma unroll
      for (int j = 0; j < kRowBlocks; ++j) {
        // key kl of the tile is visible to this lane's row iff kl < lim
        const int lim = pre ? count : min(count, i_row[j] - base + 1);
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int kl = (rr >> 2) * 8 + hf * 4 + (rr & 3);
          s[j][0][rr] = kl < lim ? s[j][0][rr] : -INFINITY;
          s[j][1][rr] = kl + 32 < lim ? s[j][1][rr] : -INFINITY;
        }
      }
    }
    float mx[kRowBlocks];
    bool need = false;
#pragma unroll
    for (int j = 0; j < kRowBlocks; ++j) {
      float m = fmaxf(s[j][0][0], s[j][1][0]);
#pragma unroll
      for (int rr = 1; rr < 16; ++rr) m = fmaxf(m, fmaxf(s[j][0][rr], s[j][1][rr]));
      mx[j] = fmaxf(m, xor_lane(m, 32)) * c_log2;
      need |= mx[j] > m_run[j] + kPfRescale;
    }
    if (__any(need)) {
      keep_branch();
#pragma unroll
      for (int j = 0; j < kRowBlocks; ++j) {
        const float mn = fmaxf(m_run[j], mx[j]);
        const float alpha = fast_exp2(m_run[j] - mn);
        m_run[j] = mn;
        l_run[j] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) o[j][db][rr] *= alpha;
      }
    }
    // probabilities, packed as the B operand of the PV product; row sums add the
    // rounded values (the ones PV uses) two at a time with a dot product against (1, 1)
    s16x8 pk[kRowBlocks][4];
#pragma unroll
    for (int j = 0; j < kRowBlocks; ++j) {
      float ls = l_run[j];
#pragma unroll
      for (int kp4 = 0; kp4 < 4; ++kp4) {
        const int mb = kp4 >> 1, r0 = (kp4 & 1) * 8;
        uint32_t pw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = fast_exp2(fmaf(s[j][mb][r0 + 2 * e], c_log2, -m_run[j]));
          const float p1 = fast_exp2(fmaf(s[j][mb][r0 + 2 * e + 1], c_log2, -m_run[j]));
          pw[e] = pack2<T>(p0, p1);
          ls = T::dot2(pw[e], T::kOnePair, ls);
        }
        pk[j][kp4] = __builtin_bit_cast(s16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
      }
      l_run[j] = ls;
    }
    // O^T += V^T P^T: each transposed V operand read feeds both row blocks
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      s16x8 a[4];
#pragma unroll
      for (int kp4 = 0; kp4 < 4; ++kp4) {
        const s16x4 lo = lds_read_tr16(sk + vaddr[db][0] + 16 * kp4 * D);
        const s16x4 hi = lds_read_tr16(sk + vaddr[db][1] + 16 * kp4 * D);
        a[kp4] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int j = 0; j < kRowBlocks; ++j)
#pragma unroll
        for (int kp4 = 0; kp4 < 4; ++kp4) o[j][db] = T::mfma32(a[kp4], pk[j][kp4], o[j][db]);
    }
  };

  int ids[1];
  tile_blocks(ld_tile, ids);
  load_tile(ld_tile, ids, 0);
  tile_blocks(KS + ld_tile, ids);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int st = 0; st < nstage; ++st) {
    load_tile(KS * st + KS + ld_tile, ids, (st + 1) & 1);   // next stage, lands during this one
    tile_blocks(KS * st + 2 * KS + ld_tile, ids);
    const int t = KS * st + kh;
    if (wave_active && t < total) compute(t, smem + (kh * 2 + (st & 1)) * L::TILE);
    __builtin_amdgcn_s_waitcnt(0);          // this wave's LDS-direct loads have landed
    __syncthreads();
  }

  // Merge the two key halves of each row group through LDS (the stage buffers are free):
  // key-half 1 waves publish (output, max, sum); key-half 0 waves combine and store.
  float* mbuf = reinterpret_cast<float*>(smem);
  constexpr int OPW = kRowBlocks * NDB * 16;       // output floats per lane
  static_assert(KS == 1 || (kRowWaves * (OPW + 2 * kRowBlocks) * 64) * 4 <= 2 * KS * L::TILE * 2,
                "merge buffer fits");
  float* my = mbuf + rw * (OPW + 2 * kRowBlocks) * 64;
  if (KS == 1) {
#pragma unroll
    for (int j = 0; j < kRowBlocks; ++j) {
      float lt = l_run[j];
      lt += xor_lane(lt, 32);
      if (!rvalid[j]) continue;
      const float inv = 1.0f / lt;
      uint16_t* orow = out + ((int64_t)(cu_b + i_row[j]) * hq + kvh * G + g_row[j]) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int d = 32 * db + r4 * 8 + hf * 4;
          uint2 uu;
          uu.x = pack2<T>(o[j][db][4 * r4 + 0] * inv, o[j][db][4 * r4 + 1] * inv);
          uu.y = pack2<T>(o[j][db][4 * r4 + 2] * inv, o[j][db][4 * r4 + 3] * inv);
          *reinterpret_cast<uint2*>(orow + d) = uu;
        }
    }
    return;
  }
  if (kh == 1) {
#pragma unroll
    for (int j = 0; j < kRowBlocks; ++j) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) my[((j * NDB + db) * 16 + rr) * 64 + lane] = o[j][db][rr];
      my[(OPW + 2 * j) * 64 + lane] = m_run[j];
      my[(OPW + 2 * j + 1) * 64 + lane] = l_run[j];
    }
  }
  __syncthreads();
  if (kh == 1) return;
#pragma unroll
  for (int j = 0; j < kRowBlocks; ++j) {
    const float m1 = my[(OPW + 2 * j) * 64 + lane];
    const float l1 = my[(OPW + 2 * j + 1) * 64 + lane];
    const float M = fmaxf(m_run[j], m1);
    const float a0 = fast_exp2(m_run[j] - M), a1 = fast_exp2(m1 - M);
    float lt = l_run[j] * a0 + l1 * a1;
    lt += xor_lane(lt, 32);
    if (!rvalid[j]) continue;
    const float inv0 = a0 / lt, inv1 = a1 / lt;
    uint16_t* orow = out + ((int64_t)(cu_b + i_row[j]) * hq + kvh * G + g_row[j]) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * db + r4 * 8 + hf * 4;
        float vals[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          vals[e] = o[j][db][4 * r4 + e] * inv0 + my[((j * NDB + db) * 16 + 4 * r4 + e) * 64 + lane] * inv1;
        uint2 uu;
        uu.x = pack2<T>(vals[0], vals[1]);
        uu.y = pack2<T>(vals[2], vals[3]);
        *reinterpret_cast<uint2*>(orow + d) = uu;
      }
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
  // Up to two work-groups per CU fit: with fewer work-groups than 2 x CUs the keys are
  // split inside each work-group instead, so every SIMD still runs two waves.
  const bool split = real < 2LL * device_cu_count();
  if (split)
    hipLaunchKernelGGL((prefill_kernel<T, D, 2>), dim3((unsigned)padded), dim3(512), 0, s,
                       (const uint16_t*)p.k, (const uint16_t*)p.v, p.block_stride, p.num_blocks,
                       (const uint16_t*)q, (const uint16_t*)kn, (const uint16_t*)vn, (uint16_t*)out,
                       cu, plen, bt, bt_stride, batch, hq, p.num_kv_heads, total_q, max_tiles, c,
                       (int)padded, (int)real);
  else
    hipLaunchKernelGGL((prefill_kernel<T, D, 1>), dim3((unsigned)padded), dim3(256), 0, s,
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
