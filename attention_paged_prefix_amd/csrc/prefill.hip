// Paged prefill: the rows of a new chunk attend to the sequence's cached prefix, read
// from the block pool through its block table, and causally to the chunk's own K/V.
//
// What is computed follows kvboost 0.6.0, "How it works" steps 3 and 5 (cached prefix
// plus live suffix in one forward pass) and "Flash Attention (CUDA)" (tiled attention
// with online softmax; fp16/bf16; head dims 64/96/128; causal masking that skips
// future K/V tiles).  That page's CUDA kernel is prior art; this kernel is laid out for
// CDNA4 (gfx950):
//
//  * Each wave owns 32 "virtual rows" v = i*G + g (chunk row i, query head kvh*G + g),
//    so the G query heads that share a KV head share every K/V tile staged in LDS
//    (GQA packing; works for any G, including 5).
//  * K/V tiles of 64 keys = four 16-token blocks, copied straight from the pool (or the
//    chunk's own K/V) into LDS by buffer loads with an LDS destination, 1 KiB per
//    instruction, through buffer resources sized to the valid rows (rows past the end
//    read as zero, with no memory traffic).  The 16-byte chunks of each LDS row are
//    permuted so that both operand read patterns are bank-conflict free.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16 (A = K rows
//    from LDS, B = Q held in registers), so each lane owns one query row; the output is
//    accumulated transposed, O^T += V^T P^T: the score accumulators are already the B
//    operand and V is read transposed with ds_read_b64_tr_b16.
//  * Software pipelined inside each wave: while the S MFMAs of tile j+1 run, the VALU
//    turns tile j's scores into probabilities; while the PV MFMAs of tile j run, it takes
//    tile j+1's row max.  K is staged one tile ahead of V.
//  * Online softmax in the exp2 domain, x = scale*log2(e)*q.k - m in one FMA (fp32; the
//    queries are not rescaled in 16 bits, which would cost precision at large scores).
//    The reference m is the first tile's row maximum; it only moves (and the output is
//    only rescaled) when a tile's partial row sum of probabilities exceeds 2^8 (a score
//    more than about 2^8 above it), which the sums already computed for the denominator
//    reveal, so no per-tile row maximum is taken.  Only tiles crossing the causal
//    diagonal or the end of the keys are masked; tiles entirely in the future of every
//    row are never visited.
#include <type_traits>

#include "kvb_device.h"
#include "kvb_launch.h"

namespace kvb {

constexpr int kRowWaves = 4;             // waves along the rows (32 rows each)
constexpr int kBM = 32 * kRowWaves;      // virtual rows per work-group
constexpr int kKT = 64;                  // keys per tile
constexpr float kPfNegBig = -1.0e30f;
// A lane's partial row sum of one tile's probabilities (32 keys) above this means some
// score is more than about 2^8 above the reference: the reference moves up.  Inf (an
// fp16 probability that overflowed) compares above it too.
constexpr float kPfSumLimit = 256.0f;

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

// Shared-prefix (cascade) form.  The rows are the single queries of `total_q` sequences
// (q as [sequence][query head][D], like decode) that all share one prefix, given as the
// block list `bt` of length `shared_len`; row i sees the shared keys below ctx[i].  The
// key tiles are split over `nks` work-groups of `ks_tiles` tiles, and each work-group
// writes (unnormalised output, max, sum) partials, in the exp2 domain, to workspace slot
// `ks` of its rows, for the decode merge.  With ctx null the kernel is ordinary prefill.
struct PfCascade {
  const int32_t* ctx;
  int max_ctx;                               // contexts are clamped to this, as in decode
  int shared_len;
  int ks_tiles, nks;
  float* ws_o;                               // [row][ws_slots][D], row = sequence*hq + head
  float* ws_ml;                              // [row][ws_slots][2]
  int ws_slots;
};

// Fused slot scatter (ordinary prefill only): with `slots` set, the chunk's own K/V rows
// are also written into the pool at their slots, as kvb_write_kv would, in the same launch.
// The prefill never reads those slots (its prefix rows are below P_b, the chunk's keys
// come from k_new/v_new), so the writes need no ordering against its reads.
struct PfWrite {
  const int64_t* slots;                      // [total_q]; slot = block*16 + row, < 0 = skip
  uint16_t* k;                               // the pool (same storage as kp / vp)
  uint16_t* v;
};

// 8-bit or 4-bit pool (QB = bits per code; kp/vp then hold codes, block_stride bytes):
// K code c of channel e stands for c * k_scale[kvh][e], V code c of token row r for
// c * v_scale[(block * hkv + kvh) * 16 + r].  The codes of each prefix block are staged
// into LDS by the wave that owns the block, then widened by the same wave into the 16-bit
// tile (V times its token's scale); the K channel scales are folded into the queries.
struct PfQuant {
  const float* v_scale;
  const float* k_scale;
};

// Widening of staged codes into 16-bit tile values.  K codes are widened exactly (their
// channel scales are folded into the queries); V codes become code * s, the token's
// scale s applied in fp32 and the product rounded to nearest even.  In fp16 both start
// from the same bit trick: a code biased to unsigned and placed under the exponent of
// 1024 is the fp16 value 1024 + code + bias, exact; K subtracts the constant in fp16,
// V takes (1024 + code + bias) * s - (1024 + bias) * s in one mixed-precision FMA.
// Four int8 codes (one dword, channel order) -> two packed pairs.  ns = -1152 * s.
template <typename T, bool V>
__device__ inline void widen_q8(uint32_t x, float s, float ns, uint32_t& a, uint32_t& b) {
  if constexpr (std::is_same<T, F16>::value) {
    const uint32_t u = x ^ 0x80808080u;                     // code + 128
    const f16x2v h0 = __builtin_bit_cast(f16x2v, __builtin_amdgcn_perm(0x64646464u, u, 0x04010400u));
    const f16x2v h1 = __builtin_bit_cast(f16x2v, __builtin_amdgcn_perm(0x64646464u, u, 0x04030402u));
    if constexpr (!V) {
      const f16x2v bias = {(_Float16)-1152.f, (_Float16)-1152.f};
      a = __builtin_bit_cast(uint32_t, h0 + bias);
      b = __builtin_bit_cast(uint32_t, h1 + bias);
    } else {
      f16x2v r0, r1;
      r0.x = (_Float16)__builtin_fmaf((float)h0.x, s, ns);
      r0.y = (_Float16)__builtin_fmaf((float)h0.y, s, ns);
      r1.x = (_Float16)__builtin_fmaf((float)h1.x, s, ns);
      r1.y = (_Float16)__builtin_fmaf((float)h1.y, s, ns);
      a = __builtin_bit_cast(uint32_t, r0);
      b = __builtin_bit_cast(uint32_t, r1);
    }
  } else {
    const int32_t xi = (int32_t)x;
    float f0 = (float)((xi << 24) >> 24), f1 = (float)((xi << 16) >> 24);
    float f2 = (float)((xi << 8) >> 24), f3 = (float)(xi >> 24);
    if constexpr (V) {
      f0 *= s;
      f1 *= s;
      f2 *= s;
      f3 *= s;
    }
    a = pack2<T>(f0, f1);
    b = pack2<T>(f2, f3);
  }
}
// Eight 4-bit codes (one dword; channel 2i in the low nibble of byte i, two's
// complement) -> four packed pairs.  In fp16, byte k is copied into both halves with its
// low nibble (biased, + 8) under the exponent of 1024 in the low half and its high nibble
// times 16 in the high half; K removes both biases with one packed FMA, V applies s.
template <typename T, bool V>
__device__ inline void widen_q4(uint32_t x, float s, uint4& o) {
  uint32_t w[4];
  if constexpr (std::is_same<T, F16>::value) {
    const uint32_t u = x ^ 0x88888888u;
    const f16x2v mul = {(_Float16)1.f, (_Float16)0.0625f};
    const f16x2v add = {(_Float16)-1032.f, (_Float16)-72.f};
    const float s16 = s * 0.0625f, nlo = -1032.f * s, nhi = -72.f * s;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t y = __builtin_amdgcn_perm(0u, u, 0x0c000c00u | ((uint32_t)k << 16) | (uint32_t)k);
      const f16x2v z = __builtin_bit_cast(f16x2v, (y & 0x00F0000Fu) | 0x64006400u);
      if constexpr (!V) {
        w[k] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(z, mul, add));
      } else {
        f16x2v r;
        r.x = (_Float16)__builtin_fmaf((float)z.x, s, nlo);
        r.y = (_Float16)__builtin_fmaf((float)z.y, s16, nhi);
        w[k] = __builtin_bit_cast(uint32_t, r);
      }
    }
  } else {
    const int32_t xi = (int32_t)x;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float f0 = (float)((xi << (28 - 8 * k)) >> 28), f1 = (float)((xi << (24 - 8 * k)) >> 28);
      if constexpr (V) {
        f0 *= s;
        f1 *= s;
      }
      w[k] = pack2<T>(f0, f1);
    }
  }
  o = make_uint4(w[0], w[1], w[2], w[3]);
}

// Work-group = 4 * KS waves.  Wave w handles the 32 virtual rows 32*(w & 3) .. +31 of
// the work-group's 128 and the key tiles t with t % KS == (w >> 2) ("key part").  With
// KS = 2 (small grids: 8 waves, one work-group per CU) the two waves of a row group split
// the keys and merge their (output, max, sum) through LDS at the end; with KS = 1 (large
// grids) two independent 4-wave work-groups share a CU.
//
// Step j of a key part covers its tile KS*j + part.  The loop is software pipelined
// inside each wave: step j issues the S MFMAs of tile j+1 while the VALU turns tile j's
// scores into probabilities, then the PV MFMAs of tile j while the VALU takes tile j+1's
// row max and scales its scores.  K is therefore staged one tile ahead of V: LDS holds
// two K buffers and two V buffers per key part; step j loads K of tile j+2 and V of tile
// j+1, and one barrier per step publishes them.
// MODE: kModePrefill (prefix from the pool, the chunk's own K/V from k_new/v_new),
// kModeCascade (the shared-prefix form above), kModePooled (every key, the chunk's own
// included, read from the pool through the block table after kvb_write_kv).
constexpr int kModePrefill = 0, kModeCascade = 1, kModePooled = 2;

template <typename T, int D, int KS, int MODE, int QB = 0, int RW = kRowWaves>
__global__ void __launch_bounds__(64 * RW * KS, RW * KS == 4 ? 2 : 1)
prefill_kernel(const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
               int64_t block_stride, int num_blocks, const uint16_t* __restrict__ q,
               const uint16_t* __restrict__ kn, const uint16_t* __restrict__ vn,
               uint16_t* __restrict__ out, const int32_t* __restrict__ cu,
               const int32_t* __restrict__ plen, const int32_t* __restrict__ bt, int bt_stride,
               int batch, int hq, int hkv, int total_q, int max_tiles, float c_log2, int padded,
               int real, const int32_t* __restrict__ order, PfCascade cas, PfWrite wr,
               PfQuant qz) {
  using L = PfLayout<D>;
  constexpr int CPR = L::CPR;
  constexpr int NKK = D / 16;                // MFMA k-steps over head_dim
  constexpr int NDB = D / 32;                // 32-wide d blocks of the output
  constexpr int NLD = CPR / 4;               // 1 KiB load instructions per 16-row block
  constexpr int HT = kKT * D;                // elements of one K (or V) tile
  constexpr uint32_t HTB = HT * 2;           // bytes of one K (or V) tile
  constexpr int NPV = 4 * NDB;               // PV MFMAs per tile (2 V reads each)
  static_assert(2 * NLD == NKK, "one load per S step");
  // RW row waves of 32 rows: 4 (each wave stages K and V of its block of every tile), or 8
  // (ordinary prefill, one key part: waves 0-3 stage the K blocks, waves 4-7 the V blocks)
  static_assert(RW == 4 || (RW == 8 && KS == 1 && MODE == kModePrefill), "row-wave forms");
  constexpr int BM = 32 * RW;                // virtual rows per work-group
  static_assert(QB == 0 || (MODE == kModePrefill && (QB == 8 || QB == 4)), "quantised pools: prefill only");
  // quantised pool: code bytes per token row and per block; a block's codes are staged by
  // QNL loads of 1 KiB (the tail past the block reads as zero) into QAREA bytes of LDS
  constexpr int QROW = D * (QB ? QB : 16) / 8;
  constexpr int QNL = (kBlock * QROW + 1023) / 1024;
  constexpr uint32_t QAREA = QB ? 1024u * QNL : 0u;

  // Tile buffers per key part: NBUF for K and NBUF for V.  Two (tiles loaded one step
  // ahead) in general; three (two steps ahead, so a step's loads stay in flight across its
  // barrier) for the 16-bit ordinary prefill at head dims 64 and 96, where they fit with
  // two work-groups per CU.
  constexpr int NBUF = (MODE == kModePrefill && QB == 0 && RW == 4 && D <= 96) ? 3 : 2;
  // [key part][K | V buffers][64 x D], then (quantised pool) per wave: K codes, V codes
  // (8 row waves: the codes of its one tensor)
  constexpr uint32_t QW = (RW == 8 ? 1u : 2u) * QAREA;       // code bytes per wave
  __shared__ __attribute__((aligned(16))) uint16_t smem[KS * 2 * NBUF * HT + KS * RW * QW / 2];

  int lid = xcd_logical_id(blockIdx.x, padded);
  if (lid >= real) return;
  // with a dispatch plan, the position in the XCD's range names the work item
  if (order) lid = order[lid];
  // logical id -> (kvh, b, key split, tile), tile fastest and KV head slowest
  constexpr bool cascade = MODE == kModeCascade;
  constexpr bool pooled = MODE == kModePooled;
  int r = lid;
  const int tile = r % max_tiles; r /= max_tiles;
  const int ks = cascade ? r % cas.nks : 0;
  if (cascade) r /= cas.nks;
  const int b = r % batch;
  const int kvh = r / batch;
  const int G = hq / hkv;
  const int cu_b = cascade ? 0 : min(max(cu[b], 0), total_q);
  const int C = cascade ? total_q : max(0, min(cu[b + 1], total_q) - cu_b);
  const int nrows = C * G;
  const int v0 = tile * BM;
  if (v0 >= nrows) return;
  const int P0 = max(0, min(cascade ? cas.shared_len : plen[b], bt_stride * kBlock));

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = uniform(tid >> 6);
  const int lr = lane & 31, hf = lane >> 5;
  const int rw = w & (RW - 1);                              // row group
  const int kh = KS == 1 ? 0 : w / RW;                       // key part
  // which tensors this wave stages: both (4 row waves), K or V (8 row waves)
  const bool st_k = RW == 4 || w < 4, st_v = RW == 4 || w >= 4;

  // this lane's query row (virtual row v = i*G + g)
  const int vrow = v0 + 32 * rw + lr;
  const bool rvalid = vrow < nrows;
  const int i_row = rvalid ? vrow / G : C;
  const int g_row = rvalid ? vrow - (vrow / G) * G : 0;
  s16x8 qreg[NKK];
  {
    const uint16_t* qrow = q + ((int64_t)(cu_b + i_row) * hq + kvh * G + g_row) * D + 8 * hf;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      if (rvalid) qreg[kk] = *reinterpret_cast<const s16x8*>(qrow + 16 * kk);
      else qreg[kk] = s16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  const bool wave_active = v0 + 32 * rw < nrows;

  const int last_row = min(nrows, v0 + BM) - 1;
  const int i_first = v0 / G;
  // cascade: each row (sequence) sees only the shared keys below its context length.
  // wg_lim is the smallest such limit over the work-group's rows; keys at or past the
  // largest one are not even loaded (they read as zero), so every key row that reaches
  // the PV product holds a real token of some sequence of this work-group.
  // pooled: the chunk's keys follow the prefix in the pool; chunk row i sees keys up to
  // P0 + i, and keys past the work-group's last row are not loaded.
  int row_lim = 0x7fffffff, wg_lim = 0x7fffffff, P = P0;
  if constexpr (pooled) {
    row_lim = rvalid ? P0 + i_row + 1 : 0;
    wg_lim = P0 + i_first + 1;
    P = min(P0 + last_row / G + 1, bt_stride * kBlock);
  }
  if constexpr (cascade) {
    const int cap = min(P0, cas.max_ctx);
    row_lim = rvalid ? min(cap, max(0, cas.ctx[i_row])) : 0;
    int mn = 0x7fffffff, mx = 0;
    for (int i = i_first + lane; i <= last_row / G; i += 64) {
      const int l = min(cap, max(0, cas.ctx[i]));
      mn = min(mn, l);
      mx = max(mx, l);
    }
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
      mn = min(mn, __shfl_xor(mn, sh, 64));
      mx = max(mx, __shfl_xor(mx, sh, 64));
    }
    wg_lim = uniform(mn);
    P = uniform(mx);
  }
  // key tiles [t_begin, total): prefix tiles below n_pre, then the chunk's own tiles
  // (none in the cascade form, where this work-group covers one split of the prefix)
  const int t_begin = cascade ? ks * cas.ks_tiles : 0;
  const int n_pre = cascade ? min((P + kKT - 1) / kKT, t_begin + cas.ks_tiles) : (P + kKT - 1) / kKT;
  const int self_n = (cascade || pooled) ? 0 : last_row / G + 1;   // chunk keys needed here
  const int n_self = (self_n + kKT - 1) / kKT;
  const int total = n_pre + n_self;
  const int nstage = max(1, (total - t_begin + KS - 1) / KS);
  // prefix tiles of this key part (its steps u < n_pre_part compute prefix scores)
  const int n_pre_part = max(0, (n_pre - t_begin - kh + KS - 1) / KS);

  // Quantised pool: prefix scores are taken with the queries times kscale[e] / kmx (kmx =
  // the KV head's largest K channel scale, so no query element grows and fp16 cannot
  // overflow) against the integer codes, and scaled by c_log2 * kmx; the chunk's own
  // tiles use the plain queries and c_log2.  c_cur is the factor of the tile whose
  // scores the current step computes.
  float c_cur = c_log2;
  if constexpr (QB != 0) {
    const float* ksc = qz.k_scale + (int64_t)kvh * D;
    float kmx = 0.f;
    for (int e = lane; e < D; e += 64) kmx = fmaxf(kmx, ksc[e]);
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) kmx = fmaxf(kmx, __shfl_xor(kmx, sh, 64));
    const float kinv = kmx > 0.f ? 1.f / kmx : 0.f;
    if (n_pre_part > 0) {
      c_cur = fmaxf(c_log2 * kmx, 1e-30f);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const u32x4 w4 = __builtin_bit_cast(u32x4, qreg[kk]);
        u32x4 o4;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = 16 * kk + 8 * hf + 2 * i;
          o4[i] = pack2<T>(lo_f32<T>(w4[i]) * (ksc[e] * kinv), hi_f32<T>(w4[i]) * (ksc[e + 1] * kinv));
        }
        qreg[kk] = __builtin_bit_cast(s16x8, o4);
      }
    }
  }
  // the plain queries again (quantised pool, at the first tile of the chunk itself);
  // the row is recomputed from an opaque copy of the thread id so that nothing of it
  // stays live across the loop
  auto reload_q = [&]() {
    int tq = threadIdx.x;
    asm volatile("" : "+v"(tq));
    const int vr = v0 + 32 * rw + (tq & 31);
    const int ir = vr / G;
    const uint16_t* qr = q + ((int64_t)(cu_b + ir) * hq + kvh * G + (vr - ir * G)) * D + 8 * ((tq >> 5) & 1);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      if (vr < nrows) qreg[kk] = *reinterpret_cast<const s16x8*>(qr + 16 * kk);
      else qreg[kk] = s16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  };

  f32x16 o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) o[i] = f32x16{};
  // m_run: the row's reference (exp2 domain); l_run: this lane's half of the row sum
  float m_run = 0.f, l_run = 0.f;

  // ---- LDS: key part kh owns 2*NBUF tile buffers (bytes): K0 V0 K1 V1 with two, K0 K1 K2
  // V0 V1 V2 with three.  All read and write addresses are a per-lane register plus a
  // constant.
  char* const lds = reinterpret_cast<char*>(smem);
  const uint32_t part_base = (uint32_t)(kh * 2 * NBUF * HTB);
  // byte offsets of K buffer i and V buffer i within the key part (two buffers: K0 V0 K1 V1)
  constexpr auto kOffK = [](int i) -> uint32_t { return (uint32_t)((NBUF == 2 ? 2 * i : i) * HTB); };
  constexpr auto kOffV = [](int i) -> uint32_t { return (uint32_t)((NBUF == 2 ? 2 * i + 1 : NBUF + i) * HTB); };
  constexpr uint32_t kOffK0 = kOffK(0), kOffV0 = kOffV(0), kOffK1 = kOffK(1);

  // ---- loader: the 4 waves of key part kh stage that part's tiles; wave (w & 3) loads
  // block (w & 3) of a tile.  Instruction m of a block fills LDS chunks 64m..64m+63 of
  // that block; lane L's chunk holds row (64m+L)/CPR, logical chunk inv(row, (64m+L)%CPR).
  // Byte offset = row * (source row pitch) + column bytes; the pitch is D*2 in the pool
  // and hkv*D*2 in the chunk's own K/V.
  // ld_offK/V[m]: the byte offset for a pool block (row pitch D*2); a source with another
  // pitch adds row * (pitch - D*2).  The row of instruction m is ld_row0 + m * 64/CPR
  // where CPR divides 64 (head dims 64, 128), else kept per instruction.
  const int ld_blk = w & 3;
  constexpr bool kRowAffine = 64 % CPR == 0;
  uint32_t ld_offK[NLD], ld_offV[NLD], ld_rows[kRowAffine ? 1 : NLD];
#pragma unroll
  for (int m = 0; m < NLD; ++m) {
    const int pos = 64 * m + lane;
    const int rb = pos / CPR, cp = pos - (pos / CPR) * CPR;
    if (!kRowAffine || m == 0) ld_rows[m] = (uint32_t)rb;
    ld_offK[m] = (uint32_t)rb * (uint32_t)(D * 2) + (uint32_t)L::invK(rb, cp) * 16;
    ld_offV[m] = (uint32_t)rb * (uint32_t)(D * 2) + (uint32_t)L::invV(rb, cp) * 16;
  }
  auto ld_row = [&](int m) -> uint32_t {
    if constexpr (kRowAffine) return ld_rows[0] + (uint32_t)(m * (64 / CPR));
    else return ld_rows[m];
  };
  const uint32_t ld_dst = part_base + (uint32_t)(kBlock * ld_blk * CPR * 16);
  const int32_t* bt_row = bt + (int64_t)b * bt_stride;
  const int64_t head_off = (int64_t)kvh * kBlock * D;
  const uint16_t* kbase = kp + head_off;                          // + block * block_stride
  const uint16_t* vbase = vp + head_off;
  const uint16_t* knb = kn + ((int64_t)cu_b * hkv + kvh) * D;     // + row * hkv * D
  const uint16_t* vnb = vn + ((int64_t)cu_b * hkv + kvh) * D;
  const uint32_t self_row_bytes = (uint32_t)(hkv * D * 2);
  const uint32_t bs32 = (uint32_t)block_stride;
  // quantised pool: the KV head's codes in a block
  const uint8_t* kq_base = reinterpret_cast<const uint8_t*>(kp) + (int64_t)kvh * kBlock * QROW;
  const uint8_t* vq_base = reinterpret_cast<const uint8_t*>(vp) + (int64_t)kvh * kBlock * QROW;

  // tiles of the chunk itself crossing the causal diagonal, or the end of the keys, need
  // per-row masking (uniform per work-group)
  // (by-value captures: a select between two captured references otherwise becomes a
  // load through a selected pointer into a closure held in scratch memory)
  auto tile_needs_mask = [=](int t) {
    const bool pre = t < n_pre;
    const int base = pre ? t * kKT : (t - n_pre) * kKT;
    const int count = pre ? min(kKT, P - base) : min(kKT, self_n - base);
    return (count < kKT) || (!pre && base + kKT - 1 > i_first) || (pre && base + kKT > wg_lim);
  };

  // Descriptor table of this wave's tile sequence: lane i describes the wave's block of
  // tile KS*(u0+i)+kh (u = step index): K and V source addresses and valid bytes (rows
  // past the end read as zero; past the last tile the size is zero), plus wave-wide bit
  // masks of "prefix tile" and "needs masking".  Filled 64 tiles at a time with one
  // gathered block-table read; a step then only reads lanes out of it.
  uint32_t tk_lo, tk_hi, tv_lo, tv_hi, t_nb, t_pb = 0;
  uint64_t pre_bits, mask_bits;
  int u0 = 0;
  auto refill = [&](int u_first) {
    const int t = t_begin + KS * (u_first + lane) + kh;
    const bool pre = t < n_pre;
    const int jb = t * 4 + ld_blk;
    const bool inpre = pre && jb * kBlock < P;
    const int pb = inpre ? bt_row[jb] : -1;
    const bool pvalid = inpre && (uint32_t)pb < (uint32_t)num_blocks;
    const int rows_pre = max(0, min(kBlock, P - jb * kBlock));
    const int row0 = (t - n_pre) * kKT + kBlock * ld_blk;
    const int rows_self = (!pre && t < total) ? max(0, min(kBlock, self_n - row0)) : 0;
    uint64_t ak, av;
    if constexpr (QB == 0) {
      const uint64_t off = pre ? (uint64_t)(pvalid ? (uint32_t)pb : 0u) * bs32
                               : (uint64_t)(uint32_t)min(max(row0, 0), C) * (uint32_t)(hkv * D);
      ak = (uint64_t)(pre ? kbase : knb) + 2 * off;
      av = (uint64_t)(pre ? vbase : vnb) + 2 * off;
    } else {
      // codes: byte offsets, block_stride in bytes
      const uint64_t offp = (uint64_t)(pvalid ? (uint32_t)pb : 0u) * (uint64_t)bs32;
      const uint64_t offs = 2 * (uint64_t)(uint32_t)min(max(row0, 0), C) * (uint32_t)(hkv * D);
      ak = pre ? (uint64_t)kq_base + offp : (uint64_t)knb + offs;
      av = pre ? (uint64_t)vq_base + offp : (uint64_t)vnb + offs;
      t_pb = pvalid ? (uint32_t)pb : 0xffffffffu;
    }
    tk_lo = (uint32_t)ak;
    tk_hi = (uint32_t)(ak >> 32);
    tv_lo = (uint32_t)av;
    tv_hi = (uint32_t)(av >> 32);
    t_nb = pre ? (pvalid ? (uint32_t)(rows_pre * QROW) : 0u)
               : (rows_self > 0 ? (uint32_t)(rows_self - 1) * self_row_bytes + D * 2 : 0u);
    pre_bits = __ballot(pre);
    mask_bits = __ballot(tile_needs_mask(t));
  };
  struct LdDesc {
    __amdgpu_buffer_rsrc_t rs;
    uint32_t dpitch;                                // row pitch - D*2 (bytes)
    uint32_t dst;                                   // LDS byte address of the block
  };
  auto desc = [&](int li, bool is_v, uint32_t buf_off) -> LdDesc {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(is_v ? tv_lo : tk_lo), li);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(is_v ? tv_hi : tk_hi), li);
    const int nb = __builtin_amdgcn_readlane((int)t_nb, li);
    LdDesc d;
    d.rs = __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, nb, kBufDword3);
    d.dpitch = ((pre_bits >> li) & 1) ? 0u : self_row_bytes - (uint32_t)(D * 2);
    d.dst = ld_dst + buf_off;
    return d;
  };
  // load instruction m (1 KiB) of a part; `pre` (compile-time): the tile is known to be
  // a prefix tile, whose offsets are precomputed
  // (quantised pool: only the chunk's own tiles are loaded this way, so the offsets are
  // recomputed from an opaque lane id at each use instead of held in registers)
  auto issue = [&](const LdDesc& d, bool is_v, int m, auto pre_c) {
    uint32_t base, row;
    if constexpr (QB != 0) {
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int pos = 64 * m + ln;
      const int rb = pos / CPR, cp = pos - (pos / CPR) * CPR;
      base = (uint32_t)rb * (uint32_t)(D * 2) + (uint32_t)(is_v ? L::invV(rb, cp) : L::invK(rb, cp)) * 16;
      row = (uint32_t)rb;
    } else {
      base = is_v ? ld_offV[m] : ld_offK[m];
      row = ld_row(m);
    }
    const uint32_t off = decltype(pre_c)::value ? base : base + row * d.dpitch;
    buf_load16_lds(d.rs, off, lds + d.dst + 64 * 16 * m);
  };
  auto issue_all = [&](const LdDesc& d, bool is_v, auto pre_c) {
#pragma unroll
    for (int m = 0; m < NLD; ++m) issue(d, is_v, m, pre_c);
  };
  using Gen = std::false_type;
  using Pre = std::true_type;

  // ---- quantised pool: each wave stages the codes of its own block of a prefix tile
  // into its code area (K codes, then V codes; no other wave reads them) and later widens
  // them into the 16-bit tile.  Lane L widens row L/4 of the block, 8-code chunks
  // (L%4)*NCQ .. +NCQ-1.
  const uint32_t q_area = (uint32_t)(KS * 2 * NBUF * HTB) + (uint32_t)w * QW;
  // LDS offset of the staged V codes within the wave's area
  constexpr uint32_t QV = RW == 8 ? 0u : QAREA;
  constexpr int NCQ = D / 32;
  auto qload = [&](int li, bool is_v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(is_v ? tv_lo : tk_lo), li);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(is_v ? tv_hi : tk_hi), li);
    const int nb = __builtin_amdgcn_readlane((int)t_nb, li);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, nb, kBufDword3);
#pragma unroll
    for (int i = 0; i < QNL; ++i)
      buf_load16_lds(rs, 1024u * i + 16u * lane, lds + q_area + (is_v ? QV : 0u) + 1024u * i);
  };
  // the V scale of this lane's row of the block (0 past its valid rows or for a missing
  // block: the buffer holds only the valid rows' scales)
  auto qscale = [&](int li) -> float {
    const int pb = __builtin_amdgcn_readlane((int)t_pb, li);
    const int nb = __builtin_amdgcn_readlane((int)t_nb, li);
    const float* sp = qz.v_scale + ((int64_t)max(pb, 0) * hkv + kvh) * kBlock;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(sp, (uint32_t)(nb / QROW) * 4u);
    return __builtin_bit_cast(float, buf_load4(rs, (uint32_t)(lane >> 2) * 4u));
  };
  // Widening: lane L holds code dwords NCW of row L/4 of each staged block (contiguous);
  // both blocks are read before either is widened.
  constexpr int NCW = NCQ * (QB ? QB : 8) / 4;
  struct QCodes { uint32_t k[NCW], v[NCW]; };
  auto qread = [&]() -> QCodes {
    QCodes c;
    const char* src = lds + q_area + (uint32_t)((lane >> 2) * QROW + (lane & 3) * NCW * 4);
#pragma unroll
    for (int h = 0; h < (RW == 8 ? 1 : 2); ++h) {
      // 8 row waves: the one staged tensor, in c.k
      uint32_t* d = h ? c.v : c.k;
      const char* p = src + (h ? QAREA : 0u);
      if constexpr (NCW % 4 == 0) {
#pragma unroll
        for (int i = 0; i < NCW / 4; ++i) {
          const uint4 x = *reinterpret_cast<const uint4*>(p + 16 * i);
          d[4 * i] = x.x; d[4 * i + 1] = x.y; d[4 * i + 2] = x.z; d[4 * i + 3] = x.w;
        }
      } else if constexpr (NCW % 2 == 0) {
#pragma unroll
        for (int i = 0; i < NCW / 2; ++i) {
          const uint2 x = *reinterpret_cast<const uint2*>(p + 8 * i);
          d[2 * i] = x.x; d[2 * i + 1] = x.y;
        }
      } else {
#pragma unroll
        for (int i = 0; i < NCW; ++i) d[i] = *reinterpret_cast<const uint32_t*>(p + 4 * i);
      }
    }
    return c;
  };
  auto qwiden = [&](auto is_v_c, const uint32_t (&cw)[NCW], uint32_t buf_off, float vs) {
    constexpr bool is_v = decltype(is_v_c)::value;
    const int r = lane >> 2, c0 = (lane & 3) * NCQ;
    const int trow = kBlock * ld_blk + r;
    // LDS byte address of chunk c0 + i of the row.  At head dims 64 and 128 the lane's
    // chunks differ only in their low bits: K positions are the first one's with those
    // bits XORed, V positions consecutive; head dim 96 computes each.
    const uint32_t row_base = part_base + buf_off + (uint32_t)(trow * CPR) * 16;
    const uint32_t a0 = row_base + (uint32_t)(is_v ? L::posV(trow, c0) : L::posK(trow, c0)) * 16;
    auto chunk_addr = [&](int i) -> uint32_t {
      if constexpr (D == 96)
        return row_base + (uint32_t)(is_v ? L::posV(trow, c0 + i) : L::posK(trow, c0 + i)) * 16;
      else if constexpr (is_v)
        return a0 + (uint32_t)(16 * i);
      else
        return a0 ^ (uint32_t)(16 * i);
    };
    const float ns = -1152.f * vs;
#pragma unroll
    for (int i = 0; i < NCQ; ++i) {
      uint4 o;
      if constexpr (QB == 8) {
        widen_q8<T, is_v>(cw[2 * i], vs, ns, o.x, o.y);
        widen_q8<T, is_v>(cw[2 * i + 1], vs, ns, o.z, o.w);
      } else {
        widen_q4<T, is_v>(cw[i], vs, o);
      }
      *reinterpret_cast<uint4*>(lds + chunk_addr(i)) = o;
    }
  };
  using IsK = std::false_type;
  using IsV = std::true_type;
  float vs_cur = 0.f;                               // V scale of the staged V codes

  // ---- per-lane LDS read addresses (bytes, including this key part's base)
  // K operand: row 32*half + lr, logical chunk 2*kk + hf
  uint32_t kaddr[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) kaddr[kk] = part_base + (uint32_t)(lr * CPR + L::posK(lr, 2 * kk + hf)) * 16;
  // V transpose-read source: rows 16*kp4 + 4*hf + (l%16)/4 (+8 for the high half),
  // columns 32*db + 16*((l/16)%2) + 4*(l%4), i.e. chunk 4*db + 2*((l/16)%2) + (l%4)/2
  // At head dims 128 and 64 the V chunk permutation repeats every 8 rows, so the high
  // half's address is the low half's plus a constant (one register per d block).
  constexpr bool kVRep8 = D != 96;
  constexpr int NVH = kVRep8 ? 1 : 2;
  uint32_t vaddr[NDB][NVH];
  {
    const int s4 = (lane & 15) >> 2;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int hi = 0; hi < NVH; ++hi) {
        const int row = 4 * hf + s4 + 8 * hi;
        const int c = 4 * db + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
        vaddr[db][hi] = part_base + (uint32_t)((row * CPR + L::posV(row, c)) * 16 + 8 * (lane & 1));
      }
  }
  auto k_operand = [&](uint32_t off, int kk, int half) {
    return *reinterpret_cast<const s16x8*>(lds + (kaddr[kk] + off + (uint32_t)(half * 32 * D * 2)));
  };
  auto v_operand = [&](uint32_t off, int db, int kp4) {
    const uint32_t a_hi = kVRep8 ? vaddr[db][0] + (uint32_t)(8 * CPR * 16) : vaddr[db][NVH - 1];
    const s16x4 lo = lds_read_tr16(reinterpret_cast<const uint16_t*>(lds + (vaddr[db][0] + off + (uint32_t)(kp4 * 16 * D * 2))));
    const s16x4 hi = lds_read_tr16(reinterpret_cast<const uint16_t*>(lds + (a_hi + off + (uint32_t)(kp4 * 16 * D * 2))));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };

  // keys of tile t this lane's row may not see -> -inf
  auto mask = [=](int t, f32x16* s) {
    const bool pre = t < n_pre;
    const int base = pre ? t * kKT : (t - n_pre) * kKT;
    const int count = pre ? min(kKT, P - base) : min(kKT, self_n - base);
    const int lim = pre ? min(count, row_lim - base) : min(count, i_row - base + 1);
    // key (rr/4)*8 + 4*hf + rr%4 (+32 in the second half): the lane's half moves to the
    // limit, so each comparison is against an immediate (per-key constants kept in
    // registers across the loop cost a dozen of them)
    const int limh = lim - 4 * hf;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      const int kc = (rr >> 2) * 8 + (rr & 3);
      s[0][rr] = kc < limh ? s[0][rr] : -INFINITY;
      s[1][rr] = kc + 32 < limh ? s[1][rr] : -INFINITY;
    }
  };
  // exp2 of the two scores of pair e (kp4 = e/4, element e%4) of a tile, packed
  // At head dims 64 and 96 (and 128 for the 16-bit pool with one key part) phase 2 of a
  // step (PV MFMAs) also takes the exponentials of the first half of the next tile's
  // scores (pe), so that both phases carry about the same VALU work under their MFMAs;
  // the other forms at 128 do not have the registers (the code pools spill, and with two
  // key parts it measured slower).
  constexpr bool kEarlyExp = D <= 96 || (D == 128 && QB == 0 && KS == 1);
  float pe[16];
#pragma unroll
  for (int rr = 0; rr < 16; ++rr) pe[rr] = 0.f;
  // packed probabilities of pair e, the first half from pe
  auto pack_pair_pe = [&](const f32x16 (&x)[2], int e) -> uint32_t {
    const int kp4 = e >> 2, ee = e & 3, mb = kp4 >> 1, r0 = (kp4 & 1) * 8;
    if (kEarlyExp && mb == 0) return pack2<T>(pe[r0 + 2 * ee], pe[r0 + 2 * ee + 1]);
    return pack2<T>(fast_exp2(x[mb][r0 + 2 * ee]), fast_exp2(x[mb][r0 + 2 * ee + 1]));
  };
  auto pack_pair = [&](const f32x16 (&x)[2], int e) -> uint32_t {
    const int kp4 = e >> 2, ee = e & 3, mb = kp4 >> 1, r0 = (kp4 & 1) * 8;
    return pack2<T>(fast_exp2(x[mb][r0 + 2 * ee]), fast_exp2(x[mb][r0 + 2 * ee + 1]));
  };
  // Probabilities of tile x (packed as the four B operands of the PV product) and this
  // lane's half of their row sum, which adds the rounded values (the ones PV uses) two
  // at a time with a dot product against (1, 1).
  auto probs = [&](const f32x16 (&x)[2], u32x4 (&pw)[4]) -> float {
    float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      pw[e >> 2][e & 3] = pack_pair(x, e);
      if (e & 1) ls1 = T::dot2(pw[e >> 2][e & 3], T::kOnePair, ls1);
      else ls0 = T::dot2(pw[e >> 2][e & 3], T::kOnePair, ls0);
    }
    return ls0 + ls1;
  };
  // Rare path: some score of tile x lies more than about 2^8 above the row's reference.
  // The reference moves up to the tile's row maximum: the output and the sum so far are
  // rescaled and the tile's probabilities recomputed.
  auto raise_reference = [&](f32x16 (&x)[2], u32x4 (&pw)[4]) -> float {
    float mx = fmaxf(x[0][0], x[1][0]);
#pragma unroll
    for (int rr = 1; rr < 16; ++rr) mx = fmaxf(mx, fmaxf(x[0][rr], x[1][rr]));
    const float d = fmaxf(halves_max(mx), 0.f);     // rows that stay below keep their reference
    const float alpha = fast_exp2(-d);
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) o[db][rr] *= alpha;
    m_run += d;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      x[0][rr] -= d;
      x[1][rr] -= d;
    }
    return probs(x, pw);
  };

  // ---- prologue: K and V of step 0, K of step 1; scores of step 0, whose row maximum is
  // the first reference
  refill(0);
  if constexpr (QB == 0) {
    if (st_k) issue_all(desc(0, false, kOffK0), false, Gen{});
    if (st_v) issue_all(desc(0, true, kOffV0), true, Gen{});
    if (st_k) issue_all(desc(1, false, kOffK1), false, Gen{});
  } else {
    // tiles 0 and 1 widened here, in two rounds through the one code area; the V codes
    // of tile 1 and the K codes of tile 2 stay staged for step 0
    const bool p0 = pre_bits & 1, p1 = (pre_bits >> 1) & 1, p2 = (pre_bits >> 2) & 1;
    if (p0) {
      if (st_k) qload(0, false);
      if (st_v) {
        qload(0, true);
        vs_cur = qscale(0);
      }
    } else {
      if (st_k) issue_all(desc(0, false, kOffK0), false, Gen{});
      if (st_v) issue_all(desc(0, true, kOffV0), true, Gen{});
    }
    __builtin_amdgcn_s_waitcnt(0);                  // this wave's own block
    if (p0) {
      const QCodes c = qread();
      if (st_k) qwiden(IsK{}, c.k, kOffK0, 0.f);
      if (st_v) qwiden(IsV{}, RW == 8 ? c.k : c.v, kOffV0, vs_cur);
    }
    if (p1) {
      if (st_k) qload(1, false);
      if (st_v) {
        qload(1, true);
        vs_cur = qscale(1);
      }
    } else {
      if (st_k) issue_all(desc(1, false, kOffK1), false, Gen{});
    }
    __builtin_amdgcn_s_waitcnt(0);
    if (p1 && st_k) {
      const QCodes c = qread();
      qwiden(IsK{}, c.k, kOffK1, 0.f);
    }
    if (p2 && st_k) qload(2, false);
  }
  f32x16 s_cur[2];
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if constexpr (NBUF == 3) {
    // two steps ahead: K of tile 2 and V of tile 1 fly while the first scores are taken
    issue_all(desc(2, false, kOffK(2)), false, Gen{});
    issue_all(desc(1, true, kOffV(1)), true, Gen{});
  }
  if (wave_active) {
    s_cur[0] = f32x16{};
    s_cur[1] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      s_cur[0] = T::mfma32(k_operand(kOffK0, kk, 0), qreg[kk], s_cur[0]);
      s_cur[1] = T::mfma32(k_operand(kOffK0, kk, 1), qreg[kk], s_cur[1]);
    }
    if (mask_bits & 1) mask(t_begin + kh, s_cur);
    float m = fmaxf(s_cur[0][0], s_cur[1][0]);
#pragma unroll
    for (int rr = 1; rr < 16; ++rr) m = fmaxf(m, fmaxf(s_cur[0][rr], s_cur[1][rr]));
    m = halves_max(m) * c_cur;
    // a row with no visible key in its first tile has none in the later ones either
    // (visibility only shrinks with the key index); its reference stays 0
    m_run = m == -INFINITY ? 0.f : m;
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) {
      s_cur[0][rr] = fmaf(s_cur[0][rr], c_cur, -m_run);
      s_cur[1][rr] = fmaf(s_cur[1][rr], c_cur, -m_run);
    }
    if constexpr (kEarlyExp) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) pe[rr] = fast_exp2(s_cur[0][rr]);
    }
  }
  __syncthreads();                                  // K buffer 0 is reloaded in step 0

  // ---- step j: loads K of tile j+NBUF and V of tile j+NBUF-1; S MFMAs of tile j+1, PV
  // MFMAs of tile j.  Tile t sits in K buffer t mod NBUF and V buffer t mod NBUF.  The
  // buffer index is a compile-time constant (the loop is unrolled by NBUF), so every LDS
  // address is a register plus an immediate.
  auto step = [&](int j, auto par_c, auto pre_c) {
    constexpr int PAR = decltype(par_c)::value;                 // j mod NBUF
    // K of tile j+NBUF into K buffer PAR (it held tile j, read in step j-1), V of tile
    // j+NBUF-1 into the V buffer of tile j-1; S of tile j+1 and PV of tile j read theirs
    constexpr uint32_t offK_ld = kOffK(PAR), offV_ld = kOffV((PAR + NBUF - 1) % NBUF);
    constexpr uint32_t offK_rd = kOffK((PAR + 1) % NBUF), offV_rd = kOffV(PAR);
    // next 64 tiles of the sequence (a quantised pool stages codes one tile further)
    if (j + NBUF + (QB ? 1 : 0) - u0 >= 64) {
      keep_branch();
      u0 = j + 1;
      refill(u0);
    }
    const int lk = j + NBUF - u0, lv = j + NBUF - 1 - u0;
    const LdDesc dk = desc(lk, false, offK_ld);
    const LdDesc dv = desc(lv, true, offV_ld);
    const bool need_mask = (mask_bits >> (j + 1 - u0)) & 1;
    // K of tile j+NBUF and V of tile j+NBUF-1: loaded straight into LDS, or (prefix tiles
    // of a quantised pool, two buffers) widened from the codes staged in the previous
    // step, whose place then takes the codes of K j+3 and V j+2
    bool k_direct = true, v_direct = true;
    if constexpr (QB != 0) {
      if (!decltype(pre_c)::value && j + 1 == n_pre_part) {   // tile j+1: the chunk's first own tile
        keep_branch();
        reload_q();
        c_cur = c_log2;
      }
      const bool kq = decltype(pre_c)::value || ((pre_bits >> lk) & 1);
      const bool vq = decltype(pre_c)::value || ((pre_bits >> lv) & 1);
      const QCodes c = qread();
      if (kq && st_k) qwiden(IsK{}, c.k, offK_ld, 0.f);
      if (vq && st_v) qwiden(IsV{}, RW == 8 ? c.k : c.v, offV_ld, vs_cur);
      if (st_k && ((pre_bits >> (lk + 1)) & 1)) qload(lk + 1, false);
      if (st_v && ((pre_bits >> (lv + 1)) & 1)) {
        qload(lv + 1, true);
        vs_cur = qscale(lv + 1);
      }
      k_direct = !kq;
      v_direct = !vq;
    }
    if (!wave_active) {
      if (k_direct && st_k) issue_all(dk, false, pre_c);
      if (v_direct && st_v) issue_all(dv, true, pre_c);
      return;
    }
    // Hand-interleaved: each step of a phase is a scheduling region of its own, so
    // operand reads issued there stay two MFMA steps ahead of their use and the VALU
    // work of the other tile fills the MFMA shadow.
    // Phase 1: S MFMAs of tile j+1, probabilities of tile j (exp + pack) and their row
    // sums, loads.
    f32x16 s_nxt[2] = {f32x16{}, f32x16{}};
    s16x8 ka[NKK][2];
    // probabilities of tile j, written in place as the four B operands of the PV product
    u32x4 pw[4];
    float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
    for (int kk = 0; kk < 2 && kk < NKK; ++kk) {
      ka[kk][0] = k_operand(offK_rd, kk, 0);
      ka[kk][1] = k_operand(offK_rd, kk, 1);
    }
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      __builtin_amdgcn_sched_barrier(0);
      // one load per step: bunched at the step start, the loads of all waves queue at
      // the memory pipeline and stall the issuing waves
      if (kk < NLD) {
        if (k_direct && st_k) issue(dk, false, kk, pre_c);
      } else {
        if (v_direct && st_v) issue(dv, true, kk - NLD, pre_c);
      }
      if (kk + 2 < NKK) {
        ka[kk + 2][0] = k_operand(offK_rd, kk + 2, 0);
        ka[kk + 2][1] = k_operand(offK_rd, kk + 2, 1);
      }
      s_nxt[0] = T::mfma32(ka[kk][0], qreg[kk], s_nxt[0]);
      s_nxt[1] = T::mfma32(ka[kk][1], qreg[kk], s_nxt[1]);
#pragma unroll
      for (int e = 0; e < 16; ++e) {              // pair e = (kp4 = e/4, element e%4)
        if (e * NKK / 16 == kk) {
          // each packed word is pinned here, in phase 1: pinning the assembled operand
          // instead made the compiler rebuild it with copies before the PV product
          uint32_t w2 = pack_pair_pe(s_cur, e);
          asm volatile("" : "+v"(w2));
          pw[e >> 2][e & 3] = w2;
        }
        if (kk > 0 && e * NKK / 16 == kk - 1) {   // row sums one MFMA step behind
          if (e & 1) ls1 = T::dot2(pw[e >> 2][e & 3], T::kOnePair, ls1);
          else ls0 = T::dot2(pw[e >> 2][e & 3], T::kOnePair, ls0);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (e * NKK / 16 == NKK - 1) {
        if (e & 1) ls1 = T::dot2(pw[e >> 2][e & 3], T::kOnePair, ls1);
        else ls0 = T::dot2(pw[e >> 2][e & 3], T::kOnePair, ls0);
      }
    if (need_mask) {
      keep_branch();
      mask(t_begin + KS * (j + 1) + kh, s_nxt);
    }
    float ls = ls0 + ls1;
    if (__any(!(ls <= kPfSumLimit))) {
      keep_branch();
      ls = raise_reference(s_cur, pw);
    }
    l_run += ls;
    s16x8 pk[4];
#pragma unroll
    for (int kp4 = 0; kp4 < 4; ++kp4) pk[kp4] = __builtin_bit_cast(s16x8, pw[kp4]);
    // Phase 2: PV MFMAs of tile j; exp2 arguments of tile j+1 (four per unit).
    s16x8 va[NPV];
#pragma unroll
    for (int i = 0; i < 2; ++i) va[i] = v_operand(offV_rd, i >> 2, i & 3);
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      if (i + 2 < NPV) va[i + 2] = v_operand(offV_rd, (i + 2) >> 2, (i + 2) & 3);
      o[i >> 2] = T::mfma32(va[i], pk[i & 3], o[i >> 2]);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (u * NPV / 8 != i) continue;
        const int h = u >> 2, r0 = (u & 3) * 4;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) s_nxt[h][r0 + rr] = fmaf(s_nxt[h][r0 + rr], c_cur, -m_run);
        // exponentials of the first half one unit group later, beside the second half's FMAs
        if (kEarlyExp && h == 1) {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) pe[r0 + rr] = fast_exp2(s_nxt[0][r0 + rr]);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::"v"(s_nxt[0]), "v"(s_nxt[1]));   // scaled scores stay in phase 2
    if constexpr (kEarlyExp) {
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) asm volatile("" ::"v"(pe[rr]));
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) s_cur[h] = s_nxt[h];
  };
  // End of a step: this wave's loads for the next step have landed (two buffers: all of
  // them; three: all but the NKK issued in this step, which the step after next reads),
  // then the work-group's barrier.
  // (With three buffers the barrier is the bare instruction: __syncthreads() fences
  // work-group memory, which waits for every outstanding load, the in-flight LDS-direct
  // ones included.  LDS reads of this step complete first, and the empty asm statements
  // keep the compiler from moving memory operations across.)
  auto sync = [&]() {
    if constexpr (NBUF == 2) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    } else {
      __builtin_amdgcn_s_waitcnt((NKK & 15) | ((NKK >> 4) << 14) | (7 << 4));   // vmcnt(NKK) lgkmcnt(0)
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
  };
  using Par0 = std::integral_constant<int, 0>;
  using Par1 = std::integral_constant<int, 1>;
  using Par2 = std::integral_constant<int, 2>;
  // Steps whose loads (K of tile j + 2 NBUF - 1 at the latest) are prefix tiles of this key
  // part take the precomputed offsets; the chunk's own tiles and the tail the general
  // form.  Every step ends in one barrier in both loops, so the key parts may switch
  // loops at different steps.  The loops are unrolled by NBUF, so the buffer of every step
  // is a compile-time constant.
  int j = 0;
  if constexpr (NBUF == 2) {
    for (; j + 3 < n_pre_part && j + 2 < nstage; j += 2) {
      step(j, Par0{}, Pre{});
      sync();
      step(j + 1, Par1{}, Pre{});
      sync();
    }
    for (; j + 2 < nstage; j += 2) {
      step(j, Par0{}, Gen{});
      sync();
      step(j + 1, Par1{}, Gen{});
      sync();
    }
    if (j + 1 < nstage) {
      step(j, Par0{}, Gen{});
      sync();
      ++j;
    }
  } else {
    for (; j + 5 < n_pre_part && j + 3 < nstage; j += 3) {
      step(j, Par0{}, Pre{});
      sync();
      step(j + 1, Par1{}, Pre{});
      sync();
      step(j + 2, Par2{}, Pre{});
      sync();
    }
    for (; j + 3 < nstage; j += 3) {
      step(j, Par0{}, Gen{});
      sync();
      step(j + 1, Par1{}, Gen{});
      sync();
      step(j + 2, Par2{}, Gen{});
      sync();
    }
    if (j + 1 < nstage) {
      step(j, Par0{}, Gen{});
      sync();
      ++j;
    }
    if (j + 1 < nstage) {
      step(j, Par1{}, Gen{});
      sync();
      ++j;
    }
    // the last steps' loads (past the end, or not read again) land before LDS is reused
    __builtin_amdgcn_s_waitcnt(0);
  }
  // last tile: probabilities and PV (V buffer of the last step)
  auto last = [&](auto par_c) {
    constexpr uint32_t off = kOffV(decltype(par_c)::value);
    u32x4 pw[4];
    float ls = probs(s_cur, pw);
    if (__any(!(ls <= kPfSumLimit))) {
      keep_branch();
      ls = raise_reference(s_cur, pw);
    }
    l_run += ls;
#pragma unroll
    for (int i = 0; i < NPV; ++i)
      o[i >> 2] = T::mfma32(v_operand(off, i >> 2, i & 3), __builtin_bit_cast(s16x8, pw[i & 3]), o[i >> 2]);
  };
  if (wave_active) {
    const int par = j % NBUF;
    if (par == 0) last(Par0{});
    else if (NBUF == 2 || par == 1) last(Par1{});
    else last(Par2{});
  }

  // Fused slot scatter: token i of the chunk is written by the work-group holding its first
  // virtual row i*G, so each token is written exactly once; 16 bytes per thread and item.
  if (MODE == kModePrefill && wr.slots) {
    const int i_lo = (v0 + G - 1) / G;
    const int i_hi = min(C, (v0 + BM + G - 1) / G);
    const int n_items = max(0, i_hi - i_lo) * 2 * CPR;
    for (int it = (int)threadIdx.x; it < n_items; it += (int)blockDim.x) {
      const int tok = i_lo + it / (2 * CPR);
      const int part = (it / CPR) & 1;                // 0: K, 1: V
      const int ch = it - (it / CPR) * CPR;
      const int64_t slot = wr.slots[cu_b + tok];
      if (slot < 0 || (slot >> 4) >= num_blocks) continue;     // outside the pool: skipped
      const int64_t src = ((int64_t)(cu_b + tok) * hkv + kvh) * D + 8 * ch;
      const int64_t dst = (slot >> 4) * block_stride + ((int64_t)kvh * kBlock + (slot & 15)) * D + 8 * ch;
      const uint4 val = *reinterpret_cast<const uint4*>((part ? vn : kn) + src);
      *reinterpret_cast<uint4*>((part ? wr.v : wr.k) + dst) = val;
    }
  }

  // Output row of this lane, recomputed from an opaque copy of the thread id so that the
  // pre-loop values need not stay live (in registers) across the main loop.
  int tid_e = threadIdx.x;
  asm volatile("" : "+v"(tid_e));
  const int vrow_e = v0 + 32 * rw + (tid_e & 31);
  const bool rvalid_e = vrow_e < nrows;
  const int i_e = vrow_e / G;
  const int64_t row_e = (int64_t)(cu_b + i_e) * hq + kvh * G + (vrow_e - i_e * G);
  const int hf_e = (tid_e >> 5) & 1;                 // the lane's half of the row's columns

  // Final values of this lane's row: get(db, r) is the unnormalised output, M the
  // reference max and L the row sum.  Ordinary prefill stores the normalised row in the
  // input type; the cascade form stores the partial (unnormalised output, M, L).
  auto emit = [&](auto get, float M, float L) {
    if (!rvalid_e) return;
    if (cascade) {
      float* wo = cas.ws_o + (row_e * cas.ws_slots + ks) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          *reinterpret_cast<float4*>(wo + 32 * db + r4 * 8 + hf_e * 4) =
              make_float4(get(db, 4 * r4), get(db, 4 * r4 + 1), get(db, 4 * r4 + 2), get(db, 4 * r4 + 3));
      if (hf_e == 0) {
        cas.ws_ml[(row_e * cas.ws_slots + ks) * 2 + 0] = M;
        cas.ws_ml[(row_e * cas.ws_slots + ks) * 2 + 1] = L;
      }
      return;
    }
    const float inv = 1.0f / L;
    uint16_t* const orow = out + row_e * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        uint2 uu;
        uu.x = pack2<T>(get(db, 4 * r4 + 0) * inv, get(db, 4 * r4 + 1) * inv);
        uu.y = pack2<T>(get(db, 4 * r4 + 2) * inv, get(db, 4 * r4 + 3) * inv);
        *reinterpret_cast<uint2*>(orow + 32 * db + r4 * 8 + hf_e * 4) = uu;
      }
  };

  // Merge the two key parts of each row group through LDS (the tile buffers are free):
  // key-part 1 waves publish (output, max, sum); key-part 0 waves combine and store.
  float* mbuf = reinterpret_cast<float*>(smem);
  constexpr int OPW = NDB * 16;                    // output floats per lane
  static_assert(KS == 1 || (RW * (OPW + 2) * 64) * 4 <= KS * 2 * NBUF * HT * 2, "merge buffer fits");
  float* my = mbuf + rw * (OPW + 2) * 64;
  // a row that saw no key here (sum 0) takes a reference far below any other, so a merge
  // with another part of its keys gives it no weight
  const float l_row = halves_sum(l_run);
  if (l_row == 0.f) m_run = kPfNegBig;
  if (KS == 1) {
    emit([&](int db, int rr) { return o[db][rr]; }, m_run, l_row);
    return;
  }
  __syncthreads();                                  // every wave is done with the tiles
  if (kh == 1) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) my[(db * 16 + rr) * 64 + lane] = o[db][rr];
    my[OPW * 64 + lane] = m_run;
    my[(OPW + 1) * 64 + lane] = l_run;
  }
  __syncthreads();
  if (kh == 1) return;
  const float m1 = my[OPW * 64 + lane];
  const float l1 = my[(OPW + 1) * 64 + lane];
  const float M = fmaxf(m_run, m1);
  const float a0 = fast_exp2(m_run - M), a1 = fast_exp2(m1 - M);
  const float lt = halves_sum(l_run * a0 + l1 * a1);
  emit([&](int db, int rr) { return o[db][rr] * a0 + my[(db * 16 + rr) * 64 + lane] * a1; }, M, lt);
}

// Longest-first dispatch plan.  The dispatcher starts work-groups in grid order, so on a
// grid of several rounds the last work-groups to start set the tail.  One work-group per
// XCD range (the logical ids one XCD runs) gives every item the key count of its
// sequence's last row (prefix plus chunk; 0 for tiles past the chunk), orders the range
// by it in 32 buckets relative to the range's largest count (a stable counting sort),
// largest first, and writes the item for each position (table order when every
// non-empty item is within 2x of the largest).  All row tiles of one (sequence, KV head)
// share that key, so they stay together in table order and stream its K/V through L2 at
// about the same time (keyed by each tile's own last row, the tiles of a long chunk fell
// into two buckets and re-read the prefix from HBM later); the plan is deterministic.
// Items never leave their XCD range, so each XCD keeps its KV heads in L2.
constexpr int kPlanThreads = 256;
constexpr int kPlanMax = 4096;          // items per XCD range sorted in LDS
constexpr int kPlanBuckets = 32;

__global__ void __launch_bounds__(kPlanThreads)
prefill_plan_kernel(const int32_t* __restrict__ cu, const int32_t* __restrict__ plen, int batch,
                    int G, int total_q, int bt_stride, int max_tiles, int bm, int padded, int real,
                    int32_t* __restrict__ order) {
  constexpr int NB = kPlanBuckets + 1;               // cost buckets, then the empty items
  constexpr int NW = kPlanThreads / 64;
  __shared__ int cost_s[kPlanMax];
  __shared__ int cnt[NB * kPlanThreads];             // [bucket][thread]: counts, then offsets
  __shared__ int s_wmax[NW], s_wmin[NW], s_wsum[NW];
  const int per = padded / kNumXcd;
  const int lo = blockIdx.x * per;
  const int n = min(per, real - lo);
  if (n <= 0) return;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  // item costs: prefix plus chunk of the item's sequence (0: an empty tile)
  int mx = 0, mn = 0x7fffffff;
  for (int i = t; i < n; i += kPlanThreads) {
    const int lid = lo + i;
    const int tile = lid % max_tiles;
    const int b = (lid / max_tiles) % batch;
    const int cu_b = min(max(cu[b], 0), total_q);
    const int C = max(0, min(cu[b + 1], total_q) - cu_b);
    const int64_t P0 = max((int64_t)0, min((int64_t)plen[b], (int64_t)bt_stride * kBlock));
    const int64_t nrows = (int64_t)C * G, v0 = (int64_t)tile * bm;
    const int cost = (int)(v0 < nrows ? min(P0 + C, (int64_t)0x3fffffff) : 0);
    cost_s[i] = cost;
    mx = max(mx, cost);
    if (cost > 0) mn = min(mn, cost);
  }
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) {
    mx = max(mx, __shfl_xor(mx, sh, 64));
    mn = min(mn, __shfl_xor(mn, sh, 64));
  }
  if (lane == 0) {
    s_wmax[wv] = mx;
    s_wmin[wv] = mn;
  }
  __syncthreads();
  int cmax = s_wmax[0], cmin = s_wmin[0];
#pragma unroll
  for (int k = 1; k < NW; ++k) {
    cmax = max(cmax, s_wmax[k]);
    cmin = min(cmin, s_wmin[k]);
  }
  if (2 * (int64_t)cmin > cmax) {
    // every tile within 2x of the largest: nothing to balance, and table order keeps
    // the tiles of one sequence and KV head together
    for (int i = t; i < n; i += kPlanThreads) order[lo + i] = lo + i;
    return;
  }
  // bucket kPlanBuckets - 1 holds the largest counts; empty tiles after every bucket
  auto bucket = [&](int c) {
    return c > 0 ? kPlanBuckets - 1 - (int)min((int64_t)kPlanBuckets - 1, (int64_t)c * kPlanBuckets / ((int64_t)cmax + 1))
                 : kPlanBuckets;
  };
  // Stable counting sort by bucket: thread t takes the contiguous items [i0, i1), counts
  // them per bucket in its own column, the counts are scanned in (bucket, thread) order,
  // and each thread places its items in order from its column's offsets.
  const int K = (n + kPlanThreads - 1) / kPlanThreads;
  const int i0 = min(n, t * K), i1 = min(n, i0 + K);
  for (int b = 0; b < NB; ++b) cnt[b * kPlanThreads + t] = 0;
  for (int i = i0; i < i1; ++i) ++cnt[bucket(cost_s[i]) * kPlanThreads + t];
  __syncthreads();
  // exclusive scan of the NB * kPlanThreads counts (bucket-major): thread t owns the
  // consecutive entries [NB t, NB t + NB)
  int run = 0;
  for (int k = 0; k < NB; ++k) run += cnt[NB * t + k];
  int incl = run;
#pragma unroll
  for (int sh = 1; sh < 64; sh <<= 1) {
    const int y = __shfl_up(incl, sh, 64);
    incl += lane >= sh ? y : 0;
  }
  if (lane == 63) s_wsum[wv] = incl;
  __syncthreads();
  int base = incl - run;
  for (int k = 0; k < wv; ++k) base += s_wsum[k];
  for (int k = 0; k < NB; ++k) {
    const int c = cnt[NB * t + k];
    cnt[NB * t + k] = base;
    base += c;
  }
  __syncthreads();
  for (int i = i0; i < i1; ++i) {
    const int pos = cnt[bucket(cost_s[i]) * kPlanThreads + t]++;
    order[lo + pos] = lo + i;
  }
}

int64_t prefill_plan_bytes(int batch, int hq, int total_q) {
  if (batch <= 0 || hq <= 0 || total_q <= 0) return 0;
  // items: batch * hkv * ceil(max_q * G / kBM) <= batch * (ceil(total_q * hq / kBM) + hq),
  // and no plan is made beyond kPlanMax items per XCD range
  int64_t items = (int64_t)batch * (((int64_t)total_q * hq + kBM - 1) / kBM + hq);
  if (items > (int64_t)kNumXcd * kPlanMax) items = (int64_t)kNumXcd * kPlanMax;
  return (items * 4 + 255) / 256 * 256;
}

template <typename T, int D, int MODE, int QB = 0>
static hipError_t launch_prefill_t(const kvb_pool& p, const void* q, const void* kn, const void* vn,
                                   void* out, const int32_t* cu, const int32_t* plen,
                                   const int32_t* bt, int bt_stride, int batch, int hq,
                                   int total_q, int max_q_len, float scale, const PfCascade& cas,
                                   int32_t* plan_ws, hipStream_t s, const int64_t* slots = nullptr,
                                   PfQuant qz = PfQuant{nullptr, nullptr}) {
  const PfWrite wr{slots, (uint16_t*)p.k, (uint16_t*)p.v};
  const int G = hq / p.num_kv_heads;
  const long long rows = (long long)max_q_len * G;
  const int cus = device_cu_count();
  // Quantised pool at head dim 96 on a grid of at least four rounds of one 256-row
  // work-group per CU: 8 row waves per work-group, each staging and widening one tensor of
  // its block of every tile, so a widened tile serves twice the rows.  Measured against
  // the 4-row-wave form: ragged mix at head dim 96 (fp16) 0.96x; at head dim 64 (bf16)
  // 1.02-1.03x; long_prefix (head dim 128, 2.5 rounds) 1.02x.  The 16-bit pool keeps 4 row
  // waves and two independent work-groups per CU everywhere (8 row waves: 1.05-1.06x).
  const long long real8 = (long long)batch * p.num_kv_heads * ((rows + 255) / 256);
  const bool rw8 = MODE == kModePrefill && QB != 0 && D == 96 && real8 >= 4LL * cus;
  const int bm = rw8 ? 256 : kBM;
  const int max_tiles = (int)((rows + bm - 1) / bm);
  const long long real = (long long)batch * p.num_kv_heads * cas.nks * max_tiles;
  if (real == 0) return hipSuccess;
  const long long padded = (real + kNumXcd - 1) / kNumXcd * kNumXcd;
  // scale 0 (all scores equal) is kept positive so masked -inf scores stay -inf
  const float c = fmaxf(scale * 1.4426950408889634f, 1e-30f);
  // Up to two work-groups per CU fit: with fewer work-groups than 2 x CUs the keys are
  // split inside each work-group instead, so every SIMD still runs two waves.
  const bool split = !rw8 && real < 2LL * cus;
  // a plan pays off only on a grid of several rounds
  const int32_t* order = nullptr;
  if (MODE == kModePrefill && plan_ws && !split && padded / kNumXcd <= kPlanMax) {
    hipLaunchKernelGGL(prefill_plan_kernel, dim3(kNumXcd), dim3(kPlanThreads), 0, s, cu, plen,
                       batch, G, total_q, bt_stride, max_tiles, bm, (int)padded, (int)real, plan_ws);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    order = plan_ws;
  }
  if constexpr (MODE == kModePrefill && QB != 0 && D == 96) {
    if (rw8) {
      hipLaunchKernelGGL((prefill_kernel<T, D, 1, MODE, QB, 8>), dim3((unsigned)padded), dim3(512), 0, s,
                         (const uint16_t*)p.k, (const uint16_t*)p.v, p.block_stride, p.num_blocks,
                         (const uint16_t*)q, (const uint16_t*)kn, (const uint16_t*)vn, (uint16_t*)out,
                         cu, plen, bt, bt_stride, batch, hq, p.num_kv_heads, total_q, max_tiles, c,
                         (int)padded, (int)real, order, cas, wr, qz);
      return hipGetLastError();
    }
  }
  if (split)
    hipLaunchKernelGGL((prefill_kernel<T, D, 2, MODE, QB>), dim3((unsigned)padded), dim3(512), 0, s,
                       (const uint16_t*)p.k, (const uint16_t*)p.v, p.block_stride, p.num_blocks,
                       (const uint16_t*)q, (const uint16_t*)kn, (const uint16_t*)vn, (uint16_t*)out,
                       cu, plen, bt, bt_stride, batch, hq, p.num_kv_heads, total_q, max_tiles, c,
                       (int)padded, (int)real, order, cas, wr, qz);
  else
    hipLaunchKernelGGL((prefill_kernel<T, D, 1, MODE, QB>), dim3((unsigned)padded), dim3(256), 0, s,
                       (const uint16_t*)p.k, (const uint16_t*)p.v, p.block_stride, p.num_blocks,
                       (const uint16_t*)q, (const uint16_t*)kn, (const uint16_t*)vn, (uint16_t*)out,
                       cu, plen, bt, bt_stride, batch, hq, p.num_kv_heads, total_q, max_tiles, c,
                       (int)padded, (int)real, order, cas, wr, qz);
  return hipGetLastError();
}

template <typename F>
static hipError_t dispatch_prefill(const kvb_pool& p, F&& f) {
  const bool bf = p.dtype == KVB_BF16;
  switch (p.head_dim) {
    case 64:  return bf ? f(BF16{}, std::integral_constant<int, 64>{}) : f(F16{}, std::integral_constant<int, 64>{});
    case 96:  return bf ? f(BF16{}, std::integral_constant<int, 96>{}) : f(F16{}, std::integral_constant<int, 96>{});
    default:  return bf ? f(BF16{}, std::integral_constant<int, 128>{}) : f(F16{}, std::integral_constant<int, 128>{});
  }
}

hipError_t launch_prefill(const kvb_pool& p, const void* q, const void* kn, const void* vn, void* out,
                          const int32_t* cu, const int32_t* plen, const int32_t* bt, int bt_stride,
                          int batch, int hq, int total_q, int max_q_len, int max_prefix_len,
                          float scale, void* plan_ws, hipStream_t s, const int64_t* slots) {
  (void)max_prefix_len;
  const PfCascade none{nullptr, 0, 0, 0, 1, nullptr, nullptr, 0};
  return dispatch_prefill(p, [&](auto t, auto d) {
    return launch_prefill_t<decltype(t), decltype(d)::value, kModePrefill>(p, q, kn, vn, out, cu, plen, bt, bt_stride,
                                                             batch, hq, total_q, max_q_len, scale, none,
                                                             (int32_t*)plan_ws, s, slots);
  });
}

hipError_t launch_prefill_quant(const kvb_pool_q8& p, int bits, int dtype, const void* q,
                                const void* kn, const void* vn, void* out, const int32_t* cu,
                                const int32_t* plen, const int32_t* bt, int bt_stride, int batch,
                                int hq, int total_q, int max_q_len, float scale, void* plan_ws,
                                hipStream_t s) {
  // the kernel takes the code pools where it takes the 16-bit ones (block_stride in bytes)
  const kvb_pool view{p.k, p.v, p.block_stride, p.num_blocks, kBlock, p.num_kv_heads, p.head_dim, dtype};
  const PfCascade none{nullptr, 0, 0, 0, 1, nullptr, nullptr, 0};
  const PfQuant qz{p.v_scale, p.k_scale};
  return dispatch_prefill(view, [&](auto t, auto d) {
    if (bits == 4)
      return launch_prefill_t<decltype(t), decltype(d)::value, kModePrefill, 4>(
          view, q, kn, vn, out, cu, plen, bt, bt_stride, batch, hq, total_q, max_q_len, scale, none,
          (int32_t*)plan_ws, s, nullptr, qz);
    return launch_prefill_t<decltype(t), decltype(d)::value, kModePrefill, 8>(
        view, q, kn, vn, out, cu, plen, bt, bt_stride, batch, hq, total_q, max_q_len, scale, none,
        (int32_t*)plan_ws, s, nullptr, qz);
  });
}

hipError_t launch_prefill_pooled(const kvb_pool& p, const void* q, void* out, const int32_t* cu,
                                 const int32_t* plen, const int32_t* bt, int bt_stride, int batch,
                                 int hq, int total_q, int max_q_len, float scale, hipStream_t s) {
  const PfCascade none{nullptr, 0, 0, 0, 1, nullptr, nullptr, 0};
  return dispatch_prefill(p, [&](auto t, auto d) {
    return launch_prefill_t<decltype(t), decltype(d)::value, kModePooled>(
        p, q, nullptr, nullptr, out, cu, plen, bt, bt_stride, batch, hq, total_q, max_q_len, scale,
        none, nullptr, s);
  });
}

void cascade_plan(int batch, int hkv, int hq, int shared_len, int* nks, int* ks_tiles) {
  const int n_tiles = (shared_len + kKT - 1) / kKT;
  if (n_tiles <= 0) { *nks = 0; *ks_tiles = 0; return; }
  const long long units = (long long)hkv * (((long long)batch * (hq / hkv) + kBM - 1) / kBM);
  // about one work-group per CU, at least two tiles each (both key parts busy)
  long long ns = (device_cu_count() + units - 1) / units;
  if (ns > n_tiles) ns = n_tiles;
  if (ns < 1) ns = 1;
  int kt = (int)((n_tiles + ns - 1) / ns);
  if (kt < 2) kt = 2;
  *ks_tiles = kt;
  *nks = (n_tiles + kt - 1) / kt;
}

hipError_t launch_cascade_shared(const kvb_pool& p, const void* q, const int32_t* ctx, int max_ctx,
                                 const int32_t* shared_blocks, int shared_len, int batch, int hq,
                                 float scale, int nks, int ks_tiles, float* ws_o, float* ws_ml,
                                 int ws_slots, hipStream_t s) {
  if (nks <= 0 || batch <= 0) return hipSuccess;
  const PfCascade cas{ctx, max_ctx, shared_len, ks_tiles, nks, ws_o, ws_ml, ws_slots};
  const int nsb = (shared_len + kBlock - 1) / kBlock;
  return dispatch_prefill(p, [&](auto t, auto d) {
    return launch_prefill_t<decltype(t), decltype(d)::value, kModeCascade>(p, q, nullptr, nullptr, nullptr, nullptr,
                                                             nullptr, shared_blocks, nsb, 1, hq, batch,
                                                             batch, scale, cas, nullptr, s);
  });
}

}  // namespace kvb
