// Paged decode with an even share of the batch's blocks per wave (the plain, 8-bit and
// 4-bit pools).
//
// The computation is the split decode's (kvboost 0.6.0, "CPU paged attention": the
// one-query case of the chunk attention; kvstream 0.1.0, "Request lifecycle" step 2), with
// another division of the work.  One work-group per (sequence, split) makes the
// work-groups as uneven as the contexts: on a batch of ragged contexts the last ones
// start late and run alone, so the HBM stream thins out long before the kernel ends.
// Here:
//  * The blocks of the whole batch form one list, ordered (KV head, head chunk, sequence,
//    block); a unit is one (KV head, head chunk, sequence).  The list is cut into ranges
//    of S blocks, one per wave, and the grid is sized to be resident at once (one
//    work-group of eight waves per CU), so every wave starts at once and all of them
//    have about the same bytes to read.  Consecutive waves take consecutive ranges and
//    the work-group -> XCD mapping keeps each XCD on a contiguous part of the list (a few
//    KV heads), so blocks shared between sequences are re-read from that XCD's L2.
//  * A wave streams through its range without a break at unit boundaries: its K/V loads
//    run one step (two blocks) ahead across them, and the queries of the next unit are
//    fetched as soon as the current unit's last scores are taken.  A step never mixes two
//    units.  Blocks after the first 64 of a context are read with the streaming
//    (non-temporal) policy, so that blocks shared between requests, which sit at the
//    start of their sequences, stay in L2 for the other sequences' waves.
//  * At the end of each unit inside its range a wave writes either the normalised output
//    (the range holds the whole unit) or a partial record (unnormalised output, running
//    max, sum); decode_stream_merge combines the records of a unit by log-sum-exp.  The
//    record of wave w for unit u is number w + u: the units a wave meets never come
//    before those of the wave ahead of it, so w + u never repeats, and a unit's records
//    are consecutive.
//  * The step itself (K/V staged through a per-wave LDS slot with 1 KiB contiguous
//    loads, S^T = K Q^T and O^T += V^T P^T on 16x16x32 MFMA, lazily rescaled exp2
//    softmax) is the split decode's.  (K read straight into MFMA operand registers needs
//    64-byte pieces of 16 rows per load instruction; measured on MI355X it is slower than
//    the contiguous loads plus the LDS round trip.)
#include "decode_common.h"
#include "kvb_launch.h"

namespace kvb {

namespace {

// One work-group of eight waves per CU: waves of two work-groups on one CU do not share
// the memory pipeline evenly (the older work-group's waves win its arbitration, and the
// younger one finishes its equal share long after, with half the loads in flight).
constexpr int kStrWaves = 8;
constexpr int kStrThreads = 64 * kStrWaves;
constexpr int kStrMaxBatch = 1024;   // block-count prefix sums held in LDS
constexpr int kStrMaxSpan = 64;      // blocks per wave (a pair range of two: two table entries per lane)
constexpr int kStrMinSpan = 16;      // shorter ranges would add partials for little gain
constexpr int kStrKeepBlocks = 64;   // blocks of a context read with the normal policy

struct DecStream {
  int batch, hq, hkv, nchunks, nhc;   // nhc: query heads per unit, min(G, 16)
  int max_ctx, bt_stride;
  int span;                           // blocks per wave range; 0: balanced
  int waves;                          // waves in the grid
  int resident;                       // waves the device holds at once
  int32_t* hdr;                       // [0] = S, [1] = blocks per (KV head, chunk), [2 + b] = prefix sums
  float* ws_o;                        // records x nhc x D
  float* ws_ml;                       // records x nhc x 2
};

}  // namespace

int64_t stream_hdr_bytes(int batch) { return ((int64_t)(batch + 3) * 4 + 255) / 256 * 256; }
// (max, sum) pairs of the records, rounded up so that the partial outputs after them
// start 256-byte aligned
static int64_t stream_ml_bytes(int64_t records, int nhc) { return (records * nhc * 8 + 255) / 256 * 256; }

// One step's loads: per block, the K and V rows of one KV head in 16-byte chunks (16-bit
// pool: D/32 chunks per lane; codes: 128/QB per chunk), and the V scales of the code
// pools.  Over a bf16 pool the V scales go into the probabilities of the PV product
// (kScaleP: the scales of the four key rows whose probabilities the lane holds); over an
// fp16 pool the V codes are scaled while staged (the scale of each chunk's key row),
// since a probability (up to 2^8 under the lazy rescale) times a V scale (up to
// 65504/127) can leave the fp16 range, while code * scale cannot.
template <typename T, int D, int QB> struct StrStep {
  static constexpr int VCH = QB ? (D * QB / 8 + 63) / 64 : D / 32;
  static constexpr bool kScaleP = QB != 0 && std::is_same<T, BF16>::value;
  uint4 k[2][VCH];
  uint4 v[2][VCH];
  f32x4 vsp[kScaleP ? 2 : 1];
  float vsr[2][QB != 0 && !kScaleP ? VCH : 1];
};

template <typename T, int D, int QB>
__global__ void __launch_bounds__(kStrThreads, 1)
decode_stream_kernel(const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
                     int64_t block_stride, int num_blocks, const uint16_t* __restrict__ q,
                     uint16_t* __restrict__ out, const int32_t* __restrict__ ctx_lens,
                     const int32_t* __restrict__ bt, float c_log2, DecStream ds, DecQ8 q8) {
  constexpr bool Q8 = QB != 0;
  using Step = StrStep<T, D, QB>;
  constexpr bool kScaleP = Step::kScaleP;
  constexpr int NKK = D / 32;
  constexpr int NDB = D / 16;
  constexpr int CPR = D / 8;                // 16-byte chunks per 16-bit V row
  constexpr int VCH = Step::VCH;
  constexpr int CH = D * QB / 8;            // code chunks per block (quantised V)
  constexpr int CPRQ = D * QB / 128;        // code chunks per key row
  constexpr int VROW = D + 16;              // V row stride (elements): 8 banks apart per row
  constexpr int KROW = D + 8;               // K row stride (elements): 4 banks apart per row
  constexpr int SLOT = 32 * (VROW + KROW);  // two blocks of V, then of K, per wave

  __shared__ __attribute__((aligned(16))) uint16_t sV[kStrWaves * SLOT];
  __shared__ int s_cum[kStrMaxBatch + 1];
  __shared__ int s_wsum[kStrWaves];
  __shared__ int s_last[kStrWaves];          // unit of each wave's last step (-1: none)

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = uniform(tid >> 6);
  const int c16 = lane & 15, g4 = lane >> 4;
  const int batch = ds.batch;
  const int G = ds.hq / ds.hkv;
  const int cap = min(ds.max_ctx, ds.bt_stride * kBlock);

  // s_cum[b]: blocks of the contexts of sequences 0..b-1 (two sequences per thread)
  static_assert(2 * kStrThreads >= kStrMaxBatch, "one pass over the batch");
  {
    int v[2], sum = 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int b = 2 * tid + i;
      const int n = b < batch ? min(ctx_lens[b], cap) : 0;
      sum += n > 0 ? (n + kBlock - 1) / kBlock : 0;
      v[i] = sum;
    }
    int x = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) s_wsum[w] = x;
    __syncthreads();
    int excl = x - sum;
    for (int ww = 0; ww < w; ++ww) excl += s_wsum[ww];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int b = 2 * tid + i;
      if (b < batch) s_cum[b + 1] = excl + v[i];
    }
    if (tid == 0) s_cum[0] = 0;
    __syncthreads();
  }
  const int Tb = s_cum[batch];                       // blocks per (KV head, head chunk)
  const int64_t total = (int64_t)ds.hkv * ds.nchunks * Tb;
  // S: blocks per wave (two waves per pair range).  Balanced: the list over the waves the
  // device holds at once.  Work-groups per XCD that take ranges (the rest return at once):
  // as few as cover the list, the same number on every XCD; hardware work-group h runs on
  // XCD h % 8, and logical work-group xcd * use + h / 8 keeps each XCD on a contiguous part
  // of the list.
  int S = ds.span;
  if (S <= 0) {
    S = (int)((total + ds.resident - 1) / ds.resident);
    S = max(S, kStrMinSpan);
    S = min((S + 1) & ~1, kStrMaxSpan);
  }
  constexpr int kWavesPerXcdWg = kNumXcd * kStrWaves;
  const int per = gridDim.x / kNumXcd;
  const int use = (int)max((int64_t)1, min((int64_t)per, (total + (int64_t)kWavesPerXcdWg * S - 1) /
                                                           ((int64_t)kWavesPerXcdWg * S)));
  const int R = 2 * S;                               // blocks per pair range
  if (blockIdx.x == 0) {
    for (int i = tid; i <= batch; i += kStrThreads) ds.hdr[2 + i] = s_cum[i];
    if (tid == 0) {
      ds.hdr[0] = R;
      ds.hdr[1] = Tb;
    }
  }
  const int xcd = blockIdx.x % kNumXcd, j = blockIdx.x / kNumXcd;
  if (j >= use) return;                              // the whole work-group
  const int lid = xcd * use + j;
  // Waves w and w + 4 share pair range pp: the first takes the first half of its steps,
  // the second the rest; the unit the two halves share is combined in LDS at the end, so
  // the pair writes one output or record per unit.
  const int side = w / (kStrWaves / 2);
  const int pp = lid * (kStrWaves / 2) + (w % (kStrWaves / 2));
  const int64_t p0 = (int64_t)pp * R;
  const int len = (int)max((int64_t)0, min((int64_t)R, total - p0));

  // The pair range's block table: lane i describes blocks p0 + i and p0 + 64 + i of the list
  // (unit, block index in the context, physical block or -1 outside the pool, valid key
  // rows).
  int t_u[2] = {-1, -1}, t_blk[2] = {0, 0}, t_pb[2] = {-1, -1}, t_rows[2] = {0, 0};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (lane + 64 * h >= len) continue;
    const int64_t p = p0 + lane + 64 * h;
    const int group = (int)(p / Tb);
    const int r = (int)(p - (int64_t)group * Tb);
    int lo = 0, hi = batch;                          // the b with s_cum[b] <= r < s_cum[b + 1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_cum[mid] <= r) lo = mid;
      else hi = mid;
    }
    const int blk = r - s_cum[lo];
    const int n = min(ctx_lens[lo], cap);
    const int pb = bt[(int64_t)lo * ds.bt_stride + blk];
    t_u[h] = group * batch + lo;
    t_blk[h] = blk;
    t_pb[h] = (pb >= 0 && pb < num_blocks) ? pb : -1;
    t_rows[h] = t_pb[h] >= 0 ? min(kBlock, n - blk * kBlock) : 0;
  }
  auto rl = [](int x, int i) { return __builtin_amdgcn_readlane(x, i); };
  // entry i (wave-uniform, 0 <= i < 128) of a table
  auto tab = [&](const int (&x)[2], int i) -> int {
    const int a = rl(x[0], i & 63), b = rl(x[1], i & 63);
    return i < 64 ? a : b;
  };

  uint16_t* slot = sV + w * SLOT;           // V rows 0..31 of the current step
  uint16_t* kslot = slot + 32 * VROW;       // K rows 0..31
  constexpr bool kWholeRows = 64 % CPR == 0;
  const int v_st = (lane / CPR) * VROW + (lane % CPR) * 8;
  const int k_st = (lane / CPR) * KROW + (lane % CPR) * 8;

  // A step: blocks at offsets i and i + 1 of the range (n = 2) when both belong to unit
  // u; n = 0: no step.
  struct Desc {
    int i, n, u, rows0, rows1;
  };
  auto desc_at = [&](int i) -> Desc {
    Desc d;
    d.i = i;
    d.u = tab(t_u, i);
    d.n = (i + 1 < len && tab(t_u, i + 1) == d.u) ? 2 : 1;
    d.rows0 = tab(t_rows, i);
    d.rows1 = d.n == 2 ? tab(t_rows, i + 1) : 0;
    return d;
  };
  auto desc_after = [&](const Desc& d) -> Desc {
    if (d.n == 0 || d.i + d.n >= len) return Desc{0, 0, 0, 0, 0};
    return desc_at(d.i + d.n);
  };

  // Both blocks of a step through buffer resources sized to their valid rows: rows past
  // the context and blocks outside the pool read as zero and cost no memory traffic.
  auto load = [&](const Desc& d, Step& R) __attribute__((always_inline)) {
    const int kvh = (d.u / batch) / ds.nchunks;
    const bool nt = !Q8 && tab(t_blk, d.i) >= kStrKeepBlocks;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int pb = hb < d.n ? tab(t_pb, d.i + hb) : -1;
      const int rows = hb == 0 ? d.rows0 : d.rows1;
      if constexpr (Q8) {
        // codes: D*QB/8 bytes per key row; block_stride counts bytes
        const int64_t qoff = (int64_t)(pb >= 0 ? pb : 0) * block_stride + (int64_t)kvh * kBlock * D * QB / 8;
        const uint8_t* kb = reinterpret_cast<const uint8_t*>(kp) + qoff;
        const uint8_t* vb = reinterpret_cast<const uint8_t*>(vp) + qoff;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, (uint32_t)(rows * D * QB / 8));
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, (uint32_t)(rows * D * QB / 8));
#pragma unroll
        for (int j = 0; j < VCH; ++j) {
          R.k[hb][j] = buf_load16(rk, (uint32_t)(j * 64 + lane) * 16);
          R.v[hb][j] = buf_load16(rv, (uint32_t)(j * 64 + lane) * 16);
        }
        // V scales (rows past the context read as 0): of key rows 4*g4 .. 4*g4+3, or of
        // the key row of each chunk
        const float* sb = q8.v_scale + ((int64_t)(pb >= 0 ? pb : 0) * ds.hkv + kvh) * kBlock;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(sb, (uint32_t)(rows * 4));
        if constexpr (kScaleP) {
          R.vsp[hb] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * g4, 0, 0));
        } else {
#pragma unroll
          for (int j = 0; j < VCH; ++j)
            R.vsr[hb][j] = __builtin_bit_cast(
                float, __builtin_amdgcn_raw_buffer_load_b32(rs, (j * 64 + lane) / CPRQ * 4, 0, 0));
        }
      } else {
        const int64_t off = (int64_t)(pb >= 0 ? pb : 0) * block_stride + (int64_t)kvh * kBlock * D;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(kp + off, (uint32_t)(rows * D * 2));
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vp + off, (uint32_t)(rows * D * 2));
        if (nt) {
#pragma unroll
          for (int j = 0; j < VCH; ++j) {
            R.k[hb][j] = buf_load16_nt(rk, (uint32_t)(8 * (j * 64 + lane)) * 2);
            R.v[hb][j] = buf_load16_nt(rv, (uint32_t)(8 * (j * 64 + lane)) * 2);
          }
        } else {
#pragma unroll
          for (int j = 0; j < VCH; ++j) {
            R.k[hb][j] = buf_load16(rk, (uint32_t)(8 * (j * 64 + lane)) * 2);
            R.v[hb][j] = buf_load16(rv, (uint32_t)(8 * (j * 64 + lane)) * 2);
          }
        }
      }
    }
  };

  // Queries of unit u as the B operand (column c16 = head chunk*16 + c16 of the KV group,
  // d chunk 4*kk + g4).  At a unit change they are fetched as soon as the last scores of
  // the previous unit have been taken (before the loads of the step after next), and the
  // 8-bit pool's per-channel K scales of the unit's KV head, fetched with them, are
  // folded in just before the unit's first scores.
  s16x8 qb[NKK];
  f32x4 ksc[Q8 ? 2 * NKK : 1];
  auto fetch_q = [&](int u) __attribute__((always_inline)) {
    const int group = u / batch, b = u - group * batch;
    const int kvh = group / ds.nchunks, chunk = group - kvh * ds.nchunks;
    const int hl = chunk * kDecHeads + c16;
    // columns past the KV group repeat its last head (finite scores in columns that are
    // never written out), so the loads need no select that would wait for them here
    const int64_t qrow = (int64_t)b * ds.hq + kvh * G + min(hl, G - 1);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
      qb[kk] = *reinterpret_cast<const s16x8*>(q + qrow * D + 8 * (4 * kk + g4));
    if constexpr (Q8) {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const float* ks = q8.k_scale + kvh * D + 8 * (4 * kk + g4);
        ksc[2 * kk] = *reinterpret_cast<const f32x4*>(ks);
        ksc[2 * kk + 1] = *reinterpret_cast<const f32x4*>(ks + 4);
      }
    }
  };
  // q . k = sum_e (q_e s_e) code_e
  auto fold_q = [&]() __attribute__((always_inline)) {
    if constexpr (Q8) {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const f32x4 a = ksc[2 * kk], c = ksc[2 * kk + 1];
        const float sc[8] = {a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
        uint32_t wv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          wv[i] = pack2<T>(T::to_f32((uint16_t)qb[kk][2 * i]) * sc[2 * i],
                           T::to_f32((uint16_t)qb[kk][2 * i + 1]) * sc[2 * i + 1]);
        qb[kk] = __builtin_bit_cast(s16x8, make_uint4(wv[0], wv[1], wv[2], wv[3]));
      }
    }
  };

  f32x4 o[NDB];
  float m_run, l_run;
  auto reset = [&]() {
#pragma unroll
    for (int i = 0; i < NDB; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run = kNegBig;
    l_run = 0.f;
  };

  // K and V of a step into this wave's LDS slot in their natural [key][d] layout (codes
  // widened to the 16-bit type: K codes exactly, V codes exactly over a bf16 pool and
  // times their key's V scale over an fp16 pool); rows past the context arrive as zeros.
  auto stage = [&](const Step& R) __attribute__((always_inline)) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int j = 0; j < VCH; ++j) {
        if constexpr (Q8) {
          const int c = j * 64 + lane;
          if (c >= CH) continue;                    // chunks past the block (some lanes)
          const int row = c / CPRQ, col = (c - row * CPRQ) * (128 / QB);
          uint16_t* vrow = slot + (hb * 16 + row) * VROW + col;
          uint16_t* krow = kslot + (hb * 16 + row) * KROW + col;
          if constexpr (QB == 8) {
            uint4 lo, hi;
            codes_to<T>(R.v[hb][j], kScaleP ? 1.f : R.vsr[hb][kScaleP ? 0 : j], lo, hi);
            *reinterpret_cast<uint4*>(vrow) = lo;
            *reinterpret_cast<uint4*>(vrow + 8) = hi;
            codes_to<T>(R.k[hb][j], 1.f, lo, hi);
            *reinterpret_cast<uint4*>(krow) = lo;
            *reinterpret_cast<uint4*>(krow + 8) = hi;
          } else {
            uint4 o4[4];
            nibbles_to<T>(R.v[hb][j], kScaleP ? 1.f : R.vsr[hb][kScaleP ? 0 : j], o4);
#pragma unroll
            for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(vrow + 8 * i) = o4[i];
            nibbles_to<T>(R.k[hb][j], 1.f, o4);
#pragma unroll
            for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(krow + 8 * i) = o4[i];
          }
        } else {
          int vo, ko;
          if constexpr (kWholeRows) {
            vo = v_st + (hb * 16 + j * (64 / CPR)) * VROW;
            ko = k_st + (hb * 16 + j * (64 / CPR)) * KROW;
          } else {
            const int c = j * 64 + lane;
            const int row = c / CPR;
            vo = (hb * 16 + row) * VROW + (c - row * CPR) * 8;
            ko = (hb * 16 + row) * KROW + (c - row * CPR) * 8;
          }
          *reinterpret_cast<uint4*>(slot + vo) = R.v[hb][j];
          *reinterpret_cast<uint4*>(kslot + ko) = R.k[hb][j];
        }
      }
  };

  // S^T = K Q^T per block (A operand: key row c16 from the LDS slot).
  auto scores = [&](const Step& R, f32x4 (&s)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      s[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const s16x8 a = *reinterpret_cast<const s16x8*>(kslot + (hb * 16 + c16) * KROW + 8 * (4 * kk + g4));
        s[hb] = T::mfma16(a, qb[kk], s[hb]);
      }
    }
  };

  // Softmax update and O^T += V^T P^T for the step whose V is in the LDS slot (rows0,
  // rows1: valid keys of its two blocks).  Code pools over bf16 (kScaleP): the slot holds
  // the V codes, and the V scale of each key multiplies its probability in the PV operand
  // instead (sum_k p_k s_k c_k: one multiply per probability instead of one per value);
  // the row sum takes the probabilities themselves.
  auto update = [&](const f32x4 (&s)[2], int rows0, int rows1, const f32x4 (&vs)[kScaleP ? 2 : 1])
      __attribute__((always_inline)) {
    const int rows[2] = {rows0, rows1};
    float t[8];
    float mx = -INFINITY;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const bool ok = 4 * g4 + rr < rows[hb];
        const float tv = ok ? s[hb][rr] * c_log2 : -INFINITY;
        t[hb * 4 + rr] = tv;
        mx = fmaxf(mx, tv);
      }
    }
    mx = halves_max(fmaxf(mx, xor16(mx)));
    if (__any(mx > m_run + kRescaleThreshold)) {
      keep_branch();
      const float mn = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - mn);
      m_run = mn;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) o[db][rr] *= alpha;
    }
    uint32_t pw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p0v = fast_exp2(t[2 * e] - m_run);
      const float p1v = fast_exp2(t[2 * e + 1] - m_run);
      l_run += p0v + p1v;
      if constexpr (kScaleP)
        pw[e] = pack2<T>(p0v * vs[e >> 1][2 * (e & 1)], p1v * vs[e >> 1][2 * (e & 1) + 1]);
      else
        pw[e] = pack2<T>(p0v, p1v);
    }
    const s16x8 pb8 = __builtin_bit_cast(s16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
    __builtin_amdgcn_wave_barrier();
    // A operand rows d = 16*db + c16, keys 4*g4.. of block 0 then block 1
    const int src_row = 4 * g4 + (c16 >> 2);
    const int src_col = 4 * (c16 & 3);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const s16x4 lo = lds_read_tr16(slot + src_row * VROW + 16 * db + src_col);
      const s16x4 hi = lds_read_tr16(slot + (16 + src_row) * VROW + 16 * db + src_col);
      const s16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      o[db] = T::mfma16(a, pb8, o[db]);
    }
    __builtin_amdgcn_wave_barrier();
  };

  // End of unit u (all of its blocks in the pair range done): the normalised output when
  // the pair range holds all of the unit's blocks, else the partial record pp + u.  Lane
  // (c16, g4) holds o[db][rr] = O[head c16][d = 16*db + 4*g4 + rr].
  auto finish_unit = [&](int u) __attribute__((always_inline)) {
    const float lsum = halves_sum(l_run + xor16(l_run));
    const int group = u / batch, b = u - group * batch;
    const int kvh = group / ds.nchunks, chunk = group - kvh * ds.nchunks;
    const int hl = chunk * kDecHeads + c16;
    const int64_t start = (int64_t)group * Tb + s_cum[b];
    const int64_t end = (int64_t)group * Tb + s_cum[b + 1];
    const bool whole = start >= p0 && end <= p0 + len;
    if (hl < G) {
      if (whole) {
        const int64_t row = (int64_t)b * ds.hq + kvh * G + hl;
        const float inv = 1.f / lsum;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const uint2 v2 = make_uint2(pack2<T>(o[db][0] * inv, o[db][1] * inv),
                                      pack2<T>(o[db][2] * inv, o[db][3] * inv));
          *reinterpret_cast<uint2*>(out + row * D + 16 * db + 4 * g4) = v2;
        }
      } else {
        const int64_t rec = ((int64_t)pp + u) * ds.nhc + c16;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          *reinterpret_cast<f32x4*>(ds.ws_o + rec * D + 16 * db + 4 * g4) = o[db];
        if (g4 == 0) *reinterpret_cast<float2*>(ds.ws_ml + rec * 2) = make_float2(m_run, lsum);
      }
    }
    reset();
  };

  // Steps of the pair range: each unit piece of m blocks takes ceil(m/2) steps.  Position
  // p < len starts a step when it starts a piece or sits an even number of blocks into
  // one; step k starts at the k-th such position.
  uint64_t st0, st1;
  int nsteps;
  {
    // the shuffles run in every lane (a cross-lane read inside a lane-dependent branch
    // would read inactive lanes), then lane 0 of the second half takes position 63
    const int prev0 = __shfl_up(t_u[0], 1, 64);
    const int sh1 = __shfl_up(t_u[1], 1, 64);
    const int last_first = rl(t_u[0], 63);
    const int prev1 = lane == 0 ? last_first : sh1;
    const uint64_t s0 = __ballot(lane < len && (lane == 0 || prev0 != t_u[0]));
    const uint64_t s1 = __ballot(lane + 64 < len && prev1 != t_u[1]);
    const uint64_t upto = lane == 63 ? ~0ull : ((2ull << lane) - 1);
    // the last piece start at or before p (position 0 always starts one)
    const int last0 = 63 - (int)__builtin_clzll((s0 & upto) | 1ull);
    const int last1 = (s1 & upto) ? 64 + 63 - (int)__builtin_clzll(s1 & upto)
                                  : 63 - (int)__builtin_clzll(s0 | 1ull);
    st0 = __ballot(lane < len && ((lane - last0) & 1) == 0);
    st1 = __ballot(lane + 64 < len && ((lane + 64 - last1) & 1) == 0);
    nsteps = __builtin_popcountll(st0) + __builtin_popcountll(st1);
  }
  const uint64_t below = (1ull << lane) - 1;
  const int rank0 = __builtin_popcountll(st0 & below);
  const int rank1 = __builtin_popcountll(st0) + __builtin_popcountll(st1 & below);
  // The side's next step, or an absent one (n = 0) after its last: steps
  // [0, ceil(nsteps/2)) in order for the first side, the rest from the last one down for
  // the second, so that the unit the two share is the last one of each.  (Handing the steps
  // out one at a time through an LDS counter balances the pair at run time, but the
  // partials then depend on timing and the rounding of the result changes from run to
  // run; measured on MI355X it is only about 1% faster.)
  const int half_steps = (nsteps + 1) / 2;
  int taken = 0;
  auto claim = [&]() -> Desc {
    const int k = side == 0 ? taken : nsteps - 1 - taken;
    if (side == 0 ? k >= half_steps : k < half_steps) return Desc{0, 0, 0, 0, 0};
    ++taken;
    const uint64_t m0 = __ballot(((st0 >> lane) & 1) && rank0 == k);
    const uint64_t m1 = __ballot(((st1 >> lane) & 1) && rank1 == k);
    return desc_at(m0 ? (int)__builtin_ctzll(m0) : 64 + (int)__builtin_ctzll(m1));
  };

  Desc cur = claim();
  Desc nx = cur.n ? claim() : Desc{0, 0, 0, 0, 0};
  if (cur.n) fetch_q(cur.u);
  bool fresh = cur.n != 0;      // qb holds a new unit's raw queries (8-bit: fold pending)
  int last_u = cur.n ? cur.u : -1;
  reset();
  // X holds the current step, Y the next one (in flight while X is computed); X then takes
  // the loads of the step after Y.  Loads are issued for absent steps too (n = 0:
  // zero-size resources, no memory traffic), so a buffer's old contents are never kept
  // alive beside its new ones.  The two buffers are used in turn, so no register copy
  // waits on loads in flight.  (A second step in flight, issued before the softmax and PV
  // of the current one, measured no faster.)
  Step A, B;
  load(cur, A);
  load(nx, B);
  auto half = [&](Step& X) __attribute__((always_inline)) {
    stage(X);
    __builtin_amdgcn_wave_barrier();
    if (fresh) {
      fold_q();
      fresh = false;
    }
    f32x4 s[2];
    scores(X, s);
    const bool change = nx.n != 0 && nx.u != cur.u;
    if (change) {
      fetch_q(nx.u);
      fresh = true;
    }
    const Desc n2 = nx.n ? claim() : Desc{0, 0, 0, 0, 0};
    f32x4 vs[kScaleP ? 2 : 1];
#pragma unroll
    for (int i = 0; i < (kScaleP ? 2 : 1); ++i) vs[i] = X.vsp[i];
    load(n2, X);
    update(s, cur.rows0, cur.rows1, vs);
    if (change) finish_unit(cur.u);
    if (nx.n) last_u = nx.u;
    cur = nx;
    nx = n2;
  };
  // An absent step changes nothing (no keys), so the loop runs both halves every time
  // and has no exit between them; such an exit would join the loop head with A loaded
  // last and make the wait before A's staging cover B's loads too.
  do {
    half(A);
    half(B);
  } while (cur.n != 0);

  // The last unit of each side may have steps on the other side too: the first side
  // leaves its partial (per lane: o, running max, sum) in its LDS slot and the second side
  // folds it into its own before writing the unit.
  float* part = reinterpret_cast<float*>(sV + w * SLOT);
  if (lane == 0) s_last[w] = last_u;
  if (side == 0 && last_u >= 0) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) part[(db * 4 + rr) * 64 + lane] = o[db][rr];
    part[NDB * 4 * 64 + lane] = m_run;
    part[(NDB * 4 + 1) * 64 + lane] = l_run;
  }
  __syncthreads();
  const int partner_last = s_last[w ^ (kStrWaves / 2)];
  if (last_u >= 0) {
    if (side == 1 && partner_last == last_u) {
      const float* fp = reinterpret_cast<const float*>(sV + (w ^ (kStrWaves / 2)) * SLOT);
      const float mf = fp[NDB * 4 * 64 + lane];
      const float M = fmaxf(m_run, mf);
      const float ab = fast_exp2(m_run - M), af = fast_exp2(mf - M);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) o[db][rr] = o[db][rr] * ab + fp[(db * 4 + rr) * 64 + lane] * af;
      l_run = l_run * ab + fp[(NDB * 4 + 1) * 64 + lane] * af;
      m_run = M;
    }
    if (!(side == 0 && partner_last == last_u)) finish_unit(last_u);
  }
}

// One wave per (sequence, query head) row.  The row's unit covers blocks [start, end) of
// the list; its records are w + u for the waves w = start/S .. (end-1)/S.  A unit inside
// one wave's range was written directly; an empty context gives a zero row.
template <typename T, int D>
__global__ void __launch_bounds__(64 * kMergeRows)
decode_stream_merge_kernel(const float* __restrict__ ws_o, const float* __restrict__ ws_ml,
                           const int32_t* __restrict__ hdr, uint16_t* __restrict__ out, int batch,
                           int hq, int hkv, int nchunks, int nhc) {
  constexpr int NV = (D + 63) / 64;    // d values per lane: d = lane + 64 * i
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kMergeRows + uniform(threadIdx.x >> 6);
  if (row >= batch * hq) return;
  const int b = row / hq, h = row - b * hq;
  const int G = hq / hkv, kvh = h / G, hl = h - kvh * G;
  const int chunk = hl / kDecHeads, hc = hl - chunk * kDecHeads;
  const int S = hdr[0], Tb = hdr[1], c0 = hdr[2 + b], c1 = hdr[3 + b];
  if (c1 <= c0) {
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (lane + 64 * i < D) out[(int64_t)row * D + lane + 64 * i] = 0;
    return;
  }
  const int group = kvh * nchunks + chunk;
  const int64_t u = (int64_t)group * batch + b;
  const int64_t start = (int64_t)group * Tb + c0, end = start + (c1 - c0);
  const int64_t first = start / S, last = (end - 1) / S;
  if (first == last) return;
  const int ns = (int)(last - first + 1);
  const int64_t rec0 = first + u;
  auto rec_of = [&](int s) -> int64_t { return (rec0 + min(s, ns - 1)) * nhc + hc; };
  float2 mine;                         // (max, sum) of record s0 + lane % 8
  // lanes past the head dimension re-read its last element (never written out), so the
  // loads need no branch
  float v[kMergeBatch][NV];
  auto load = [&](int s0) {
    mine = *reinterpret_cast<const float2*>(ws_ml + 2 * rec_of(s0 + (lane & (kMergeBatch - 1))));
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const float* po = ws_o + rec_of(s0 + j) * D;
#pragma unroll
      for (int i = 0; i < NV; ++i) v[j][i] = po[min(lane + 64 * i, D - 1)];
    }
  };
  float M = kNegBig, L = 0.f;
  float o[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) o[i] = 0.f;
  load(0);
  for (int s0 = 0;;) {
    float mj[kMergeBatch], lj[kMergeBatch];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      mj[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine.x), j));
      lj[j] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine.y), j));
    }
    float Mb = M;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) Mb = s0 + j < ns ? fmaxf(Mb, mj[j]) : Mb;
    const float a = fast_exp2(M - Mb);
    L *= a;
#pragma unroll
    for (int i = 0; i < NV; ++i) o[i] *= a;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const bool ok = s0 + j < ns;
      const float sc = ok ? fast_exp2(mj[j] - Mb) : 0.f;
      L = fmaf(sc, ok ? lj[j] : 0.f, L);
#pragma unroll
      for (int i = 0; i < NV; ++i) o[i] = fmaf(sc, ok ? v[j][i] : 0.f, o[i]);
    }
    M = Mb;
    s0 += kMergeBatch;
    if (s0 >= ns) break;
    load(s0);
  }
  const float inv = 1.f / L;
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (lane + 64 * i < D) out[(int64_t)row * D + lane + 64 * i] = T::from_f32(o[i] * inv);
}

StreamPlan decode_stream_plan(int batch, int hkv, int hq, int d, int max_ctx, int split_blocks) {
  StreamPlan sp{};
  const int G = hq / hkv;
  const int nchunks = (G + kDecHeads - 1) / kDecHeads;
  const int nhc = G < kDecHeads ? G : kDecHeads;
  const int64_t max_blocks = max_ctx > 0 ? ((int64_t)max_ctx + kBlock - 1) / kBlock : 0;
  const int64_t tmax = (int64_t)hkv * nchunks * batch * max_blocks;
  int64_t waves;
  if (split_blocks > 0) {
    sp.span = split_blocks < kStrMaxSpan ? split_blocks : kStrMaxSpan;
    waves = (tmax + sp.span - 1) / sp.span;
  } else {
    sp.span = 0;
    waves = (tmax + kStrMaxSpan - 1) / kStrMaxSpan;
  }
  const int64_t resident = (int64_t)kStrWaves * device_cu_count();
  if (split_blocks <= 0 && waves < resident) waves = resident;
  // whole work-groups on every XCD
  const int64_t unit = (int64_t)kStrWaves * kNumXcd;
  if (waves < 1) waves = 1;
  waves = (waves + unit - 1) / unit * unit;
  sp.waves = waves;
  sp.resident = resident;
  sp.records = waves + (int64_t)hkv * nchunks * batch;
  sp.bytes = stream_hdr_bytes(batch) + stream_ml_bytes(sp.records, nhc) + sp.records * nhc * d * 4;
  return sp;
}

bool decode_use_stream(int batch) { return batch <= kStrMaxBatch; }

template <typename T, int D, int QB>
static hipError_t launch_stream_t(const kvb_pool& p, const void* q, void* out, const int32_t* ctx,
                                  const int32_t* bt, int bt_stride, int batch, int hq, int max_ctx,
                                  const StreamPlan& sp, float scale, void* ws, hipStream_t s,
                                  DecQ8 q8) {
  const int G = hq / p.num_kv_heads;
  DecStream ds{};
  ds.batch = batch;
  ds.hq = hq;
  ds.hkv = p.num_kv_heads;
  ds.nchunks = (G + kDecHeads - 1) / kDecHeads;
  ds.nhc = G < kDecHeads ? G : kDecHeads;
  ds.max_ctx = max_ctx;
  ds.bt_stride = bt_stride;
  ds.span = sp.span;
  ds.waves = (int)sp.waves;
  ds.resident = (int)sp.resident;
  ds.hdr = (int32_t*)ws;
  ds.ws_ml = (float*)((char*)ws + stream_hdr_bytes(batch));
  ds.ws_o = (float*)((char*)ds.ws_ml + stream_ml_bytes(sp.records, ds.nhc));
  const float c = scale * 1.4426950408889634f;
  hipLaunchKernelGGL((decode_stream_kernel<T, D, QB>), dim3((unsigned)(sp.waves / kStrWaves)),
                     dim3(kStrThreads), 0, s, (const uint16_t*)p.k, (const uint16_t*)p.v,
                     p.block_stride, p.num_blocks, (const uint16_t*)q, (uint16_t*)out, ctx, bt, c,
                     ds, q8);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = batch * hq;
  hipLaunchKernelGGL((decode_stream_merge_kernel<T, D>), dim3((unsigned)((rows + kMergeRows - 1) / kMergeRows)),
                     dim3(64 * kMergeRows), 0, s, ds.ws_o, ds.ws_ml, ds.hdr, (uint16_t*)out, batch,
                     hq, ds.hkv, ds.nchunks, ds.nhc);
  return hipGetLastError();
}

hipError_t launch_decode_stream(const kvb_pool& p, int bits, const DecScales& sc, const void* q,
                                void* out, const int32_t* ctx, const int32_t* bt, int bt_stride,
                                int batch, int hq, int max_ctx, const StreamPlan& sp, float scale,
                                void* ws, hipStream_t s) {
  const bool bf = p.dtype == KVB_BF16;
  const DecQ8 q8{sc.k_scale, sc.v_scale};
#define KVB_S(TT, DD, QQ) launch_stream_t<TT, DD, QQ>(p, q, out, ctx, bt, bt_stride, batch, hq, max_ctx, \
    sp, scale, ws, s, q8)
#define KVB_SB(DD) (bits == 4 ? (bf ? KVB_S(BF16, DD, 4) : KVB_S(F16, DD, 4))    \
                  : bits == 8 ? (bf ? KVB_S(BF16, DD, 8) : KVB_S(F16, DD, 8))    \
                              : (bf ? KVB_S(BF16, DD, 0) : KVB_S(F16, DD, 0)))
  switch (p.head_dim) {
    case 64:  return KVB_SB(64);
    case 96:  return KVB_SB(96);
    default:  return KVB_SB(128);
  }
#undef KVB_SB
#undef KVB_S
}

}  // namespace kvb
