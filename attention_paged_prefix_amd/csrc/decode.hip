// Paged decode: one query per sequence against its whole context in the block pool,
// split over groups of blocks and merged by log-sum-exp.
//
// The decode step is the one-query case of the chunk attention (kvboost 0.6.0, "CPU
// paged attention": only the decode loop changes; kvstream 0.1.0, "Request lifecycle"
// step 2: one slot per generated token, so the current token is already in the pool).
//
// Design (HBM-bound: about G flops per byte of K/V):
//  * One work-group (4 waves) per (sequence, KV head, head chunk of up to GC query
//    heads, split of `split_blocks` blocks).  All GC heads of a KV group read each K/V
//    block once.
//  * A wave consumes one 16-token block per step.  Lane l owns key row l/4 of the block
//    and the 16-byte chunks {l%4 + 4j} of that row: every load instruction of the wave
//    reads 16 rows x 64 contiguous bytes, and the q.k partial sums reduce over the 4
//    lanes of a quad with two DPP moves.
//  * Each lane keeps its own online-softmax state (max, sum, unnormalised output) over
//    the key rows it sees, with lazy rescaling: the reference max only moves when a
//    score exceeds it by more than 2^8 in the exp2 domain, so exponentials stay <= 256
//    and the rescale multiply is rarely taken.  The state of the 64 key slots of the
//    work-group is merged once at the end of the split (the same log-sum-exp identity).
//  * A split covering the whole context writes the normalised output directly; other
//    splits write (output, max, sum) partials that decode_merge combines.
#include "kvb_device.h"
#include "kvb_launch.h"

namespace kvb {

constexpr int kDecWaves = 4;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kMaxSplitBlocks = 256;
constexpr float kRescaleThreshold = 8.0f;   // log2 units
constexpr float kNegBig = -1.0e30f;

template <int D> struct KVRegs {
  static constexpr int NJ = D / 32;         // 16-byte chunks per lane per K (or V) row
  uint4 k[NJ];
  uint4 v[NJ];
};

template <typename T, int D, int GC>
__global__ void __launch_bounds__(kDecThreads)
decode_split_kernel(const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
                    int64_t block_stride, int num_blocks, const uint16_t* __restrict__ q,
                    uint16_t* __restrict__ out, const int32_t* __restrict__ ctx_lens,
                    const int32_t* __restrict__ bt, int bt_stride, int hq, int hkv, int nchunks,
                    int split_blocks, int nsplit, int max_ctx, float c_log2,
                    float* __restrict__ ws_o, float* __restrict__ ws_ml, int padded, int real) {
  constexpr int NJ = D / 32;
  const int lid = xcd_logical_id(blockIdx.x, padded);
  if (lid >= real) return;
  // logical id -> (b, kvh, split, chunk), chunk fastest
  int r = lid;
  const int chunk = r % nchunks; r /= nchunks;
  const int split = r % nsplit; r /= nsplit;
  const int kvh = r % hkv;
  const int b = r / hkv;
  const int G = hq / hkv;
  const int h0 = kvh * G + chunk * GC;
  const int nh = min(GC, G - chunk * GC);

  int n = ctx_lens[b];
  n = min(n, min(max_ctx, bt_stride * kBlock));
  const int tid = threadIdx.x;
  if (n <= 0) {
    if (split == 0) {
      for (int e = tid; e < nh * D; e += kDecThreads)
        out[((int64_t)b * hq + h0 + e / D) * D + (e % D)] = 0;
    }
    return;
  }
  const int nblk = (n + kBlock - 1) / kBlock;
  const int blk_begin = split * split_blocks;
  if (blk_begin >= nblk) return;
  const int blk_end = min(nblk, blk_begin + split_blocks);
  const bool single = nblk <= split_blocks;

  __shared__ int s_bt[kMaxSplitBlocks];
  __shared__ float s_m[kDecWaves][GC];
  __shared__ float s_l[kDecWaves][GC];
  __shared__ float s_acc[kDecWaves][GC][D];

  for (int i = tid; i < blk_end - blk_begin; i += kDecThreads) {
    int pb = bt[(int64_t)b * bt_stride + blk_begin + i];
    s_bt[i] = (pb >= 0 && pb < num_blocks) ? pb : -1;
  }

  const int lane = tid & 63, w = tid >> 6;
  const int ks = lane >> 2;          // key row within a block
  const int qd = lane & 3;           // chunk phase

  // query chunks, packed 16-bit pairs
  uint4 qv[GC][NJ];
#pragma unroll
  for (int h = 0; h < GC; ++h)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if (h < nh)
        qv[h][j] = *reinterpret_cast<const uint4*>(q + ((int64_t)b * hq + h0 + h) * D + 8 * (qd + 4 * j));
      else
        qv[h][j] = make_uint4(0, 0, 0, 0);
    }

  float m[GC], l[GC], acc[GC][NJ * 8];
#pragma unroll
  for (int h = 0; h < GC; ++h) {
    m[h] = kNegBig;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < NJ * 8; ++e) acc[h][e] = 0.f;
  }
  __syncthreads();

  const int64_t head_off = (int64_t)(kvh * kBlock + ks) * D;
  auto load = [&](int blk, KVRegs<D>& R) {
    const int pb = s_bt[blk - blk_begin];
    if (pb >= 0) {
      const int64_t base = (int64_t)pb * block_stride + head_off;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        R.k[j] = *reinterpret_cast<const uint4*>(kp + base + 8 * (qd + 4 * j));
        R.v[j] = *reinterpret_cast<const uint4*>(vp + base + 8 * (qd + 4 * j));
      }
    } else {
#pragma unroll
      for (int j = 0; j < NJ; ++j) { R.k[j] = make_uint4(0, 0, 0, 0); R.v[j] = make_uint4(0, 0, 0, 0); }
    }
  };

  auto step = [&](int blk, const KVRegs<D>& R) {
    const bool kvalid = (s_bt[blk - blk_begin] >= 0) && (blk * kBlock + ks < n);
    float t[GC];
#pragma unroll
    for (int h = 0; h < GC; ++h) {
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        s = T::dot2(R.k[j].x, qv[h][j].x, s);
        s = T::dot2(R.k[j].y, qv[h][j].y, s);
        s = T::dot2(R.k[j].z, qv[h][j].z, s);
        s = T::dot2(R.k[j].w, qv[h][j].w, s);
      }
      s += quad_xor1(s);
      s += quad_xor2(s);
      t[h] = kvalid ? s * c_log2 : -INFINITY;
    }
    bool need = false;
#pragma unroll
    for (int h = 0; h < GC; ++h) need |= t[h] > m[h] + kRescaleThreshold;
    if (__any(need)) {
#pragma unroll
      for (int h = 0; h < GC; ++h) {
        const float mn = fmaxf(m[h], t[h]);
        const float alpha = fast_exp2(m[h] - mn);
        m[h] = mn;
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < NJ * 8; ++e) acc[h][e] *= alpha;
      }
    }
    float p[GC];
#pragma unroll
    for (int h = 0; h < GC; ++h) {
      p[h] = fast_exp2(t[h] - m[h]);
      l[h] += p[h];
    }
    float vf[NJ * 8];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const uint32_t wv[4] = {R.v[j].x, R.v[j].y, R.v[j].z, R.v[j].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vf[j * 8 + 2 * e] = kvalid ? lo_f32<T>(wv[e]) : 0.f;
        vf[j * 8 + 2 * e + 1] = kvalid ? hi_f32<T>(wv[e]) : 0.f;
      }
    }
#pragma unroll
    for (int h = 0; h < GC; ++h)
#pragma unroll
      for (int e = 0; e < NJ * 8; ++e) acc[h][e] = fmaf(p[h], vf[e], acc[h][e]);
  };

  // Software pipeline: the next block's loads are in flight while this one is used.
  int blk = blk_begin + w;
  if (blk < blk_end) {
    KVRegs<D> cur;
    load(blk, cur);
    for (; blk < blk_end; blk += kDecWaves) {
      KVRegs<D> nxt;
      const bool more = blk + kDecWaves < blk_end;
      if (more) load(blk + kDecWaves, nxt);
      step(blk, cur);
      if (more) cur = nxt;
    }
  }

  // Merge the 16 key slots of this wave (lanes with equal l%4): xor over 4, 8, 16, 32.
#pragma unroll
  for (int h = 0; h < GC; ++h) {
    float M = m[h];
    M = fmaxf(M, xor_lane(M, 4));
    M = fmaxf(M, xor_lane(M, 8));
    M = fmaxf(M, xor_lane(M, 16));
    M = fmaxf(M, xor_lane(M, 32));
    const float sc = fast_exp2(m[h] - M);
    float lh = l[h] * sc;
    lh += xor_lane(lh, 4);
    lh += xor_lane(lh, 8);
    lh += xor_lane(lh, 16);
    lh += xor_lane(lh, 32);
#pragma unroll
    for (int e = 0; e < NJ * 8; ++e) {
      float a = acc[h][e] * sc;
      a += xor_lane(a, 4);
      a += xor_lane(a, 8);
      a += xor_lane(a, 16);
      a += xor_lane(a, 32);
      acc[h][e] = a;
    }
    if (lane < 4) {
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) s_acc[w][h][8 * (qd + 4 * j) + e] = acc[h][j * 8 + e];
      if (lane == 0) { s_m[w][h] = M; s_l[w][h] = lh; }
    }
  }
  __syncthreads();

  // Merge the 4 waves and write.
  for (int e = tid; e < nh * D; e += kDecThreads) {
    const int h = e / D, d = e - h * D;
    float M = s_m[0][h];
#pragma unroll
    for (int ww = 1; ww < kDecWaves; ++ww) M = fmaxf(M, s_m[ww][h]);
    float o = 0.f, L = 0.f;
#pragma unroll
    for (int ww = 0; ww < kDecWaves; ++ww) {
      const float sc = fast_exp2(s_m[ww][h] - M);
      o = fmaf(sc, s_acc[ww][h][d], o);
      L = fmaf(sc, s_l[ww][h], L);
    }
    const int64_t row = (int64_t)b * hq + h0 + h;
    if (single) {
      out[row * D + d] = T::from_f32(o / L);
    } else {
      ws_o[(row * nsplit + split) * D + d] = o;
      if (d == 0) {
        ws_ml[(row * nsplit + split) * 2 + 0] = M;
        ws_ml[(row * nsplit + split) * 2 + 1] = L;
      }
    }
  }
}

// One work-group of D threads per (sequence, query head); only sequences whose
// context spans more than one split have partials to combine.
template <typename T, int D>
__global__ void __launch_bounds__(128)
decode_merge_kernel(const float* __restrict__ ws_o, const float* __restrict__ ws_ml,
                    uint16_t* __restrict__ out, const int32_t* __restrict__ ctx_lens, int hq,
                    int split_blocks, int nsplit, int max_ctx, int bt_stride) {
  const int row = blockIdx.x;          // b * hq + h
  const int b = row / hq;
  int n = ctx_lens[b];
  n = min(n, min(max_ctx, bt_stride * kBlock));
  if (n <= 0) return;
  const int nblk = (n + kBlock - 1) / kBlock;
  const int ns = (nblk + split_blocks - 1) / split_blocks;
  if (ns <= 1) return;
  const int d = threadIdx.x;
  if (d >= D) return;
  const float* ml = ws_ml + (int64_t)row * nsplit * 2;
  float M = kNegBig;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, ml[2 * s]);
  float o = 0.f, L = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float sc = fast_exp2(ml[2 * s] - M);
    o = fmaf(sc, ws_o[((int64_t)row * nsplit + s) * D + d], o);
    L = fmaf(sc, ml[2 * s + 1], L);
  }
  out[(int64_t)row * D + d] = T::from_f32(o / L);
}

int decode_heads_per_wg(int G) { return G == 1 ? 1 : (G == 2 ? 2 : 4); }

void decode_plan(int batch, int hkv, int hq, int max_ctx, int split_blocks_req, int* split_blocks,
                 int* nsplit) {
  const int G = hq / hkv;
  const int gc = decode_heads_per_wg(G);
  const int nchunks = (G + gc - 1) / gc;
  const int max_blocks = max_ctx > 0 ? (max_ctx + kBlock - 1) / kBlock : 1;
  int sb = split_blocks_req;
  if (sb <= 0) {
    // aim for >= 2048 work-groups (8 per CU) without splits shorter than 16 blocks
    const long long units = (long long)batch * hkv * nchunks;
    long long want = (2048 + units - 1) / units;
    long long ns = want < 1 ? 1 : want;
    long long max_ns = (max_blocks + 15) / 16;
    if (ns > max_ns) ns = max_ns;
    if (ns < 1) ns = 1;
    sb = (int)((max_blocks + ns - 1) / ns);
    sb = (sb + 3) & ~3;
  }
  if (sb > kMaxSplitBlocks) sb = kMaxSplitBlocks;
  if (sb < 1) sb = 1;
  *split_blocks = sb;
  *nsplit = (max_blocks + sb - 1) / sb;
}

template <typename T, int D, int GC>
static hipError_t launch_decode_t(const kvb_pool& p, const void* q, void* out, const int32_t* ctx,
                                  const int32_t* bt, int bt_stride, int batch, int hq, int max_ctx,
                                  int sb, int ns, float scale, float* ws_o, float* ws_ml,
                                  hipStream_t s) {
  const int G = hq / p.num_kv_heads;
  const int nchunks = (G + GC - 1) / GC;
  const long long real = (long long)batch * p.num_kv_heads * ns * nchunks;
  const long long padded = (real + kNumXcd - 1) / kNumXcd * kNumXcd;
  const float c = scale * 1.4426950408889634f;
  hipLaunchKernelGGL((decode_split_kernel<T, D, GC>), dim3((unsigned)padded), dim3(kDecThreads), 0, s,
                     (const uint16_t*)p.k, (const uint16_t*)p.v, p.block_stride, p.num_blocks,
                     (const uint16_t*)q, (uint16_t*)out, ctx, bt, bt_stride, hq, p.num_kv_heads,
                     nchunks, sb, ns, max_ctx, c, ws_o, ws_ml, (int)padded, (int)real);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ns <= 1) return e;
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3((unsigned)(batch * hq)), dim3(128), 0, s,
                     ws_o, ws_ml, (uint16_t*)out, ctx, hq, sb, ns, max_ctx, bt_stride);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_decode_d(const kvb_pool& p, const void* q, void* out, const int32_t* ctx,
                                  const int32_t* bt, int bt_stride, int batch, int hq, int max_ctx,
                                  int sb, int ns, float scale, float* ws_o, float* ws_ml,
                                  hipStream_t s) {
  switch (decode_heads_per_wg(hq / p.num_kv_heads)) {
    case 1: return launch_decode_t<T, D, 1>(p, q, out, ctx, bt, bt_stride, batch, hq, max_ctx, sb, ns, scale, ws_o, ws_ml, s);
    case 2: return launch_decode_t<T, D, 2>(p, q, out, ctx, bt, bt_stride, batch, hq, max_ctx, sb, ns, scale, ws_o, ws_ml, s);
    default: return launch_decode_t<T, D, 4>(p, q, out, ctx, bt, bt_stride, batch, hq, max_ctx, sb, ns, scale, ws_o, ws_ml, s);
  }
}

hipError_t launch_decode(const kvb_pool& p, const void* q, void* out, const int32_t* ctx,
                         const int32_t* bt, int bt_stride, int batch, int hq, int max_ctx, int sb,
                         int ns, float scale, void* ws, hipStream_t s) {
  float* ws_o = (float*)ws;
  float* ws_ml = ws_o + decode_ws_o_floats(batch, hq, p.head_dim, ns);
  const bool bf = p.dtype == KVB_BF16;
  switch (p.head_dim) {
    case 64:  return bf ? launch_decode_d<BF16, 64>(p, q, out, ctx, bt, bt_stride, batch, hq, max_ctx, sb, ns, scale, ws_o, ws_ml, s)
                        : launch_decode_d<F16, 64>(p, q, out, ctx, bt, bt_stride, batch, hq, max_ctx, sb, ns, scale, ws_o, ws_ml, s);
    case 96:  return bf ? launch_decode_d<BF16, 96>(p, q, out, ctx, bt, bt_stride, batch, hq, max_ctx, sb, ns, scale, ws_o, ws_ml, s)
                        : launch_decode_d<F16, 96>(p, q, out, ctx, bt, bt_stride, batch, hq, max_ctx, sb, ns, scale, ws_o, ws_ml, s);
    default:  return bf ? launch_decode_d<BF16, 128>(p, q, out, ctx, bt, bt_stride, batch, hq, max_ctx, sb, ns, scale, ws_o, ws_ml, s)
                        : launch_decode_d<F16, 128>(p, q, out, ctx, bt, bt_stride, batch, hq, max_ctx, sb, ns, scale, ws_o, ws_ml, s);
  }
}

}  // namespace kvb
