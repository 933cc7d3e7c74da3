// Paged decode: one query per sequence against its whole context in the block pool,
// split over groups of blocks and merged by log-sum-exp.
//
// The decode step is the one-query case of the chunk attention (kvboost 0.6.0, "CPU
// paged attention": only the decode loop changes; kvstream 0.1.0, "Request lifecycle"
// step 2: one slot per generated token, so the current token is already in the pool).
//
// Design (HBM-bound: about G flops per byte of K/V, so the aim is bytes in flight and
// few instructions per byte):
//  * One work-group (4 waves) per (sequence, KV head, head chunk of up to 16 query
//    heads, split of `split_blocks` blocks).  The query heads of one KV group share
//    every K/V byte read.
//  * A wave consumes two 16-token blocks (32 keys) per step and has the next step's
//    K/V loads in flight while it works on the current one.
//  * Every global load instruction reads 1 KiB contiguous (four rows of a block's
//    16 x head_dim run).  K and V pass through a per-wave LDS slot in their natural
//    row-major layout (padded rows, so the operand reads are bank-conflict free).
//  * Scores S^T = K Q^T use v_mfma_f32_16x16x32 with K rows from LDS as the A operand
//    and the queries as the B operand (columns beyond the group are zero).
//  * O^T += V^T P^T also uses 16x16x32: the score accumulators already hold P^T in
//    B-operand layout, and V is read back transposed with ds_read_b64_tr_b16.
//  * Online softmax in the exp2 domain with lazy rescaling: the reference max only
//    moves when a score exceeds it by more than 2^8, so exponentials stay <= 256 and
//    the output rescale is rarely executed.
//  * A split covering the whole context writes the normalised output directly; other
//    splits write (output, max, sum) partials that decode_merge combines.
#include "decode_common.h"
#include "kvb_launch.h"

namespace kvb {

// Shared-prefix part of a grouped cascade decode (ignored by the plain form).  A group
// work-group fills its 16 query columns with `cols` heads of each of `seqs` sequences,
// so every shared block it reads serves all of them.
struct DecGroup {
  const int32_t* blocks;    // physical ids of the shared prefix blocks
  int n_blocks;             // shared prefix length / 16
  int split_blocks;         // shared blocks per group work-group
  int nsplit;               // key splits of the shared prefix: partial slots 0..nsplit-1
  int ngroups;              // sequence groups per (KV head, head chunk)
  int seqs;                 // sequences per group
  int cols;                 // heads per sequence in a group: min(G, 16)
  int per_kvh;              // group work-groups per KV head
  int batch;
};

// Sequences after which the first work-group of a sequence lands on the same shader
// engine again (engines taken in a cycle of four, nsplit work-groups per sequence).
__device__ inline int se_period(int nsplit) {
  return (nsplit & 3) == 0 ? 1 : (nsplit & 1) ? 4 : 2;
}

template <typename T, int D, bool GROUP, int QB>
__global__ void __launch_bounds__(kDecThreads, 2)
decode_split_kernel(const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
                    int64_t block_stride, int num_blocks, const uint16_t* __restrict__ q,
                    uint16_t* __restrict__ out, const int32_t* __restrict__ ctx_lens,
                    const int32_t* __restrict__ bt, int bt_stride, int hq, int hkv, int nchunks,
                    int split_blocks, int nsplit, int max_ctx, float c_log2,
                    float* __restrict__ ws_o, float* __restrict__ ws_ml, int padded, int real,
                    int blk_first, int slot0, int ws_slots, int force_partial, DecGroup grp,
                    DecQ8 q8) {
  constexpr bool Q8 = QB != 0;              // a quantised pool (8 or 4 bits per code)
  static_assert(!(GROUP && Q8), "quantised pools have the plain form only");
  using QStep = DecStepQ<D, (QB ? QB : 8)>;
  using Step = std::conditional_t<Q8, QStep, DecStep<D>>;
  constexpr int NKK = D / 32;
  constexpr int NDB = D / 16;               // 16-row d blocks of O^T
  constexpr int CPR = D / 8;                // 16-byte chunks per K/V row
  constexpr int VCH = D / 32;
  constexpr int VROW = D + 16;              // V row stride (elements): 8 banks apart per row
  constexpr int KROW = D + 8;               // K row stride (elements): 4 banks apart per row
  constexpr int SLOT = 32 * (VROW + KROW);  // two blocks of V then K per wave

  __shared__ __attribute__((aligned(16))) uint16_t sV[kDecWaves * SLOT];
  __shared__ int s_bt[kMaxSplitBlocks];
  __shared__ float s_m[kDecWaves][kDecHeads];
  __shared__ float s_l[kDecWaves][kDecHeads];
  static_assert(kDecWaves * kDecHeads * D * 4 <= kDecWaves * SLOT * 2, "merge buffer reuses the slots");
  float* s_o = reinterpret_cast<float*>(sV);  // [wave][head][D] after the main loop

  const int lid = xcd_logical_id(blockIdx.x, padded);
  if (lid >= real) return;
  const int G = hq / hkv;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = uniform(tid >> 6);
  const int c16 = lane & 15, g4 = lane >> 4;
  // logical id -> (kvh, b, split, chunk), chunk fastest and KV head slowest: each XCD
  // works on few KV heads, so prefix blocks shared by many sequences stay in its L2.
  // Sequence b takes its splits rotated by b / se_period(nsplit): the dispatcher hands an
  // XCD's work-groups to its four shader engines in a fixed cycle, and without the
  // rotation a split count sharing a factor with that cycle would send every sequence's
  // first split (often all shared-prefix blocks, cheap L2 hits) to the same engines
  // while the others carry the long private splits.  The grouped form puts each KV head's group
  // work-groups (chunk, sequence group, shared key split) ahead of its private ones.
  int kvh, b = 0, split = 0, chunk, gi = 0, ks = 0;
  bool group_wg = false;
  if constexpr (GROUP) {
    const int stride = grp.per_kvh + grp.batch * nsplit * nchunks;
    kvh = lid / stride;
    int r = lid - kvh * stride;
    if (r < grp.per_kvh) {
      group_wg = true;
      ks = r % grp.nsplit; r /= grp.nsplit;
      gi = r % grp.ngroups;
      chunk = r / grp.ngroups;
    } else {
      r -= grp.per_kvh;
      chunk = r % nchunks; r /= nchunks;
      const int sr = r % nsplit;
      b = r / nsplit;
      split = (sr + b / se_period(nsplit)) % nsplit;
    }
  } else {
    const int batch = real / (nchunks * nsplit * hkv);
    int r = lid;
    chunk = r % nchunks; r /= nchunks;
    const int sr = r % nsplit; r /= nsplit;
    b = r % batch;
    kvh = r / batch;
    split = (sr + b / se_period(nsplit)) % nsplit;
  }
  const int h0 = kvh * G + chunk * kDecHeads;
  const int nh = min(kDecHeads, G - chunk * kDecHeads);
  // Query row of column h, or -1: head h0 + h of sequence b, or in a group work-group
  // head chunk * cols + h % cols of sequence gi * seqs + h / cols.
  auto row_of = [&](int h) -> int {
    if (GROUP && group_wg) {
      const int seq = gi * grp.seqs + h / grp.cols;
      const int hl = chunk * grp.cols + h % grp.cols;
      return (h < grp.seqs * grp.cols && seq < grp.batch && hl < G) ? seq * hq + kvh * G + hl : -1;
    }
    return h < nh ? b * hq + h0 + h : -1;
  };
  const int ctx_cap = min(max_ctx, bt_stride * kBlock);

  int n, lim;                   // key bound of the loads; key bound of this lane's column
  int blk_begin, blk_end;
  bool single = false;
  const int32_t* tbl;           // block ids from blk_begin on
  if (GROUP && group_wg) {
    // every column's keys in the shared range: min(context, shared length)
    const int row = row_of(c16);
    const int shared_len = grp.n_blocks * kBlock;
    lim = row >= 0 ? min(min(ctx_lens[row / hq], ctx_cap), shared_len) : 0;
    n = lim;
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) n = max(n, __shfl_xor(n, m, 64));
    n = uniform(n);
    blk_begin = ks * grp.split_blocks;
    blk_end = min((n + kBlock - 1) / kBlock, blk_begin + grp.split_blocks);
    tbl = grp.blocks + blk_begin;
  } else {
    n = min(ctx_lens[b], ctx_cap);
    if (n <= 0) {
      if (split == 0 && !force_partial)
        for (int e = tid; e < nh * D; e += kDecThreads)
          out[((int64_t)b * hq + h0 + e / D) * D + (e % D)] = 0;
      return;
    }
    lim = n;
    // keys of this pass: blocks [blk_first, nblk) (blk_first > 0 after a shared prefix)
    const int nblk = (n + kBlock - 1) / kBlock;
    blk_begin = blk_first + split * split_blocks;
    if (blk_begin >= nblk) return;
    blk_end = min(nblk, blk_begin + split_blocks);
    single = !force_partial && nblk <= split_blocks;
    tbl = bt + (int64_t)b * bt_stride + blk_begin;
  }
  // a group work-group whose columns all end before its key split still writes its
  // (empty) partials: the merge reads every shared slot of a row
  for (int i = tid; i < blk_end - blk_begin; i += kDecThreads) {
    const int pb = tbl[i];
    s_bt[i] = (pb >= 0 && pb < num_blocks) ? pb : -1;
  }

  // queries as the B operand: column c16 (row row_of(c16)), d chunk 4*kk + g4
  s16x8 qb[NKK];
  {
    const int qrow = row_of(c16);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      if (qrow >= 0)
        qb[kk] = *reinterpret_cast<const s16x8*>(q + (int64_t)qrow * D + 8 * (4 * kk + g4));
      else
        qb[kk] = s16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  if constexpr (Q8) {
    // K's per-channel scales folded into the queries: q . k = sum_e (q_e s_e) code_e
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const float* ks = q8.k_scale + kvh * D + 8 * (4 * kk + g4);
      const f32x4 a = *reinterpret_cast<const f32x4*>(ks);
      const f32x4 c = *reinterpret_cast<const f32x4*>(ks + 4);
      const float sc[8] = {a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = pack2<T>(T::to_f32((uint16_t)qb[kk][2 * i]) * sc[2 * i],
                        T::to_f32((uint16_t)qb[kk][2 * i + 1]) * sc[2 * i + 1]);
      qb[kk] = __builtin_bit_cast(s16x8, make_uint4(w[0], w[1], w[2], w[3]));
    }
  }

  f32x4 o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegBig, l_run = 0.f;
  __syncthreads();

  const int64_t head_off = (int64_t)kvh * kBlock * D;
  uint16_t* slot = sV + w * SLOT;           // V rows 0..31
  uint16_t* kslot = slot + 32 * VROW;       // K rows 0..31
  // Store positions in the slot: when a row is a whole number of 16-byte chunks that
  // divides 64 (d = 64, 128), chunk j of every lane lands a constant number of rows
  // below chunk 0, so one base per K and V serves every store.
  constexpr bool kWholeRows = 64 % CPR == 0;
  const int v_st = (lane / CPR) * VROW + (lane % CPR) * 8;
  const int k_st = (lane / CPR) * KROW + (lane % CPR) * 8;

  // Blocks that are read once are loaded with the non-temporal policy, so that they evict
  // less of the shared-prefix blocks other work-groups re-read from L2: in the grouped
  // shared-prefix form the private splits; in the plain form every split after a
  // sequence's first (and a whole private pass after a shared prefix).  The plain form
  // cannot see which blocks are shared; prefixes shared between requests start their
  // sequences, so its first split keeps the normal policy.  The choice is made once per
  // work-group: the main loop is compiled for both policies.
  const bool stream_loads = !Q8 && (GROUP ? !group_wg : (blk_first > 0 || split > 0));

  // Both blocks of a step through buffer resources sized to their valid rows: rows past
  // the context, blocks past the split and blocks outside the pool read as zero and
  // cost no memory traffic, and every load is issued unconditionally.
  auto load = [&](int blk0, Step& R, auto nt_c) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int blk = blk0 + hb;
      const int pb = uniform(blk < blk_end ? s_bt[blk - blk_begin] : -1);
      const int rows = pb >= 0 ? min(kBlock, n - blk * kBlock) : 0;
      R.rows[hb] = rows;
      R.pos[hb] = blk * kBlock;
      const int64_t off = (int64_t)(pb >= 0 ? pb : 0) * block_stride + head_off;
      if constexpr (Q8) {
        // codes: D*QB/8 bytes per key row; block_stride counts bytes
        const int64_t qoff = (int64_t)(pb >= 0 ? pb : 0) * block_stride + (int64_t)kvh * kBlock * D * QB / 8;
        const uint8_t* kb = reinterpret_cast<const uint8_t*>(kp) + qoff;
        const uint8_t* vb = reinterpret_cast<const uint8_t*>(vp) + qoff;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, (uint32_t)(rows * D * QB / 8));
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, (uint32_t)(rows * D * QB / 8));
#pragma unroll
        for (int j = 0; j < QStep::NCH; ++j) {
          R.k[hb][j] = buf_load16(rk, (uint32_t)(j * 64 + lane) * 16);
          R.v[hb][j] = buf_load16(rv, (uint32_t)(j * 64 + lane) * 16);
        }
        const float* sb = q8.v_scale + ((int64_t)(pb >= 0 ? pb : 0) * hkv + kvh) * kBlock;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(sb, (uint32_t)(rows * 4));
#pragma unroll
        for (int j = 0; j < QStep::NCH; ++j)           // chunk j*64+lane: key row chunk / CPRQ
          R.vsc[hb][j] = __builtin_bit_cast(
              float, __builtin_amdgcn_raw_buffer_load_b32(rs, (j * 64 + lane) / QStep::CPRQ * 4, 0, 0));
        continue;
      }
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(kp + off, (uint32_t)(rows * D * 2));
      const __amdgpu_buffer_rsrc_t rv = make_rsrc(vp + off, (uint32_t)(rows * D * 2));
      if constexpr (decltype(nt_c)::value) {
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
  };

  auto step = [&](const Step& R) {
    // V of both blocks into this wave's LDS slot, natural [key][d] layout (rows past
    // the context arrive as zeros, so NaN left in unused pool slots never reaches PV).
    // Codes are widened to T on the way (chunk c: key row c / CPRQ, 128/QB columns), V
    // codes multiplied by their key's V scale there (dequantised in the LDS stage).
    if constexpr (Q8) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb)
#pragma unroll
        for (int j = 0; j < QStep::NCH; ++j) {
          const int c = j * 64 + lane;
          if (c >= QStep::CH) continue;           // chunks past the block (some lanes)
          const int row = c / QStep::CPRQ, col = (c - row * QStep::CPRQ) * (128 / QB);
          uint16_t* vrow = slot + (hb * 16 + row) * VROW + col;
          uint16_t* krow = kslot + (hb * 16 + row) * KROW + col;
          if constexpr (QB == 8) {
            uint4 lo, hi;
            codes_to<T>(R.v[hb][j], R.vsc[hb][j], lo, hi);
            *reinterpret_cast<uint4*>(vrow) = lo;
            *reinterpret_cast<uint4*>(vrow + 8) = hi;
            codes_to<T>(R.k[hb][j], 1.f, lo, hi);
            *reinterpret_cast<uint4*>(krow) = lo;
            *reinterpret_cast<uint4*>(krow + 8) = hi;
          } else {
            uint4 o4[4];
            nibbles_to<T>(R.v[hb][j], R.vsc[hb][j], o4);
#pragma unroll
            for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(vrow + 8 * i) = o4[i];
            nibbles_to<T>(R.k[hb][j], 1.f, o4);
#pragma unroll
            for (int i = 0; i < 4; ++i) *reinterpret_cast<uint4*>(krow + 8 * i) = o4[i];
          }
        }
    } else
#pragma unroll
    for (int hb = 0; hb < 2; ++hb)
#pragma unroll
      for (int j = 0; j < VCH; ++j) {
        int vo, ko;
        if constexpr (kWholeRows) {
          vo = v_st + (hb * 16 + j * (64 / CPR)) * VROW;
          ko = k_st + (hb * 16 + j * (64 / CPR)) * KROW;
        } else {
          const int c = j * 64 + lane;
          const int row = c / CPR, col = c - (c / CPR) * CPR;
          vo = (hb * 16 + row) * VROW + col * 8;
          ko = (hb * 16 + row) * KROW + col * 8;
        }
        *reinterpret_cast<uint4*>(slot + vo) = R.v[hb][j];
        *reinterpret_cast<uint4*>(kslot + ko) = R.k[hb][j];
      }
    __builtin_amdgcn_wave_barrier();
    // S^T = K Q^T per block: A operand = key row c16, d chunk 4*kk + g4
    f32x4 s[2];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      s[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const s16x8 a = *reinterpret_cast<const s16x8*>(kslot + (hb * 16 + c16) * KROW + 8 * (4 * kk + g4));
        s[hb] = T::mfma16(a, qb[kk], s[hb]);
      }
    }
    // scale + mask: lane holds keys 4*g4 + rr of each block for head column c16
    float t[8];
    float mx = -INFINITY;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        bool ok = 4 * g4 + rr < R.rows[hb];
        if constexpr (GROUP) ok = ok && R.pos[hb] + 4 * g4 + rr < lim;
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
      const float p0 = fast_exp2(t[2 * e] - m_run);
      const float p1 = fast_exp2(t[2 * e + 1] - m_run);
      l_run += p0 + p1;
      pw[e] = pack2<T>(p0, p1);
    }
    const s16x8 pb8 = __builtin_bit_cast(s16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
    __builtin_amdgcn_wave_barrier();
    // O^T += V^T P^T: A operand rows d = 16*db + c16, keys 4*g4.. of block 0 then block 1
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

  // Each wave takes every fourth pair of blocks; the next pair's loads are in flight
  // while the current pair is used (past the end they are zero-size, i.e. free), in two
  // named buffers in ping-pong so that no register copy forces a wait on loads that are
  // still in flight.
  const int nsteps = (blk_end - blk_begin - 2 * w + 2 * kDecWaves - 1) / (2 * kDecWaves);
  auto main_loop = [&](auto nt_c) {
    constexpr int kStride = 2 * kDecWaves;
    int blk0 = blk_begin + 2 * w;
    Step A, B;
    load(blk0, A, nt_c);
    for (int it = 0; it < nsteps; it += 2) {
      load(blk0 + kStride, B, nt_c);
      step(A);
      if (it + 1 >= nsteps) break;
      load(blk0 + 2 * kStride, A, nt_c);
      step(B);
      blk0 += 2 * kStride;
    }
  };
  if (nsteps > 0) {
    if (stream_loads) main_loop(std::true_type{});
    else main_loop(std::false_type{});
  }

  // row sums over the four key groups of the wave
  float lsum = l_run;
  lsum = halves_sum(lsum + xor16(lsum));
  __syncthreads();                          // V slots are reused as the merge buffer
  const int ncol = (GROUP && group_wg) ? kDecHeads : nh;
  if (c16 < ncol) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        s_o[(w * kDecHeads + c16) * D + 16 * db + 4 * g4 + rr] = o[db][rr];
    if (g4 == 0) { s_m[w][c16] = m_run; s_l[w][c16] = lsum; }
  }
  __syncthreads();

  const int slot_w = (GROUP && group_wg) ? ks : slot0 + split;
  for (int e = tid; e < ncol * D; e += kDecThreads) {
    const int h = e / D, d = e - h * D;
    const int qrow = row_of(h);
    if (qrow < 0) continue;
    float M = s_m[0][h];
#pragma unroll
    for (int ww = 1; ww < kDecWaves; ++ww) M = fmaxf(M, s_m[ww][h]);
    float ov = 0.f, L = 0.f;
#pragma unroll
    for (int ww = 0; ww < kDecWaves; ++ww) {
      const float sc = fast_exp2(s_m[ww][h] - M);
      ov = fmaf(sc, s_o[(ww * kDecHeads + h) * D + d], ov);
      L = fmaf(sc, s_l[ww][h], L);
    }
    const int64_t row = qrow;
    if (single) {
      out[row * D + d] = T::from_f32(ov / L);
    } else {
      const int64_t slot = row * ws_slots + slot_w;
      ws_o[slot * D + d] = ov;
      if (d == 0) {
        ws_ml[slot * 2 + 0] = M;
        ws_ml[slot * 2 + 1] = L;
      }
    }
  }
}

// One wave per (sequence, query head) row, four rows per work-group.  Slots: `n_shared`
// partials of a shared prefix (cascade form; 0 otherwise), then one per split of blocks
// [blk_first, nblk).  Without a shared prefix only sequences spanning more than one
// split have partials to combine (a single split wrote its row directly).
// Every slot of the row is loaded without waiting for the context length (eight at a
// time, all in flight together); slots past the row's count only enter through selects,
// so whatever they hold never reaches the result.  The merge is one memory round trip.

template <typename T, int D>
__global__ void __launch_bounds__(64 * kMergeRows)
decode_merge_kernel(const float* __restrict__ ws_o, const float* __restrict__ ws_ml,
                    uint16_t* __restrict__ out, const int32_t* __restrict__ ctx_lens, int rows,
                    int hq, int split_blocks, int ws_slots, int max_ctx, int bt_stride,
                    int blk_first, int n_shared, int cascade) {
  constexpr int NV = (D + 63) / 64;    // d values per lane: d = lane + 64 * i
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kMergeRows + uniform(threadIdx.x >> 6);
  if (row >= rows) return;
  const int b = row / hq;
  int n = ctx_lens[b];
  const float* ml = ws_ml + (int64_t)row * ws_slots * 2;
  const float* po = ws_o + (int64_t)row * ws_slots * D;
  float2 mine;                         // (max, sum) of slot s0 + lane % 8
  // lanes past the head dimension re-read its last element (never written out), so the
  // loads need no branch
  float v[kMergeBatch][NV];
  auto load = [&](int s0) {
    mine = *reinterpret_cast<const float2*>(ml + 2 * min(s0 + (lane & (kMergeBatch - 1)), ws_slots - 1));
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const int s = min(s0 + j, ws_slots - 1);
#pragma unroll
      for (int i = 0; i < NV; ++i) v[j][i] = po[(int64_t)s * D + min(lane + 64 * i, D - 1)];
    }
  };
  load(0);
  // keeps the first batch of loads ahead of the branches on the context length
  asm volatile("" :: "v"(mine.x), "v"(mine.y));
#pragma unroll
  for (int j = 0; j < kMergeBatch; ++j) {
#pragma unroll
    for (int i = 0; i < NV; ++i) asm volatile("" :: "v"(v[j][i]));
  }
  n = min(n, min(max_ctx, bt_stride * kBlock));
  if (n <= 0) {
    if (cascade)
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (lane + 64 * i < D) out[(int64_t)row * D + lane + 64 * i] = 0;
    return;
  }
  const int nblk = (n + kBlock - 1) / kBlock;
  const int ns_priv = nblk > blk_first ? (nblk - blk_first + split_blocks - 1) / split_blocks : 0;
  if (!cascade && ns_priv <= 1) return;
  const int ns = n_shared + ns_priv;
  float M = kNegBig, L = 0.f;
  float o[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) o[i] = 0.f;
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

int decode_heads_per_wg(int G) { return G < kDecHeads ? G : kDecHeads; }

void decode_plan(int batch, int hkv, int hq, int max_ctx, int split_blocks_req, int* split_blocks,
                 int* nsplit) {
  const int G = hq / hkv;
  const int nchunks = (G + kDecHeads - 1) / kDecHeads;
  const int max_blocks = max_ctx > 0 ? (max_ctx + kBlock - 1) / kBlock : 1;
  int sb = split_blocks_req;
  if (sb <= 0) {
    // about six work-groups per CU (three rounds of the two that fit at once) without
    // splits shorter than 16 blocks
    const long long units = (long long)batch * hkv * nchunks;
    const long long target = 6LL * device_cu_count();
    long long ns = (target + units - 1) / units;
    const long long max_ns = (max_blocks + 15) / 16;
    if (ns > max_ns) ns = max_ns;
    if (ns < 1) ns = 1;
    sb = (int)((max_blocks + ns - 1) / ns);
    sb = (sb + 7) & ~7;                  // whole steps for the four waves
  }
  if (sb > kMaxSplitBlocks) sb = kMaxSplitBlocks;
  if (sb < 1) sb = 1;
  *split_blocks = sb;
  *nsplit = (max_blocks + sb - 1) / sb;
}

template <typename T, int D, int QB = 0>
static hipError_t launch_decode_t(const kvb_pool& p, const void* q, void* out, const int32_t* ctx,
                                  const int32_t* bt, int bt_stride, int batch, int hq, int max_ctx,
                                  int sb, int ns, float scale, float* ws_o, float* ws_ml,
                                  hipStream_t s, DecQ8 q8 = DecQ8{}) {
  const int G = hq / p.num_kv_heads;
  const int nchunks = (G + kDecHeads - 1) / kDecHeads;
  const long long real = (long long)batch * p.num_kv_heads * ns * nchunks;
  if (real == 0) return hipSuccess;
  const long long padded = (real + kNumXcd - 1) / kNumXcd * kNumXcd;
  const float c = scale * 1.4426950408889634f;
  hipLaunchKernelGGL((decode_split_kernel<T, D, false, QB>), dim3((unsigned)padded), dim3(kDecThreads), 0, s,
                     (const uint16_t*)p.k, (const uint16_t*)p.v, p.block_stride, p.num_blocks,
                     (const uint16_t*)q, (uint16_t*)out, ctx, bt, bt_stride, hq, p.num_kv_heads,
                     nchunks, sb, ns, max_ctx, c, ws_o, ws_ml, (int)padded, (int)real, 0, 0, ns, 0,
                     DecGroup{}, q8);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || ns <= 1) return e;
  const int rows = batch * hq;
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3((unsigned)((rows + kMergeRows - 1) / kMergeRows)),
                     dim3(64 * kMergeRows), 0, s, ws_o, ws_ml, (uint16_t*)out, ctx, rows, hq, sb, ns,
                     max_ctx, bt_stride, 0, 0, 0);
  return hipGetLastError();
}

// Cascade: private pass over blocks [shared_len/16, nblk) into slots nks.., then the
// merge of the nks shared partials (written before by launch_cascade_shared) with them.
template <typename T, int D>
static hipError_t launch_decode_private_t(const kvb_pool& p, const void* q, void* out,
                                          const int32_t* ctx, const int32_t* bt, int bt_stride,
                                          int batch, int hq, int max_ctx, int sb, int ns,
                                          int blk_first, int nks, float scale, float* ws_o,
                                          float* ws_ml, hipStream_t s) {
  const int G = hq / p.num_kv_heads;
  const int nchunks = (G + kDecHeads - 1) / kDecHeads;
  const int slots = nks + ns;
  const long long real = (long long)batch * p.num_kv_heads * ns * nchunks;
  if (real > 0) {
    const long long padded = (real + kNumXcd - 1) / kNumXcd * kNumXcd;
    const float c = scale * 1.4426950408889634f;
    hipLaunchKernelGGL((decode_split_kernel<T, D, false, 0>), dim3((unsigned)padded), dim3(kDecThreads), 0, s,
                       (const uint16_t*)p.k, (const uint16_t*)p.v, p.block_stride, p.num_blocks,
                       (const uint16_t*)q, (uint16_t*)out, ctx, bt, bt_stride, hq, p.num_kv_heads,
                       nchunks, sb, ns, max_ctx, c, ws_o, ws_ml, (int)padded, (int)real, blk_first,
                       nks, slots, 1, DecGroup{}, DecQ8{});
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int rows = batch * hq;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3((unsigned)((rows + kMergeRows - 1) / kMergeRows)),
                     dim3(64 * kMergeRows), 0, s, ws_o, ws_ml, (uint16_t*)out, ctx, rows, hq, sb,
                     slots, max_ctx, bt_stride, blk_first, nks, 1);
  return hipGetLastError();
}

hipError_t launch_decode_cascade(const kvb_pool& p, const void* q, void* out, const int32_t* ctx,
                                 const int32_t* bt, int bt_stride, const int32_t* shared_blocks,
                                 int shared_len, int batch, int hq, int max_ctx, int sb, int ns,
                                 int nks, int ks_tiles, float scale, void* ws, hipStream_t s) {
  const int slots = nks + ns;
  float* ws_o = (float*)ws;
  float* ws_ml = ws_o + (int64_t)batch * hq * slots * p.head_dim;
  hipError_t e = launch_cascade_shared(p, q, ctx, max_ctx, shared_blocks, shared_len, batch, hq,
                                       scale, nks, ks_tiles, ws_o, ws_ml, slots, s);
  if (e != hipSuccess) return e;
  const int blk_first = shared_len / kBlock;
  const bool bf = p.dtype == KVB_BF16;
  switch (p.head_dim) {
    case 64:  return bf ? launch_decode_private_t<BF16, 64>(p, q, out, ctx, bt, bt_stride, batch, hq, max_ctx, sb, ns, blk_first, nks, scale, ws_o, ws_ml, s)
                        : launch_decode_private_t<F16, 64>(p, q, out, ctx, bt, bt_stride, batch, hq, max_ctx, sb, ns, blk_first, nks, scale, ws_o, ws_ml, s);
    case 96:  return bf ? launch_decode_private_t<BF16, 96>(p, q, out, ctx, bt, bt_stride, batch, hq, max_ctx, sb, ns, blk_first, nks, scale, ws_o, ws_ml, s)
                        : launch_decode_private_t<F16, 96>(p, q, out, ctx, bt, bt_stride, batch, hq, max_ctx, sb, ns, blk_first, nks, scale, ws_o, ws_ml, s);
    default:  return bf ? launch_decode_private_t<BF16, 128>(p, q, out, ctx, bt, bt_stride, batch, hq, max_ctx, sb, ns, blk_first, nks, scale, ws_o, ws_ml, s)
                        : launch_decode_private_t<F16, 128>(p, q, out, ctx, bt, bt_stride, batch, hq, max_ctx, sb, ns, blk_first, nks, scale, ws_o, ws_ml, s);
  }
}

// Grouped cascade: one launch of the split kernel holds, per KV head, the group
// work-groups over the shared prefix (partials to slots 0..sh_ns-1) and the private
// splits from block shared_len/16 (slots sh_ns..), then the merge over every slot.
void decode_group_plan(int shared_len, int sb, int* sh_split_blocks, int* sh_nsplit) {
  const int nsh = (shared_len + kBlock - 1) / kBlock;
  if (nsh <= 0) { *sh_split_blocks = 0; *sh_nsplit = 0; return; }
  int ns = (nsh + sb - 1) / sb;
  int ssb = (nsh + ns - 1) / ns;
  ssb = (ssb + 7) & ~7;                 // whole steps for the four waves
  if (ssb > kMaxSplitBlocks) ssb = kMaxSplitBlocks;
  *sh_split_blocks = ssb;
  *sh_nsplit = (nsh + ssb - 1) / ssb;
}

// The grouped form re-reads every shared block once per sequence group (from L2, beside
// the private work in the same launch); the separate pass reads it once per 128 query
// rows but costs a launch of its own on the critical path.  Measured on MI355X (d = 128,
// 32 or 64 query heads, 8 KV heads, 8..256 sequences, shared prefixes of 1K..16K tokens):
// grouped is ahead up to about 1024 group-block reads per KV head and head chunk, the
// separate pass beyond 2048.
bool cascade_use_grouped(int batch, int hkv, int hq, int shared_len) {
  const int G = hq / hkv;
  const int cols = G < kDecHeads ? G : kDecHeads;
  const long long ngroups = (batch + kDecHeads / cols - 1) / (kDecHeads / cols);
  const long long nsh = (shared_len + kBlock - 1) / kBlock;
  return ngroups * nsh <= 1024;
}

template <typename T, int D>
static hipError_t launch_decode_grouped_t(const kvb_pool& p, const void* q, void* out,
                                          const int32_t* ctx, const int32_t* bt, int bt_stride,
                                          const int32_t* shared_blocks, int shared_len, int batch,
                                          int hq, int max_ctx, int sb, int ns, int sh_sb, int sh_ns,
                                          float scale, float* ws_o, float* ws_ml, hipStream_t s) {
  const int G = hq / p.num_kv_heads;
  const int nchunks = (G + kDecHeads - 1) / kDecHeads;
  DecGroup g{};
  g.blocks = shared_blocks;
  g.n_blocks = (min(shared_len, max_ctx) + kBlock - 1) / kBlock;
  g.split_blocks = sh_sb;
  g.nsplit = sh_ns;
  g.cols = G < kDecHeads ? G : kDecHeads;
  g.seqs = kDecHeads / g.cols;
  g.ngroups = (batch + g.seqs - 1) / g.seqs;
  g.per_kvh = sh_ns > 0 ? nchunks * g.ngroups * sh_ns : 0;
  g.batch = batch;
  const int slots = sh_ns + ns;
  const int blk_first = shared_len / kBlock;
  const long long real = (long long)p.num_kv_heads * (g.per_kvh + (long long)batch * ns * nchunks);
  if (real > 0) {
    const long long padded = (real + kNumXcd - 1) / kNumXcd * kNumXcd;
    const float c = scale * 1.4426950408889634f;
    hipLaunchKernelGGL((decode_split_kernel<T, D, true, 0>), dim3((unsigned)padded), dim3(kDecThreads), 0, s,
                       (const uint16_t*)p.k, (const uint16_t*)p.v, p.block_stride, p.num_blocks,
                       (const uint16_t*)q, (uint16_t*)out, ctx, bt, bt_stride, hq, p.num_kv_heads,
                       nchunks, sb, ns, max_ctx, c, ws_o, ws_ml, (int)padded, (int)real, blk_first,
                       sh_ns, slots, 1, g, DecQ8{});
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int rows = batch * hq;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3((unsigned)((rows + kMergeRows - 1) / kMergeRows)),
                     dim3(64 * kMergeRows), 0, s, ws_o, ws_ml, (uint16_t*)out, ctx, rows, hq, sb,
                     slots, max_ctx, bt_stride, blk_first, sh_ns, 1);
  return hipGetLastError();
}

hipError_t launch_decode_grouped(const kvb_pool& p, const void* q, void* out, const int32_t* ctx,
                                 const int32_t* bt, int bt_stride, const int32_t* shared_blocks,
                                 int shared_len, int batch, int hq, int max_ctx, int sb, int ns,
                                 int sh_sb, int sh_ns, float scale, void* ws, hipStream_t s) {
  const int slots = sh_ns + ns;
  float* ws_o = (float*)ws;
  float* ws_ml = ws_o + (int64_t)batch * hq * slots * p.head_dim;
  const bool bf = p.dtype == KVB_BF16;
#define KVB_GROUPED(TT, DD) launch_decode_grouped_t<TT, DD>(p, q, out, ctx, bt, bt_stride, shared_blocks, \
    shared_len, batch, hq, max_ctx, sb, ns, sh_sb, sh_ns, scale, ws_o, ws_ml, s)
  switch (p.head_dim) {
    case 64:  return bf ? KVB_GROUPED(BF16, 64) : KVB_GROUPED(F16, 64);
    case 96:  return bf ? KVB_GROUPED(BF16, 96) : KVB_GROUPED(F16, 96);
    default:  return bf ? KVB_GROUPED(BF16, 128) : KVB_GROUPED(F16, 128);
  }
#undef KVB_GROUPED
}

hipError_t launch_decode(const kvb_pool& p, const void* q, void* out, const int32_t* ctx,
                         const int32_t* bt, int bt_stride, int batch, int hq, int max_ctx, int sb,
                         int ns, float scale, void* ws, hipStream_t s) {
  float* ws_o = (float*)ws;
  float* ws_ml = ws_o + decode_ws_o_floats(batch, hq, p.head_dim, ns);
  const bool bf = p.dtype == KVB_BF16;
  switch (p.head_dim) {
    case 64:  return bf ? launch_decode_t<BF16, 64>(p, q, out, ctx, bt, bt_stride, batch, hq, max_ctx, sb, ns, scale, ws_o, ws_ml, s)
                        : launch_decode_t<F16, 64>(p, q, out, ctx, bt, bt_stride, batch, hq, max_ctx, sb, ns, scale, ws_o, ws_ml, s);
    case 96:  return bf ? launch_decode_t<BF16, 96>(p, q, out, ctx, bt, bt_stride, batch, hq, max_ctx, sb, ns, scale, ws_o, ws_ml, s)
                        : launch_decode_t<F16, 96>(p, q, out, ctx, bt, bt_stride, batch, hq, max_ctx, sb, ns, scale, ws_o, ws_ml, s);
    default:  return bf ? launch_decode_t<BF16, 128>(p, q, out, ctx, bt, bt_stride, batch, hq, max_ctx, sb, ns, scale, ws_o, ws_ml, s)
                        : launch_decode_t<F16, 128>(p, q, out, ctx, bt, bt_stride, batch, hq, max_ctx, sb, ns, scale, ws_o, ws_ml, s);
  }
}

// Decode over a quantised pool (8 or 4 bits per code): the split kernel's quantised form
// (codes widened in the LDS stage, V codes times their key's scale there, K scales folded
// into the queries), then the same merge.  The workspace layout is the 16-bit decode's.
hipError_t launch_decode_q8(const kvb_pool_q8& p8, int bits, int dtype, const void* q, void* out,
                            const int32_t* ctx, const int32_t* bt, int bt_stride, int batch, int hq,
                            int max_ctx, int sb, int ns, float scale, void* ws, hipStream_t s) {
  const kvb_pool p{p8.k, p8.v, p8.block_stride, p8.num_blocks, kBlock, p8.num_kv_heads,
                   p8.head_dim, dtype};
  const DecQ8 q8{p8.k_scale, p8.v_scale};
  float* ws_o = (float*)ws;
  float* ws_ml = ws_o + decode_ws_o_floats(batch, hq, p.head_dim, ns);
  const bool bf = dtype == KVB_BF16;
#define KVB_DQ(TT, DD, QQ) launch_decode_t<TT, DD, QQ>(p, q, out, ctx, bt, bt_stride, batch, hq, \
    max_ctx, sb, ns, scale, ws_o, ws_ml, s, q8)
#define KVB_DQB(DD) (bits == 4 ? (bf ? KVB_DQ(BF16, DD, 4) : KVB_DQ(F16, DD, 4)) \
                               : (bf ? KVB_DQ(BF16, DD, 8) : KVB_DQ(F16, DD, 8)))
  switch (p.head_dim) {
    case 64:  return KVB_DQB(64);
    case 96:  return KVB_DQB(96);
    default:  return KVB_DQB(128);
  }
#undef KVB_DQB
#undef KVB_DQ
}

}  // namespace kvb
