/*
 * kvb.h — C ABI of the paged prefix-reuse attention library (libkvb.so, gfx950).
 *
 * The problem these calls solve is stated across three web pages:
 *   - kvboost 0.6.0 (PyPI project page), "CPU paged attention": K/V live in a fixed,
 *     pre-allocated pool of 16-token physical blocks; shared prefixes share blocks
 *     copy-on-write.
 *   - kvstream 0.1.0 (PyPI project page), "Why KVStream?" feature table and "Request
 *     lifecycle": pages allocated one slot per generated token; a prefix hit forks the
 *     cached block table copy-on-write; "Configuration": one page holds
 *     block_size x heads x head_dim x 2 x dtype_bytes.
 *   - kvboost 0.6.0, "How it works" step 5: the cached prefix and the live suffix go
 *     through one forward pass; "Flash Attention (CUDA)": fp16/bf16, head dims
 *     64/96/128, any sequence length, causal masking that skips future K/V tiles.
 *
 * Conventions shared by every call
 *   - Every pointer marked (device) is a device address on the current HIP device;
 *     (host) pointers are read during the call only.  The caller owns every buffer.
 *     The library allocates nothing, never synchronises, never reads device memory
 *     on the host and keeps no state: calls are thread-safe and asynchronous on
 *     `stream` (a hipStream_t; NULL = the null stream).
 *   - Arguments are validated on the host before any launch.  A failed check
 *     returns KVB_ERR_NULL / KVB_ERR_INVALID / KVB_ERR_UNSUPPORTED /
 *     KVB_ERR_WORKSPACE and launches nothing.  The only HIP calls validation and
 *     planning make are queries: the current device and its compute-unit count (the
 *     decode split plan and the prefill's grid form depend on it) and, in
 *     kvb_copy_blocks, the attributes of the pool pointers.  A failed launch returns
 *     KVB_ERR_LAUNCH.
 *   - Device pointers must be 16-byte aligned (KVB_ERR_INVALID otherwise).
 *   - Device-side index contents are the caller's contract (no device-to-host read
 *     checks them).  The kernels are nevertheless memory-safe against bad indices:
 *     a slot or block id outside the pool is never dereferenced (a slot is then
 *     skipped; a key in such a block is excluded from the softmax).
 *   - Softmax scale: any finite value >= 0 (1/sqrt(head_dim) is the usual choice).
 */
#ifndef KVB_H
#define KVB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVB_OK = 0,
  KVB_ERR_NULL = 1,         /* a required pointer is NULL                               */
  KVB_ERR_INVALID = 2,      /* inconsistent sizes, negative counts, misalignment        */
  KVB_ERR_UNSUPPORTED = 3,  /* head_dim not in {64,96,128}, block_size != 16, bad dtype */
  KVB_ERR_WORKSPACE = 4,    /* workspace missing or smaller than the size query returns */
  KVB_ERR_LAUNCH = 5,       /* the HIP runtime reported an error at launch              */
  KVB_ERR_TOO_LARGE = 6     /* kvb_paged_decode_noalloc: more scratch than it holds     */
} kvb_status;

typedef enum { KVB_FP16 = 0, KVB_BF16 = 1 } kvb_dtype;

/* The K/V block pool.  Layout of each of k and v (device):
 *   element (block, kv_head, row, e) at  block*block_stride + (kv_head*16 + row)*head_dim + e
 * so one (block, kv-head) tile is a contiguous 16 x head_dim run (4 KiB at head_dim 128 in
 * 16-bit types).  block_stride (elements) >= num_kv_heads*16*head_dim, a multiple of 8 and
 * below 2^31 (the byte offset of a block, block*block_stride*2, may exceed 32 bits);
 * setting v = k + num_kv_heads*16*head_dim and block_stride = 2*num_kv_heads*16*head_dim
 * interleaves K and V per block, which is exactly one page of the kvstream formula. */
typedef struct {
  void*    k;              /* (device) K pool                                  */
  void*    v;              /* (device) V pool                                  */
  int64_t  block_stride;   /* elements between consecutive physical blocks     */
  int32_t  num_blocks;     /* physical blocks in the pool (> 0)                */
  int32_t  block_size;     /* tokens per block; must be 16                     */
  int32_t  num_kv_heads;   /* > 0                                              */
  int32_t  head_dim;       /* 64, 96 or 128                                    */
  int32_t  dtype;          /* kvb_dtype                                        */
} kvb_pool;

/* Slot scatter (kvstream 0.1.0, "Why KVStream?": streaming KV allocation, one slot per
 * token).  For every t < num_tokens with 0 <= slot_mapping[t] < num_blocks*16:
 *   pool.k[slot/16][h][slot%16][:] = k_new[t][h][:]  and the same for v, for every kv head h.
 * k_new, v_new: (device) [num_tokens][num_kv_heads][head_dim] contiguous, pool dtype.
 * slot_mapping: (device) int64 [num_tokens]; negative (or out-of-pool) slots are skipped.
 * Two tokens mapped to one slot in one call leave an unspecified one of them there.
 * num_tokens == 0 is a no-op. */
kvb_status kvb_write_kv(const kvb_pool* pool, const void* k_new, const void* v_new,
                        const int64_t* slot_mapping, int32_t num_tokens, void* stream);

/* Paged prefill (kvboost 0.6.0, "How it works" steps 3 and 5; "Flash Attention (CUDA)").
 * Sequence b owns chunk rows t in [cu_q_lens[b], cu_q_lens[b+1]); chunk row i = t -
 * cu_q_lens[b] sits at position prefix_lens[b] + i and attends, for query head h, to
 *   - the cached prefix keys j < prefix_lens[b], read from the pool through
 *     block_tables[b*block_table_stride + j/16], row j%16, kv head h / (num_q_heads/num_kv_heads);
 *   - the chunk's own keys 0..i, read from k_new/v_new rows cu_q_lens[b] + 0..i.
 * out[t][h][:] = softmax(scale * q[t][h] . K^T) V, rounded to the pool dtype.
 * q, out: (device) [total_q][num_q_heads][head_dim]; k_new, v_new: (device)
 * [total_q][num_kv_heads][head_dim]; cu_q_lens: (device) int32 [batch+1], non-decreasing,
 * cu_q_lens[0] = 0, cu_q_lens[batch] = total_q; prefix_lens: (device) int32 [batch] >= 0;
 * block_tables: (device) int32 [batch][block_table_stride] with
 * block_table_stride >= ceil(max_prefix_len/16).  max_q_len >= every chunk length (and
 * <= total_q, else KVB_ERR_INVALID) and max_prefix_len >= every prefix length (host
 * bounds used for the launch grid; a larger value only costs idle work-groups).  Only pool entries of the prefix are read,
 * so kvb_write_kv of the same chunk may run before or after this call.
 * workspace: (device, optional) NULL, or at least kvb_paged_prefill_workspace_size(...)
 * bytes, 16-byte aligned (else KVB_ERR_WORKSPACE / KVB_ERR_INVALID).  With it, a grid
 * of several rounds of work-groups is started longest first (a small plan kernel sorts
 * each XCD's work items by the key count of their sequence, prefix plus chunk, into the
 * workspace first), which shortens the tail on ragged batches; the results are the same
 * bits either way.  Its contents on entry do not matter. */
kvb_status kvb_paged_prefill(const kvb_pool* pool, const void* q, const void* k_new,
                             const void* v_new, void* out, const int32_t* cu_q_lens,
                             const int32_t* prefix_lens, const int32_t* block_tables,
                             int32_t block_table_stride, int32_t batch, int32_t num_q_heads,
                             int32_t total_q, int32_t max_q_len, int32_t max_prefix_len,
                             float scale, void* workspace, size_t workspace_bytes, void* stream);

/* kvb_paged_prefill and kvb_write_kv of the same chunk in one launch: the same output, and
 * the chunk's K/V rows written into the pool at slot_mapping[t] as kvb_write_kv writes them
 * (kvboost 0.6.0, "How it works" step 5: the live suffix's KV is stored for reuse while the
 * suffix is computed; kvstream 0.1.0, "Request lifecycle" step 2: one slot per token).
 * Each token is written by the work-group that holds its first query row, after that
 * work-group's attention work, so every row is written once.
 * slot_mapping: (device) int64 [total_q], 8-byte aligned; slot = block*16 + row; a negative
 * slot or one at or past num_blocks*16 skips the token, as in kvb_write_kv.  The slots must
 * not lie in rows this call reads as prefix (rows below prefix_lens[b] of the table's
 * blocks) nor repeat within the call.  Other arguments, errors and the workspace as
 * kvb_paged_prefill (KVB_ERR_NULL also for a missing slot_mapping). */
kvb_status kvb_paged_prefill_write(const kvb_pool* pool, const void* q, const void* k_new,
                                   const void* v_new, void* out, const int64_t* slot_mapping,
                                   const int32_t* cu_q_lens, const int32_t* prefix_lens,
                                   const int32_t* block_tables, int32_t block_table_stride,
                                   int32_t batch, int32_t num_q_heads, int32_t total_q,
                                   int32_t max_q_len, int32_t max_prefix_len, float scale,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* Paged prefill with every key read from the pool: the same result as kvb_paged_prefill,
 * but the chunk's own K/V is read back through the block table (positions
 * prefix_lens[b] .. prefix_lens[b] + C_b - 1 of sequence b), after kvb_write_kv has put it
 * there, so cached and new keys take one path (kvboost 0.6.0, "How it works" steps 3 and
 * 5: the chunk attends to the cached prefix and to itself in one pass).
 * block_tables: (device) int32 [batch][block_table_stride]; row b must cover
 * prefix_lens[b] + C_b tokens (keys past block_table_stride*16 are never read), and
 * block_table_stride >= ceil(max_prefix_len/16).  Other arguments as kvb_paged_prefill;
 * no workspace. */
kvb_status kvb_paged_prefill_pooled(const kvb_pool* pool, const void* q, void* out,
                                    const int32_t* cu_q_lens, const int32_t* prefix_lens,
                                    const int32_t* block_tables, int32_t block_table_stride,
                                    int32_t batch, int32_t num_q_heads, int32_t total_q,
                                    int32_t max_q_len, int32_t max_prefix_len, float scale,
                                    void* stream);

/* Paged decode: one query per sequence over its whole context, which is already in the
 * pool (kvstream 0.1.0, "Request lifecycle" step 2; kvboost 0.6.0, "CPU paged attention":
 * only the decode loop changes).  The query of sequence b sits at position
 * context_lens[b]-1 and sees keys 0..context_lens[b]-1 through its block table.  For
 * batches of up to 1024 sequences the (KV head, sequence, block) list of the whole batch
 * is cut into equal ranges, one per wave of a grid that is resident at once; a sequence
 * whose blocks fall into several ranges has partial results (unnormalised output, running
 * max, sum) merged by log-sum-exp.  split_blocks > 0 fixes the blocks each wave takes
 * (values above 64 count as 64); 0 balances the ranges over the device.  Larger batches
 * split each sequence into groups of split_blocks blocks (0: a size from the host bounds).
 * A context length <= 0 gives a zero output row.
 * q, out: (device) [batch][num_q_heads][head_dim]; context_lens: (device) int32 [batch]
 * <= max_context_len; block_tables: (device) int32 [batch][block_table_stride] with
 * block_table_stride >= ceil(max_context_len/16).
 * workspace: (device) at least kvb_paged_decode_workspace_size(...) bytes for the same
 * batch, num_q_heads, head_dim, max_context_len and split_blocks. */
kvb_status kvb_paged_decode(const kvb_pool* pool, const void* q, void* out,
                            const int32_t* context_lens, const int32_t* block_tables,
                            int32_t block_table_stride, int32_t batch, int32_t num_q_heads,
                            int32_t max_context_len, int32_t split_blocks, float scale,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Allocation-free paged decode, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * kernels, split plan and result bits as kvb_paged_decode, with the workspace (split
 * partials and the plan's header) kept in a static device array of
 * KVB_NOALLOC_SCRATCH_BYTES bytes inside the library instead of a caller workspace.  Each GPU the library runs on holds its own copy of that array from
 * the first call on it until the process ends; that first call on a device also looks up
 * the array's address (no allocation call is made by this entry point at any time).
 * Every call on one GPU shares the array and it keeps the last call's contents (nothing in
 * it needs clearing: every partial the merge reads is written by the same call), so calls
 * that overlap on one GPU (different streams, or threads) race and must be serialised by
 * the caller.  A call whose plan needs more than KVB_NOALLOC_SCRATCH_BYTES
 * (kvb_paged_decode_workspace_size for the same arguments) returns KVB_ERR_TOO_LARGE and
 * launches nothing.  Arguments, layouts and the other errors as kvb_paged_decode. */
#define KVB_NOALLOC_SCRATCH_BYTES (16u << 20)
kvb_status kvb_paged_decode_noalloc(const kvb_pool* pool, const void* q, void* out,
                                    const int32_t* context_lens, const int32_t* block_tables,
                                    int32_t block_table_stride, int32_t batch, int32_t num_q_heads,
                                    int32_t max_context_len, int32_t split_blocks, float scale,
                                    void* stream);

/* Shared-prefix (cascade) decode: the same result as kvb_paged_decode, but the first
 * shared_len tokens of every sequence are one shared prefix, read once for all sequences'
 * queries instead of once per sequence (kvboost 0.6.0, "How batching works" step 4: a
 * shared prefix's KV is loaded once and broadcast across the batch).  Logical block
 * j < shared_len/16 of every sequence is shared_blocks[j]; those entries of block_tables
 * are not read.  A sequence with context_lens[b] < shared_len sees only its first
 * context_lens[b] tokens.  The shared part runs as one tiled pass over all queries of
 * each KV head (split over key tiles), the rest as the split decode, and every partial
 * (unnormalised output, max, sum) is merged by log-sum-exp.
 * shared_blocks: (device) int32 [ceil(shared_len/16)], may be NULL when shared_len == 0;
 * shared_len: a multiple of 16, >= 0.  Other arguments as kvb_paged_decode.
 * workspace: (device, required) at least kvb_paged_decode_cascade_workspace_size(...) bytes
 * for the same batch, heads, head_dim, max_context_len, shared_len and split_blocks. */
kvb_status kvb_paged_decode_cascade(const kvb_pool* pool, const void* q, void* out,
                                    const int32_t* context_lens, const int32_t* block_tables,
                                    int32_t block_table_stride, const int32_t* shared_blocks,
                                    int32_t shared_len, int32_t batch, int32_t num_q_heads,
                                    int32_t max_context_len, int32_t split_blocks, float scale,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* Workspace sizes in bytes (0 = none needed).  Host arithmetic on the arguments and the
 * current device's compute-unit count (the decode plan sizes its grid to the device), so a
 * size holds for the device that is current when it is queried; call the size query and
 * the decode with the same device current.  The
 * decode sizes take num_kv_heads too: the split plan counts (sequence, KV head) units;
 * they are 0 only for an empty batch or invalid arguments (max_context_len 0, every
 * context empty, still takes the plan's workspace: the call writes the zero rows). */
size_t kvb_paged_prefill_workspace_size(int32_t batch, int32_t num_q_heads, int32_t head_dim,
                                        int32_t total_q, int32_t max_prefix_len);
size_t kvb_paged_decode_workspace_size(int32_t batch, int32_t num_kv_heads, int32_t num_q_heads,
                                       int32_t head_dim, int32_t max_context_len,
                                       int32_t split_blocks);
size_t kvb_paged_decode_cascade_workspace_size(int32_t batch, int32_t num_kv_heads,
                                               int32_t num_q_heads, int32_t head_dim,
                                               int32_t max_context_len, int32_t shared_len,
                                               int32_t split_blocks);

/* Block copies between pools (kvboost 0.6.0, "CPU paged attention": shared prefixes share
 * physical blocks copy-on-write, so a sequence about to write into a shared block first
 * copies it; kvstream 0.1.0, "Why KVStream?": low-priority sequences are swapped to a CPU
 * page pool).  For i < n: block dst_ids[i] of dst (K and V, every head) becomes a copy of
 * block src_ids[i] of src, bit-exact.  src and dst may be the same pool, or one of them a
 * pool in pinned host memory that the device can address (swap out / in).  Both pools need
 * the same num_kv_heads, head_dim and dtype; block_stride may differ.  Pool memory the
 * device cannot address (pageable host memory) gives KVB_ERR_INVALID; pinned host memory
 * is used through its device-mapped address.  Pairs with an id outside its pool are skipped.  Destination blocks must be distinct and, within one pool,
 * not also sources of the same call (copies run concurrently).
 * src_ids, dst_ids: (device) int32 [n]. */
kvb_status kvb_copy_blocks(const kvb_pool* src, const kvb_pool* dst, const int32_t* src_ids,
                           const int32_t* dst_ids, int32_t n, void* stream);

/* 8-bit K/V pool (kvboost 0.6.0, "Optional: KV quantization": cached K is stored at
 * per-channel scales and V at per-token scales, about half the bytes of a 16-bit pool).
 * A code c (int8, -127..127) stands for the value c * scale.
 *   k, v (device, int8): code (block, kv_head, row, e) at
 *       block*block_stride + (kv_head*16 + row)*head_dim + e            (bytes)
 *   v_scale (device, float32): scale of token (block, kv_head, row) at
 *       (block*num_kv_heads + kv_head)*16 + row; written by kvb_write_kv_q8
 *   k_scale (device, float32): the pool's K scale of channel (kv_head, e) at
 *       kv_head*head_dim + e; chosen by the caller (for instance max |k| over the prompt's
 *       tokens / 127), finite and >= 0; read by every call, changed by none.
 * block_stride (bytes) >= num_kv_heads*16*head_dim, a multiple of 16, below 2^31. */
typedef struct {
  void*        k;             /* (device) K codes                                */
  void*        v;             /* (device) V codes                                */
  float*       v_scale;       /* (device) per-token V scales                     */
  const float* k_scale;       /* (device) per-channel K scales                   */
  int64_t      block_stride;  /* bytes between consecutive physical blocks       */
  int32_t      num_blocks;    /* physical blocks in the pool (> 0)               */
  int32_t      block_size;    /* must be 16                                      */
  int32_t      num_kv_heads;  /* > 0                                             */
  int32_t      head_dim;      /* 64, 96 or 128                                   */
} kvb_pool_q8;

/* Quantising slot scatter: kvb_write_kv's slot rule, each token coded on the way in.
 * For token t with an in-pool slot, kv head h, channel e (x taken exactly as float32):
 *   K code = rint(k_new[t][h][e] / k_scale[h][e]) clamped to [-127, 127] (0 where the
 *   scale is 0); V scale s = max_e |v_new[t][h][e]| / 127, stored in v_scale; V code =
 *   rint(v_new[t][h][e] / s) (0 where s is 0).  Divisions are IEEE float32, rint rounds
 *   half to even.  k_new, v_new: (device) [num_tokens][num_kv_heads][head_dim] in `dtype`
 *   (a kvb_dtype).  slot_mapping: (device) int64 [num_tokens]. */
kvb_status kvb_write_kv_q8(const kvb_pool_q8* pool, const void* k_new, const void* v_new,
                           int32_t dtype, const int64_t* slot_mapping, int32_t num_tokens,
                           void* stream);

/* Paged decode over the 8-bit pool: kvb_paged_decode with every key and value read as
 * the value its code stands for.  q, out: (device) [batch][num_q_heads][head_dim] in
 * `dtype`.  workspace: kvb_paged_decode_workspace_size(...) bytes for the same batch,
 * heads, head_dim, max_context_len and split_blocks (the same split plan).  Other
 * arguments as kvb_paged_decode. */
kvb_status kvb_paged_decode_q8(const kvb_pool_q8* pool, int32_t dtype, const void* q, void* out,
                               const int32_t* context_lens, const int32_t* block_tables,
                               int32_t block_table_stride, int32_t batch, int32_t num_q_heads,
                               int32_t max_context_len, int32_t split_blocks, float scale,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Paged prefill over the 8-bit pool: kvb_paged_prefill with the cached prefix read as the
 * values its codes stand for (the chunk's own K/V are the call's 16-bit rows).  The
 * codes of each prefix block are staged in LDS and widened there to 16 bits (V times its
 * token's scale, rounded to nearest even; the K channel scales are folded into the
 * queries), so no widened copy of the prefix is written anywhere.  q, k_new, v_new, out
 * in `dtype`.  workspace: (device, optional) NULL (no dispatch plan), or at least
 * kvb_paged_prefill_q8_workspace_size(...) bytes (the dispatch plan, as for
 * kvb_paged_prefill; independent of the prefix lengths); contents on entry do not
 * matter.  Other arguments as kvb_paged_prefill. */
kvb_status kvb_paged_prefill_q8(const kvb_pool_q8* pool, int32_t dtype, const void* q,
                                const void* k_new, const void* v_new, void* out,
                                const int32_t* cu_q_lens, const int32_t* prefix_lens,
                                const int32_t* block_tables, int32_t block_table_stride,
                                int32_t batch, int32_t num_q_heads, int32_t total_q,
                                int32_t max_q_len, int32_t max_prefix_len, float scale,
                                void* workspace, size_t workspace_bytes, void* stream);
size_t kvb_paged_prefill_q8_workspace_size(int32_t batch, int32_t num_kv_heads,
                                           int32_t num_q_heads, int32_t head_dim,
                                           int32_t total_q, int32_t max_prefix_len);

/* 4-bit K/V pool (kvboost 0.6.0, "Optional: KV quantization": kv_cache_bits=4).  The
 * 8-bit pool's rules with codes in [-7, 7] (V scale max |v| / 7; K scales chosen by the
 * caller, for instance max |k| / 7) and two codes per byte: channel 2i in the low nibble,
 * 2i+1 in the high nibble, each a 4-bit two's complement.  The fields are kvb_pool_q8's,
 * with k and v (device) holding code bytes (block, kv_head, row, e/2) at
 *   block*block_stride + ((kv_head*16 + row)*head_dim + e)/2
 * and block_stride (bytes) >= num_kv_heads*16*head_dim/2, a multiple of 16. */
typedef kvb_pool_q8 kvb_pool_q4;

/* As kvb_write_kv_q8, kvb_paged_decode_q8 and kvb_paged_prefill_q8 for the 4-bit pool
 * (decode: the same workspace as kvb_paged_decode; prefill:
 * kvb_paged_prefill_q8_workspace_size(...) bytes). */
kvb_status kvb_write_kv_q4(const kvb_pool_q4* pool, const void* k_new, const void* v_new,
                           int32_t dtype, const int64_t* slot_mapping, int32_t num_tokens,
                           void* stream);
kvb_status kvb_paged_decode_q4(const kvb_pool_q4* pool, int32_t dtype, const void* q, void* out,
                               const int32_t* context_lens, const int32_t* block_tables,
                               int32_t block_table_stride, int32_t batch, int32_t num_q_heads,
                               int32_t max_context_len, int32_t split_blocks, float scale,
                               void* workspace, size_t workspace_bytes, void* stream);
kvb_status kvb_paged_prefill_q4(const kvb_pool_q4* pool, int32_t dtype, const void* q,
                                const void* k_new, const void* v_new, void* out,
                                const int32_t* cu_q_lens, const int32_t* prefix_lens,
                                const int32_t* block_tables, int32_t block_table_stride,
                                int32_t batch, int32_t num_q_heads, int32_t total_q,
                                int32_t max_q_len, int32_t max_prefix_len, float scale,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Test helper: gather through the block tables into a contiguous layout, bit-exact.
 * For b < batch, j < seq_lens[b]:
 *   k_out[cu_seq_lens[b] + j][h][:] = pool.k[block_tables[b*stride + j/16]][h][j%16][:]
 * (same for v).  k_out, v_out: (device) [cu_seq_lens[batch]][num_kv_heads][head_dim];
 * seq_lens, cu_seq_lens: (device) int32; max_len >= every seq_lens[b].  Rows of keys in
 * blocks outside the pool are left untouched. */
kvb_status kvb_gather_kv(const kvb_pool* pool, const int32_t* block_tables,
                         int32_t block_table_stride, const int32_t* seq_lens,
                         const int32_t* cu_seq_lens, void* k_out, void* v_out, int32_t batch,
                         int32_t max_len, void* stream);

/* Static string for a status code. */
const char* kvb_status_str(kvb_status s);

/* Library version, e.g. "0.1.0". */
const char* kvb_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KVB_H */
