"""Seeded synthetic inputs shaped like the pages' workloads.

Everything here is input preparation: lengths, physical block placement,
per-sequence block tables, slot mappings and N(0,1) values rounded (round to
nearest even) to fp16/bf16 payloads.  No attention arithmetic lives here.

Pool layout (both K and V): ``[num_blocks][num_kv_heads][16][head_dim]`` of
16-bit payloads, one (block, kv-head) tile being a contiguous 16 x head_dim run.
The block pool of fixed 16-token blocks follows kvboost 0.6.0, section "CPU
paged attention"; one page holding block_size x heads x head_dim x 2 x
dtype_bytes follows kvstream 0.1.0, section "Configuration".

Draw order for a seed (kept fixed so the published statistics stay valid):
lengths, then ``perm = rng.permutation(num_blocks)``, then (pair sharing only)
``pairing = rng.permutation(batch)``, then values: pool K for every used prefix
block in placement order, pool V likewise, then q, k_new, v_new, and last the
optional decode-step tensors.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

BLOCK = 16
NAN_BITS = {"fp16": np.uint16(0x7E00), "bf16": np.uint16(0x7FC0)}


def blocks_for(tokens: int) -> int:
    """Blocks needed to hold ``tokens`` tokens: full blocks plus one for a tail."""
    return (int(tokens) + BLOCK - 1) // BLOCK


def round_to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to 16-bit payloads (round to nearest, ties to even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "fp16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        u = x.view(np.uint32).astype(np.uint64)
        r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        return r.astype(np.uint16)
    raise ValueError(dtype)


@dataclass
class Workload:
    name: str
    seed: int
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    num_blocks: int
    scale: float
    kind: str                      # "prefill" or "decode"
    # pool (uint16 payloads) [num_blocks][Hkv][16][d]
    k_pool: np.ndarray
    v_pool: np.ndarray
    block_tables: np.ndarray       # int32 [B][stride]
    # prefill fields
    prefix_lens: np.ndarray        # int32 [B]
    q_lens: np.ndarray             # int32 [B]
    cu_q_lens: np.ndarray          # int32 [B+1]
    q: np.ndarray                  # uint16 [T][Hq][d] (prefill) or [B][Hq][d] (decode)
    k_new: Optional[np.ndarray]    # uint16 [T][Hkv][d]
    v_new: Optional[np.ndarray]
    slot_mapping: Optional[np.ndarray]  # int64 [T]
    # decode fields
    context_lens: Optional[np.ndarray] = None  # int32 [B]
    # decode step following a prefill (optional)
    dec_q: Optional[np.ndarray] = None
    dec_k: Optional[np.ndarray] = None
    dec_v: Optional[np.ndarray] = None
    dec_slots: Optional[np.ndarray] = None
    dec_context_lens: Optional[np.ndarray] = None
    poison_block: int = -1
    shared_fraction: float = 0.0
    notes: Dict[str, object] = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.block_tables.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.cu_q_lens[-1]) if self.kind == "prefill" else self.batch

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


def _assign_blocks(nblocks: Sequence[int], groups: Sequence[Tuple[Sequence[int], int]],
                   perm: np.ndarray):
    """Map every sequence's logical blocks to physical blocks.

    ``groups`` lists (members, n): the members' logical blocks 0..n-1 (as far as
    each member has them) share n physical blocks.  Physical ids are consumed
    from ``perm`` in order: shared groups first, then each sequence's private
    blocks in sequence and logical order.
    """
    B = len(nblocks)
    table: List[List[int]] = [[-1] * int(n) for n in nblocks]
    order: List[int] = []              # physical blocks in placement order
    cur = 0
    for members, n in groups:
        ids = [int(x) for x in perm[cur:cur + n]]
        cur += n
        order.extend(ids)
        for b in members:
            for j in range(min(n, nblocks[b])):
                table[b][j] = ids[j]
    for b in range(B):
        for j in range(nblocks[b]):
            if table[b][j] < 0:
                if cur >= len(perm):
                    raise ValueError("pool too small for the workload")
                table[b][j] = int(perm[cur])
                order.append(int(perm[cur]))
                cur += 1
    return table, order, cur


def _build(name, seed, dtype, Hq, Hkv, d, num_blocks, prefix_lens, q_lens,
           groups_fn, kind, rng, with_decode=False, poison=False, pairing_draw=False,
           stride_extra=0):
    B = len(prefix_lens)
    perm = rng.permutation(num_blocks)
    pairing = rng.permutation(B) if pairing_draw else None
    groups = groups_fn(pairing)
    if kind == "prefill":
        ctx_tokens = [int(p) + int(c) + (1 if with_decode else 0) for p, c in zip(prefix_lens, q_lens)]
        filled_tokens = [int(p) for p in prefix_lens]
    else:
        ctx_tokens = [int(p) for p in prefix_lens]      # context lengths
        filled_tokens = ctx_tokens
    nblocks = [blocks_for(t) for t in ctx_tokens]
    table, order, used = _assign_blocks(nblocks, groups, perm)
    poison_block = int(perm[used]) if used < num_blocks else -1
    stride = max(max(nblocks) if nblocks else 1, 1) + stride_extra
    bt = np.full((B, stride), poison_block if poison_block >= 0 else 0, dtype=np.int32)
    for b in range(B):
        bt[b, :len(table[b])] = table[b]

    # Physical blocks that hold cached tokens, in placement order, each once,
    # with the number of leading slots that hold a valid token for some sequence.
    valid: Dict[int, int] = {}
    for b in range(B):
        for j in range(blocks_for(filled_tokens[b])):
            pb = table[b][j]
            valid[pb] = max(valid.get(pb, 0), min(BLOCK, filled_tokens[b] - BLOCK * j))
    fill_set = [pb for pb in order if pb in valid]

    shape_blk = (Hkv, BLOCK, d)
    k_pool = np.zeros((num_blocks,) + shape_blk, dtype=np.uint16)
    v_pool = np.zeros((num_blocks,) + shape_blk, dtype=np.uint16)
    nf = len(fill_set)
    kv = rng.standard_normal(size=(nf,) + shape_blk, dtype=np.float32)
    vv = rng.standard_normal(size=(nf,) + shape_blk, dtype=np.float32)
    if nf:
        idx = np.asarray(fill_set, dtype=np.int64)
        k_pool[idx] = round_to_bits(kv, dtype)
        v_pool[idx] = round_to_bits(vv, dtype)
    del kv, vv

    if poison:
        nanb = NAN_BITS[dtype]
        mask = np.ones(num_blocks, dtype=bool)
        mask[np.asarray(fill_set, dtype=np.int64)] = False
        k_pool[mask] = nanb
        v_pool[mask] = nanb
        for pb, n in valid.items():
            if n < BLOCK:
                k_pool[pb, :, n:, :] = nanb
                v_pool[pb, :, n:, :] = nanb

    scale = 1.0 / float(np.sqrt(d))
    pl = np.asarray(prefix_lens, dtype=np.int32)
    if kind == "prefill":
        ql = np.asarray(q_lens, dtype=np.int32)
        cu = np.zeros(B + 1, dtype=np.int32)
        cu[1:] = np.cumsum(ql)
        T = int(cu[-1])
        q = round_to_bits(rng.standard_normal(size=(T, Hq, d), dtype=np.float32), dtype)
        k_new = round_to_bits(rng.standard_normal(size=(T, Hkv, d), dtype=np.float32), dtype)
        v_new = round_to_bits(rng.standard_normal(size=(T, Hkv, d), dtype=np.float32), dtype)
        slots = np.empty(T, dtype=np.int64)
        for b in range(B):
            for i in range(int(ql[b])):
                pos = int(pl[b]) + i
                slots[cu[b] + i] = int(table[b][pos // BLOCK]) * BLOCK + pos % BLOCK
        w = Workload(name, seed, dtype, Hq, Hkv, d, num_blocks, scale, "prefill", k_pool, v_pool,
                     bt, pl, ql, cu, q, k_new, v_new, slots, poison_block=poison_block)
        if with_decode:
            w.dec_q = round_to_bits(rng.standard_normal(size=(B, Hq, d), dtype=np.float32), dtype)
            w.dec_k = round_to_bits(rng.standard_normal(size=(B, Hkv, d), dtype=np.float32), dtype)
            w.dec_v = round_to_bits(rng.standard_normal(size=(B, Hkv, d), dtype=np.float32), dtype)
            w.dec_context_lens = (pl + ql + 1).astype(np.int32)
            ds = np.empty(B, dtype=np.int64)
            for b in range(B):
                pos = int(pl[b] + ql[b])
                ds[b] = int(table[b][pos // BLOCK]) * BLOCK + pos % BLOCK
            w.dec_slots = ds
    else:
        q = round_to_bits(rng.standard_normal(size=(B, Hq, d), dtype=np.float32), dtype)
        zeros = np.zeros(B, dtype=np.int32)
        w = Workload(name, seed, dtype, Hq, Hkv, d, num_blocks, scale, "decode", k_pool, v_pool,
                     bt, zeros, zeros, np.zeros(B + 1, dtype=np.int32), q, None, None, None,
                     context_lens=pl.copy(), poison_block=poison_block)
    # achieved sharing: fraction of prefix-block references that hit a shared block
    refs = 0
    shared_refs = 0
    counts: Dict[int, int] = {}
    for b in range(B):
        for j in range(blocks_for(filled_tokens[b])):
            counts[table[b][j]] = counts.get(table[b][j], 0) + 1
    for b in range(B):
        for j in range(blocks_for(filled_tokens[b])):
            refs += 1
            shared_refs += counts[table[b][j]] > 1
    w.shared_fraction = shared_refs / refs if refs else 0.0
    w.notes["unique_blocks"] = len(counts)
    # physical blocks of the first sharing group (placed first: perm[0:n]), for callers
    # that pass a shared prefix as a block list
    if groups:
        w.notes["first_group"] = (list(groups[0][0]), [int(x) for x in perm[:groups[0][1]]])
    return w


def _pair_groups(prefix_lens):
    def fn(pairing):
        groups = []
        n = [int(p) // BLOCK for p in prefix_lens]
        for k in range(0, len(pairing) - 1, 2):
            a, b = int(pairing[k]), int(pairing[k + 1])
            s = min(n[a], n[b], int(round((n[a] + n[b]) / 4)))
            if s > 0:
                groups.append(([a, b], s))
        return groups
    return fn


CONFIGS = {
    # Tiny paged prefill: one sequence, 32-token prefix in 2 blocks, 16-token chunk.
    "tiny": dict(seed=1),
    # 8 sequences on one shared 2048-token prefix, 256-token chunks each, GQA 16/2.
    "shared_prompt": dict(seed=2),
    # 64 decode queries, contexts U{512..4096}, first 1024 tokens shared.
    "decode": dict(seed=3),
    # 4 sequences, 8192-token prefix, 1024-token chunk, 40/8 heads.
    "long_prefix": dict(seed=4),
    # Ragged multi-turn mix at head_dim 96 fp16 and head_dim 64 bf16.
    "ragged_d96": dict(seed=5),
    "ragged_d64": dict(seed=6),
}


def make_config(name: str, seed: Optional[int] = None, poison: bool = False,
                with_decode: bool = False) -> Workload:
    seed = CONFIGS[name]["seed"] if seed is None else seed
    rng = np.random.default_rng(seed)
    if name == "tiny":
        return _build(name, seed, "fp16", 1, 1, 64, 8, [32], [16], lambda p: [], "prefill", rng,
                      with_decode=with_decode, poison=poison)
    if name == "shared_prompt":
        B = 8
        return _build(name, seed, "bf16", 16, 2, 128, 8192, [2048] * B, [256] * B,
                      lambda p: [(list(range(B)), 2048 // BLOCK)], "prefill", rng,
                      with_decode=with_decode, poison=poison)
    if name == "decode":
        B = 64
        ctx = rng.integers(512, 4097, size=B)
        return _build(name, seed, "bf16", 32, 8, 128, 16384, [int(c) for c in ctx], [0] * B,
                      lambda p: [(list(range(B)), 1024 // BLOCK)], "decode", rng, poison=poison)
    if name == "long_prefix":
        B = 4
        return _build(name, seed, "fp16", 40, 8, 128, 8192, [8192] * B, [1024] * B,
                      lambda p: [], "prefill", rng, with_decode=with_decode, poison=poison)
    if name in ("ragged_d96", "ragged_d64"):
        B = 32
        P = rng.integers(0, 16385, size=B)
        cand = np.array([c for c in range(1, 513) if c % BLOCK])
        C = rng.choice(cand, size=B)
        dtype, d = ("fp16", 96) if name == "ragged_d96" else ("bf16", 64)
        return _build(name, seed, dtype, 32, 8, d, 32768, [int(x) for x in P], [int(x) for x in C],
                      _pair_groups([int(x) for x in P]), "prefill", rng,
                      with_decode=with_decode, poison=poison, pairing_draw=True)
    raise KeyError(name)


def make_custom(seed: int, dtype: str, num_q_heads: int, num_kv_heads: int, head_dim: int,
                prefix_lens: Sequence[int], q_lens: Sequence[int] = (), num_blocks: Optional[int] = None,
                kind: str = "prefill", share: str = "none", poison: bool = True,
                with_decode: bool = False, stride_extra: int = 0) -> Workload:
    """Small workloads for parity tests.

    ``share``: "none", "all" (every sequence shares the full blocks of the
    shortest prefix), "pairs" (random pairs share leading full blocks) or "first:N"
    (every sequence's first N blocks, as far as it has them, are shared).
    For ``kind="decode"`` ``prefix_lens`` are the context lengths.
    """
    rng = np.random.default_rng(seed)
    B = len(prefix_lens)
    if kind == "prefill":
        ctx = [int(p) + int(c) + (1 if with_decode else 0) for p, c in zip(prefix_lens, q_lens)]
    else:
        ctx = [int(p) for p in prefix_lens]
        q_lens = [0] * B
    need = sum(blocks_for(t) for t in ctx) + 1
    if share.startswith("first:"):
        need += int(share.split(":")[1])
    if num_blocks is None:
        num_blocks = need + 3
    if share == "all":
        nmin = min(int(p) for p in prefix_lens) // BLOCK if kind == "prefill" else \
            min(int(p) for p in prefix_lens) // BLOCK
        groups_fn = (lambda p: [(list(range(B)), nmin)]) if nmin > 0 else (lambda p: [])
    elif share == "pairs":
        groups_fn = _pair_groups([int(p) for p in prefix_lens])
    elif share.startswith("first:"):
        # every sequence's logical blocks 0..n-1 (as far as it has them) are the same
        # n physical blocks, whatever its length
        n_first = int(share.split(":")[1])
        groups_fn = lambda p: [(list(range(B)), n_first)]
    else:
        groups_fn = lambda p: []
    return _build(f"custom{seed}", seed, dtype, num_q_heads, num_kv_heads, head_dim, num_blocks,
                  list(prefix_lens), list(q_lens), groups_fn, kind, rng, with_decode=with_decode,
                  poison=poison, pairing_draw=(share == "pairs"), stride_extra=stride_extra)


def make(name: str, **kw) -> Workload:
    return make_config(name, **kw)


def channel_scales(k_tokens: np.ndarray, code_max: int = 127) -> np.ndarray:
    """Input choice for a quantised pool: a K scale per (KV head, channel) from example
    tokens ``[n][Hkv][d]`` (float32), the largest |k| over the tokens divided by the
    largest code (127 for 8-bit codes, 7 for 4-bit ones), in float32."""
    a = np.abs(np.asarray(k_tokens, dtype=np.float32)).max(axis=0)
    return np.divide(a, np.float32(code_max), dtype=np.float32)
