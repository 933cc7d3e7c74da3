"""Plain fp64 definitions of slot scatter, block-table gather and paged attention.

Test infrastructure only (see the package docstring).  Each function names the
passage of the pages it follows.  Pool arrays are 16-bit payloads shaped
``[num_blocks][num_kv_heads][16][head_dim]``; block tables are int32
``[batch][stride]``.
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

BLOCK_SIZE = 16  # tokens per physical block (kvboost 0.6.0, "CPU paged attention")


def decode_bits(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of fp16 / bf16 payloads (the two input dtypes named in
    kvboost 0.6.0, "Flash Attention (CUDA)", supported-properties table)."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def write_kv(k_pool: np.ndarray, v_pool: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
             slot_mapping: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Scatter each new token's K/V into its pool slot; slots that name no row of the
    pool (negative, or at or past ``num_blocks * 16``) are skipped.

    One slot per token in a fixed pool of pages (kvstream 0.1.0, "Why KVStream?",
    streaming KV allocation; "Request lifecycle" step 2).  A slot names physical
    block ``slot // 16`` and row ``slot % 16`` inside it; the pool is fixed, so a
    slot outside it names no page at all.  Returns new arrays.
    """
    kp = np.array(k_pool, copy=True)
    vp = np.array(v_pool, copy=True)
    n_slots = kp.shape[0] * BLOCK_SIZE
    for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0 or slot >= n_slots:
            continue
        blk, row = int(slot) // BLOCK_SIZE, int(slot) % BLOCK_SIZE
        kp[blk, :, row, :] = k_new[t]
        vp[blk, :, row, :] = v_new[t]
    return kp, vp


def copy_blocks(src_k: np.ndarray, src_v: np.ndarray, dst_k: np.ndarray, dst_v: np.ndarray,
                src_ids: Sequence[int], dst_ids: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """Whole-block copies between two pools of the same shape.

    A sequence about to write into a physical block it shares copy-on-write first
    gets a private copy of it (kvboost 0.6.0, "CPU paged attention"; kvstream 0.1.0,
    "Request lifecycle" step 3), and low-priority sequences are spilled to a CPU page
    pool and brought back (kvstream 0.1.0, "Why KVStream?", swap & preemption).  Block
    ``dst_ids[i]`` becomes block ``src_ids[i]`` (every head, every row); a pair with an
    id outside its pool is skipped.  Returns new destination arrays.
    """
    dk = np.array(dst_k, copy=True)
    dv = np.array(dst_v, copy=True)
    for s_id, d_id in zip(np.asarray(src_ids, dtype=np.int64), np.asarray(dst_ids, dtype=np.int64)):
        if not (0 <= s_id < src_k.shape[0] and 0 <= d_id < dk.shape[0]):
            continue
        dk[d_id] = src_k[s_id]
        dv[d_id] = src_v[s_id]
    return dk, dv


def gather_kv(pool: np.ndarray, table_row: np.ndarray, n_tokens: int) -> np.ndarray:
    """Logical tokens 0..n_tokens-1 of one sequence, gathered through its block table.

    Logical token j lives in physical block ``table_row[j // 16]`` at row ``j % 16``
    (kvstream 0.1.0, "Request lifecycle" step 3: the block table maps a sequence
    onto pool pages, possibly shared).  Returns ``[n_tokens][num_kv_heads][d]``.
    """
    n_tokens = int(n_tokens)
    if n_tokens == 0:
        return pool[:0, :, 0, :].copy()
    j = np.arange(n_tokens)
    blocks = np.asarray(table_row, dtype=np.int64)[j // BLOCK_SIZE]
    return pool[blocks, :, j % BLOCK_SIZE, :]


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, positions: Sequence[int], scale: float,
           keys: Optional[np.ndarray] = None, want_weights: bool = False):
    """Softmax attention of query rows over a logically contiguous key sequence.

    ``q``: ``[rows][d]``, ``K``/``V``: ``[L][d]`` (float64).  Row r sees key j iff
    ``j <= positions[r]`` (causal; kvboost 0.6.0, "Flash Attention (CUDA)",
    causal masking) and, when ``keys`` is given, only keys in that index set.
    The whole score matrix is materialised.  Returns (out ``[rows][d]``,
    lse ``[rows]``) and the weights if asked.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    L = K.shape[0]
    s = (q @ K.T) * float(scale)                       # [rows][L]
    visible = np.arange(L)[None, :] <= np.asarray(positions)[:, None]
    if keys is not None:
        sel = np.zeros(L, dtype=bool)
        sel[np.asarray(keys, dtype=np.int64)] = True
        visible &= sel[None, :]
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    empty = ~np.isfinite(m[:, 0])
    m = np.where(np.isfinite(m), m, 0.0)
    w = np.where(visible, np.exp(s - m), 0.0)
    den = w.sum(axis=1, keepdims=True)
    safe = np.where(den > 0, den, 1.0)
    out = (w @ V) / safe
    out[empty] = 0.0
    lse = np.where(empty, -np.inf, m[:, 0] + np.log(safe[:, 0]))
    if want_weights:
        return out, lse, w / safe
    return out, lse


def _sequence_kv(k_pool, v_pool, table_row, prefix_len, k_self, v_self, dtype):
    """Cached prefix from the pool followed by the chunk's own K/V, as float64
    ``[L][Hkv][d]`` (kvboost 0.6.0, "How it works", step 3: cached prefix plus live
    suffix, and step 5: both go through one forward pass)."""
    Kp = decode_bits(gather_kv(k_pool, table_row, prefix_len), dtype)
    Vp = decode_bits(gather_kv(v_pool, table_row, prefix_len), dtype)
    Ks = decode_bits(k_self, dtype)
    Vs = decode_bits(v_self, dtype)
    return np.concatenate([Kp, Ks], axis=0), np.concatenate([Vp, Vs], axis=0)


def paged_prefill(k_pool, v_pool, q, k_new, v_new, cu_q_lens, prefix_lens, block_tables,
                  num_q_heads: int, scale: float, dtype: str,
                  select: Optional[Iterable[Tuple[int, int, Sequence[int]]]] = None,
                  want_lse: bool = False):
    """Chunk rows attending to their cached prefix (through the block table) and
    causally to the chunk itself.

    Row i of sequence b sits at position ``P_b + i`` and sees keys ``0..P_b+i``: the
    whole cached prefix and chunk tokens ``0..i``.  Query head h reads KV head
    ``h // (num_q_heads // num_kv_heads)`` (grouped-query heads in contiguous
    groups).  Passages: kvboost 0.6.0, "How it works" steps 3 and 5; "Flash
    Attention (CUDA)", causal masking; "CPU paged attention" for the pool.

    ``select``: optional list of (b, h, rows) to compute only those rows; returns a
    dict {(b, h): out[rows][d]} then.  Otherwise returns float64 ``[T][Hq][d]``
    (and lse ``[T][Hq]`` if asked).
    """
    cu = np.asarray(cu_q_lens, dtype=np.int64)
    P = np.asarray(prefix_lens, dtype=np.int64)
    B = len(P)
    Hkv = k_pool.shape[1]
    G = num_q_heads // Hkv
    d = q.shape[-1]
    T = int(cu[-1])
    if select is not None:
        res = {}
        for b, h, rows in select:
            g = h // G
            C = int(cu[b + 1] - cu[b])
            K, V = _sequence_kv(k_pool, v_pool, block_tables[b], int(P[b]),
                                k_new[cu[b]:cu[b + 1]], v_new[cu[b]:cu[b + 1]], dtype)
            rows = np.asarray(rows, dtype=np.int64)
            assert np.all(rows < C)
            qr = decode_bits(q[cu[b] + rows, h], dtype)
            o, lse = attend(qr, K[:, g], V[:, g], P[b] + rows, scale)
            res[(b, h)] = (o, lse) if want_lse else o
        return res
    out = np.zeros((T, num_q_heads, d), dtype=np.float64)
    lse_all = np.full((T, num_q_heads), -np.inf)
    for b in range(B):
        C = int(cu[b + 1] - cu[b])
        if C == 0:
            continue
        K, V = _sequence_kv(k_pool, v_pool, block_tables[b], int(P[b]),
                            k_new[cu[b]:cu[b + 1]], v_new[cu[b]:cu[b + 1]], dtype)
        pos = P[b] + np.arange(C)
        for h in range(num_q_heads):
            g = h // G
            o, lse = attend(decode_bits(q[cu[b]:cu[b + 1], h], dtype), K[:, g], V[:, g], pos, scale)
            out[cu[b]:cu[b + 1], h] = o
            lse_all[cu[b]:cu[b + 1], h] = lse
    return (out, lse_all) if want_lse else out


def paged_decode(k_pool, v_pool, q, context_lens, block_tables, scale: float, dtype: str,
                 want_lse: bool = False, seqs: Optional[Sequence[int]] = None):
    """One query per sequence over its whole context, read from the pool.

    The current token's K/V is already in the pool, so ``context_lens`` counts it
    and the query sits at position ``ctx - 1`` (kvstream 0.1.0, "Request lifecycle"
    step 2: one slot per generated token; kvboost 0.6.0, "CPU paged attention":
    only the decode loop changes).  A non-positive context gives a zero row.
    Returns float64 ``[B][Hq][d]`` (and lse ``[B][Hq]``).
    """
    B, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, d), dtype=np.float64)
    lse_all = np.full((B, Hq), -np.inf)
    for b in (range(B) if seqs is None else seqs):
        n = int(context_lens[b])
        if n <= 0:
            continue
        K = decode_bits(gather_kv(k_pool, block_tables[b], n), dtype)
        V = decode_bits(gather_kv(v_pool, block_tables[b], n), dtype)
        qb = decode_bits(q[b], dtype)
        for h in range(Hq):
            o, lse = attend(qb[h:h + 1], K[:, h // G], V[:, h // G], [n - 1], scale)
            out[b, h] = o[0]
            lse_all[b, h] = lse[0]
    return (out, lse_all) if want_lse else out


def lse_merge(parts: Sequence[Tuple[np.ndarray, np.ndarray]]):
    """Combine attention results over disjoint key sets into the result over their
    union: weights ``exp(lse_s - M)`` with ``M = max lse_s``, outputs averaged by
    those weights, lse = M + log sum.  This is the exact softmax identity behind
    split decoding; empty parts (lse = -inf) contribute nothing."""
    lses = np.stack([p[1] for p in parts])             # [S][rows]
    outs = np.stack([p[0] for p in parts])             # [S][rows][d]
    M = lses.max(axis=0)
    Mf = np.where(np.isfinite(M), M, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - Mf[None]), 0.0)
    den = w.sum(axis=0)
    safe = np.where(den > 0, den, 1.0)
    out = (w[..., None] * outs).sum(axis=0) / safe[:, None]
    lse = np.where(den > 0, Mf + np.log(safe), -np.inf)
    return out, lse
