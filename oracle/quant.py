"""8-bit and 4-bit K/V pools: quantisation, dequantisation, and decode and prefill over them.

Test infrastructure only (see the package docstring).  The pages store cached K/V at
8 bits with per-channel scales for K and per-token scales for V (kvboost 0.6.0,
"Optional: KV quantization": the KIVI asymmetry, about 2x smaller).  They fix the two
axes and nothing else; the readings taken here:

* codes are signed integers in [-127, 127] (symmetric, no zero point): a value x with
  scale s becomes ``rint(x / s)`` clamped to that range, the division and the rounding
  (half to even) done in IEEE float32, so a GPU that does the same steps in float32
  produces the same codes; a zero scale gives code 0;
* K: one scale per (KV head, channel) for the whole pool, given by the caller (for
  example the per-channel absolute maximum of the prompt's K over its tokens, / 127);
  stored codes never change when tokens are appended;
* V: one scale per (token, KV head) = max_c |v_c| / 127 (float32), computed when the
  token is written;
* the value a code stands for is ``code * scale``, exact in float64;
* 4 bits (the pages' "kv_cache_bits=4"): the same rules with codes in [-7, 7] and the V
  scale max |v| / 7; two codes per byte, channel 2i in the low nibble and 2i+1 in the
  high one, each as a 4-bit two's complement.

Pool arrays: codes int8 ``[num_blocks][num_kv_heads][16][d]`` (unpacked here, also for 4
bits; ``pack_nibbles`` gives the stored bytes), V scales float32
``[num_blocks][num_kv_heads][16]``, K scales float32 ``[num_kv_heads][d]``.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .attention import BLOCK_SIZE, attend, decode_bits, gather_kv

CODE_MAX = 127
CODE_MAX4 = 7


def quantize(x: np.ndarray, s: np.ndarray, code_max: int = CODE_MAX) -> np.ndarray:
    """int8 codes of float32 values ``x`` at float32 scales ``s`` (broadcast):
    ``rint(x / s)`` in float32, clamped to [-code_max, code_max]; 0 where s == 0."""
    x = np.asarray(x, dtype=np.float32)
    s = np.broadcast_to(np.asarray(s, dtype=np.float32), x.shape)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.rint(np.divide(x, s, dtype=np.float32))
    r = np.where(s == 0, np.float32(0), r)
    return np.clip(r, -code_max, code_max).astype(np.int8)


def token_scale(v: np.ndarray, code_max: int = CODE_MAX) -> np.ndarray:
    """Per-token V scale over the last axis: max |v| / code_max in float32."""
    a = np.abs(np.asarray(v, dtype=np.float32)).max(axis=-1)
    return np.divide(a, np.float32(code_max), dtype=np.float32)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """4-bit codes ``[..][d]`` (int8 in [-7, 7]) as stored bytes ``[..][d/2]``: channel 2i
    in the low nibble, 2i+1 in the high nibble, each a 4-bit two's complement."""
    c = np.asarray(codes, dtype=np.int16) & 0xF
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """Inverse of ``pack_nibbles``: bytes ``[..][d/2]`` -> int8 codes ``[..][d]``."""
    b = np.asarray(packed, dtype=np.uint8).astype(np.int16)
    lo, hi = b & 0xF, b >> 4
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def write_kv_q8(k_codes: np.ndarray, v_codes: np.ndarray, v_scales: np.ndarray,
                k_scale: np.ndarray, k_new: np.ndarray, v_new: np.ndarray, slot_mapping: np.ndarray,
                dtype: str, code_max: int = CODE_MAX) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Quantise each new token and scatter it into its pool slot; negative slots are
    skipped (the slot rule of ``write_kv``: block ``slot // 16``, row ``slot % 16``).
    ``k_new``/``v_new`` are 16-bit payloads ``[T][Hkv][d]``.  ``code_max`` 127 (8 bits)
    or 7 (4 bits; codes kept unpacked).  Returns new arrays."""
    kc = np.array(k_codes, copy=True)
    vc = np.array(v_codes, copy=True)
    vs = np.array(v_scales, copy=True)
    kf = decode_bits(k_new, dtype).astype(np.float32)      # exact: 16-bit -> float32
    vf = decode_bits(v_new, dtype).astype(np.float32)
    for t, slot in enumerate(np.asarray(slot_mapping, dtype=np.int64)):
        if slot < 0:
            continue
        blk, row = int(slot) // BLOCK_SIZE, int(slot) % BLOCK_SIZE
        kc[blk, :, row, :] = quantize(kf[t], k_scale, code_max)
        s = token_scale(vf[t], code_max)                    # [Hkv]
        vs[blk, :, row] = s
        vc[blk, :, row, :] = quantize(vf[t], s[:, None], code_max)
    return kc, vc, vs


def dequant_k(codes: np.ndarray, k_scale: np.ndarray) -> np.ndarray:
    """Values of K codes ``[..][Hkv][d]`` at scales ``[Hkv][d]``, float64 (exact)."""
    return np.asarray(codes, dtype=np.float64) * np.asarray(k_scale, dtype=np.float64)


def dequant_v(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Values of V codes ``[..][d]`` at per-token scales ``[..]``, float64 (exact)."""
    return np.asarray(codes, dtype=np.float64) * np.asarray(scales, dtype=np.float64)[..., None]


def paged_decode_q8(k_codes, v_codes, v_scales, k_scale, q, context_lens, block_tables,
                    scale: float, dtype: str, want_lse: bool = False):
    """Decode (one query per sequence over its whole context, as ``paged_decode``) over
    the values the 8-bit pool stands for.  ``q`` holds 16-bit payloads ``[B][Hq][d]``."""
    B, Hq, d = q.shape
    Hkv = k_codes.shape[1]
    G = Hq // Hkv
    out = np.zeros((B, Hq, d), dtype=np.float64)
    lse_all = np.full((B, Hq), -np.inf)
    for b in range(B):
        n = int(context_lens[b])
        if n <= 0:
            continue
        K = dequant_k(gather_kv(k_codes, block_tables[b], n), k_scale)
        j = np.arange(n)
        blocks = np.asarray(block_tables[b], dtype=np.int64)[j // BLOCK_SIZE]
        Vs = v_scales[blocks, :, j % BLOCK_SIZE]                      # [n][Hkv]
        V = dequant_v(gather_kv(v_codes, block_tables[b], n), Vs)
        qb = decode_bits(q[b], dtype)
        for h in range(Hq):
            o, lse = attend(qb[h:h + 1], K[:, h // G], V[:, h // G], [n - 1], scale)
            out[b, h] = o[0]
            lse_all[b, h] = lse[0]
    return (out, lse_all) if want_lse else out


def paged_prefill_q8(k_codes, v_codes, v_scales, k_scale, q, k_new, v_new, cu_q_lens, prefix_lens,
                     block_tables, num_q_heads: int, scale: float, dtype: str, select=None):
    """Chunk prefill (as ``attention.paged_prefill``: row i of sequence b at position
    ``P_b + i`` sees the whole cached prefix and chunk tokens ``0..i``) with the cached
    prefix read from the 8-bit pool as the values its codes stand for; the chunk's own
    K/V are the call's 16-bit rows.  Returns float64 ``[T][Hq][d]``; with ``select``, a
    list of (b, h, rows), only those rows, as a dict {(b, h): out[rows][d]} (the same
    arithmetic, for sampled rows of large workloads)."""
    cu = np.asarray(cu_q_lens, dtype=np.int64)
    P = np.asarray(prefix_lens, dtype=np.int64)
    Hkv = k_codes.shape[1]
    G = num_q_heads // Hkv
    T, _, d = q.shape
    want = None
    if select is not None:
        want = {}
        for b, h, rows in select:
            want.setdefault(int(b), []).append((int(h), np.asarray(rows, dtype=np.int64)))
    res = {}
    out = np.zeros((T, num_q_heads, d), dtype=np.float64) if want is None else None
    for b in range(len(P)):
        C = int(cu[b + 1] - cu[b])
        if C == 0 or (want is not None and b not in want):
            continue
        n = int(P[b])
        j = np.arange(n)
        blocks = np.asarray(block_tables[b], dtype=np.int64)[j // BLOCK_SIZE]
        Kp = dequant_k(gather_kv(k_codes, block_tables[b], n), k_scale)
        Vp = dequant_v(gather_kv(v_codes, block_tables[b], n), v_scales[blocks, :, j % BLOCK_SIZE])
        K = np.concatenate([Kp, decode_bits(k_new[cu[b]:cu[b + 1]], dtype)], axis=0)
        V = np.concatenate([Vp, decode_bits(v_new[cu[b]:cu[b + 1]], dtype)], axis=0)
        if want is not None:
            for h, rows in want[b]:
                assert np.all(rows < C)
                o, _ = attend(decode_bits(q[cu[b] + rows, h], dtype), K[:, h // G], V[:, h // G],
                              n + rows, scale)
                res[(b, h)] = o
            continue
        pos = n + np.arange(C)
        for h in range(num_q_heads):
            o, _ = attend(decode_bits(q[cu[b]:cu[b + 1], h], dtype), K[:, h // G], V[:, h // G], pos, scale)
            out[cu[b]:cu[b + 1], h] = o
    return res if want is not None else out
