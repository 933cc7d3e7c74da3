"""Paged prefix-reuse attention for MI355X (gfx950): Python binding of libkvb.so.

The calls mirror the C ABI in ``include/kvb.h`` (kvb_write_kv, kvb_paged_prefill,
kvb_paged_decode, kvb_gather_kv and the workspace-size queries).  This layer only
marshals arguments: it takes torch device tensors for memory, passes their
addresses and the current HIP stream, and raises on a non-OK status.  Every step
of the computation runs in the library's HIP kernels; if the library is missing
the calls raise instead of falling back to anything else.

Pool layout: ``[num_blocks][num_kv_heads][16][head_dim]`` for K and for V (16-bit
payloads), one (block, kv-head) tile a contiguous 16 x head_dim run.  The pool of
fixed 16-token blocks follows kvboost 0.6.0, section "CPU paged attention".
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import KVB_BF16, KVB_FP16, KvbError, KvbPool, KvbPoolQ8  # noqa: F401

__all__ = [
    "Pool", "write_kv", "paged_prefill", "paged_prefill_pooled", "paged_decode", "paged_decode_noalloc",
    "paged_decode_cascade", "copy_blocks",
    "PoolQ8", "write_kv_q8", "paged_decode_q8", "paged_prefill_q8", "paged_prefill_q8_workspace_size",
    "PoolQ4", "write_kv_q4", "paged_decode_q4", "paged_prefill_q4",
    "gather_kv",
    "paged_prefill_workspace_size", "paged_decode_workspace_size",
    "paged_decode_cascade_workspace_size", "version", "KvbError",
]

BLOCK_SIZE = 16
_DT = {torch.float16: KVB_FP16, torch.bfloat16: KVB_BF16}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _index(device, dtype, min_rows: int, **tensors) -> None:
    """The kernels read index tensors through raw device pointers: each must be a contiguous
    ``dtype`` tensor on ``device`` (any GPU when None) with at least ``min_rows`` rows
    (elements when 1-D); None passes."""
    for name, t in tensors.items():
        if t is None:
            continue
        on = t.is_cuda if device is None else t.device == device
        if t.dtype != dtype or not t.is_contiguous() or not on or t.dim() == 0 or t.shape[0] < min_rows:
            raise ValueError(f"{name} must be a contiguous {dtype} tensor of at least {min_rows} "
                             f"rows on {device if device is not None else 'the GPU'}")


def _gpu(**tensors) -> None:
    """Tensors the kernels read or write through raw pointers must be in GPU memory (None
    passes)."""
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")


def _shaped(shape, dtypes, **tensors) -> None:
    """Data tensors are addressed from the pool's head dim and the call's sizes: each must be
    contiguous, of one of ``dtypes`` and of exactly ``shape`` (None passes)."""
    for name, t in tensors.items():
        if t is not None and (tuple(t.shape) != tuple(shape) or t.dtype not in dtypes
                              or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous tensor of shape {tuple(shape)} "
                             f"and dtype {' or '.join(str(d) for d in dtypes)}")


def _qkv(pool, q, k_new=None, v_new=None, out=None) -> None:
    # q/out [rows][Hq][d] and k_new/v_new [rows][Hkv][d] at the pool's head dim; a 16-bit pool
    # also fixes their dtype
    if q.dim() != 3:
        raise ValueError("q must be [rows][num_q_heads][head_dim]")
    dts = (pool.k.dtype,) if isinstance(pool, Pool) else tuple(_DT)
    _shaped((q.shape[0], q.shape[1], pool.head_dim), dts, q=q)
    _shaped(q.shape, (q.dtype,), out=out)
    _shaped((q.shape[0], pool.num_kv_heads, pool.head_dim), (q.dtype,), k_new=k_new, v_new=v_new)


def _pool_memory(*tensors) -> None:
    # pools may also sit in pinned host memory, which the GPU reaches at the same address
    if not all(t.is_cuda or t.is_pinned() for t in tensors):
        raise ValueError("pool tensors must be in GPU memory or in pinned host memory")


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


@dataclass
class Pool:
    """K/V block pool.  ``k``/``v`` are device tensors whose element (block, head,
    row, e) sits at ``block*block_stride + (head*16 + row)*head_dim + e``."""
    k: torch.Tensor
    v: torch.Tensor
    num_blocks: int
    num_kv_heads: int
    head_dim: int
    block_stride: int

    @classmethod
    def from_tensors(cls, k: torch.Tensor, v: torch.Tensor) -> "Pool":
        """Pool from two contiguous ``[num_blocks][num_kv_heads][16][head_dim]`` tensors."""
        nb, hkv, bs, d = k.shape
        if bs != BLOCK_SIZE or v.shape != k.shape or not k.is_contiguous() or not v.is_contiguous():
            raise ValueError("pool tensors must be contiguous [num_blocks][num_kv_heads][16][head_dim]")
        return cls(k, v, nb, hkv, d, hkv * BLOCK_SIZE * d)

    @classmethod
    def interleaved(cls, kv: torch.Tensor) -> "Pool":
        """Pool from one ``[num_blocks][2][num_kv_heads][16][head_dim]`` tensor: K and V of a
        block side by side, i.e. one page of block_size x heads x head_dim x 2 x dtype_bytes."""
        nb, two, hkv, bs, d = kv.shape
        if two != 2 or bs != BLOCK_SIZE or not kv.is_contiguous():
            raise ValueError("expected contiguous [num_blocks][2][num_kv_heads][16][head_dim]")
        return cls(kv[:, 0], kv[:, 1], nb, hkv, d, 2 * hkv * BLOCK_SIZE * d)

    @property
    def dtype(self) -> torch.dtype:
        return self.k.dtype

    def c_struct(self) -> KvbPool:
        if self.k.dtype not in _DT:
            raise ValueError(f"unsupported pool dtype {self.k.dtype}")
        _pool_memory(self.k, self.v)
        return KvbPool(self.k.data_ptr(), self.v.data_ptr(), self.block_stride, self.num_blocks,
                       BLOCK_SIZE, self.num_kv_heads, self.head_dim, _DT[self.k.dtype])


def version() -> str:
    return _lib.load().kvb_version().decode()


def write_kv(pool: Pool, k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
             stream=None) -> None:
    """kvb_write_kv: scatter ``k_new/v_new [T][Hkv][d]`` into pool slots ``slot_mapping`` (int64)."""
    _index(k_new.device, torch.int64, 0, slot_mapping=slot_mapping)
    if min(k_new.shape[0], v_new.shape[0]) < slot_mapping.numel():
        raise ValueError("k_new/v_new need a row for every entry of slot_mapping")
    _gpu(k_new=k_new, v_new=v_new)
    _shaped((k_new.shape[0], pool.num_kv_heads, pool.head_dim),
            (pool.k.dtype,) if isinstance(pool, Pool) else tuple(_DT), k_new=k_new)
    _shaped(k_new.shape, (k_new.dtype,), v_new=v_new)
    lib = _lib.load()
    ps = pool.c_struct()
    _lib.check("kvb_write_kv", lib.kvb_write_kv(
        ctypes.byref(ps), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), int(slot_mapping.numel()),
        _stream(stream)))


def paged_prefill_workspace_size(batch: int, num_q_heads: int, head_dim: int, total_q: int,
                                 max_prefix_len: int) -> int:
    return int(_lib.load().kvb_paged_prefill_workspace_size(batch, num_q_heads, head_dim, total_q,
                                                            max_prefix_len))


def paged_decode_workspace_size(batch: int, num_kv_heads: int, num_q_heads: int, head_dim: int,
                                max_context_len: int, split_blocks: int = 0) -> int:
    return int(_lib.load().kvb_paged_decode_workspace_size(batch, num_kv_heads, num_q_heads, head_dim,
                                                           max_context_len, split_blocks))


def paged_decode_cascade_workspace_size(batch: int, num_kv_heads: int, num_q_heads: int,
                                        head_dim: int, max_context_len: int, shared_len: int,
                                        split_blocks: int = 0) -> int:
    return int(_lib.load().kvb_paged_decode_cascade_workspace_size(
        batch, num_kv_heads, num_q_heads, head_dim, max_context_len, shared_len, split_blocks))


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return workspace
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return workspace


def _prefill_index(q, cu_q_lens, prefix_lens, block_tables) -> None:
    batch = prefix_lens.numel() if isinstance(prefix_lens, torch.Tensor) else 0
    _index(q.device, torch.int32, batch, prefix_lens=prefix_lens, block_tables=block_tables)
    _index(q.device, torch.int32, batch + 1, cu_q_lens=cu_q_lens)


def paged_prefill(pool: Pool, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                  cu_q_lens: torch.Tensor, prefix_lens: torch.Tensor, block_tables: torch.Tensor,
                  scale: float, max_q_len: int, max_prefix_len: int,
                  out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  stream=None, dispatch_plan: bool = True,
                  slot_mapping: Optional[torch.Tensor] = None) -> torch.Tensor:
    """kvb_paged_prefill.  ``q [T][Hq][d]``, ``k_new/v_new [T][Hkv][d]``, ``cu_q_lens`` int32
    [B+1], ``prefix_lens`` int32 [B], ``block_tables`` int32 [B][stride].
    ``dispatch_plan=False`` passes no workspace: work-groups start in table order instead
    of longest first (same results).  With ``slot_mapping`` (int64 [T]) the call is
    kvb_paged_prefill_write: the chunk's K/V is also written into the pool at those slots,
    as write_kv would, in the same launch."""
    _prefill_index(q, cu_q_lens, prefix_lens, block_tables)
    if slot_mapping is not None:
        # the kernel reads total_q int64 slots through this pointer
        _index(q.device, torch.int64, q.shape[0], slot_mapping=slot_mapping)
        if slot_mapping.numel() != q.shape[0]:
            raise ValueError("slot_mapping must hold one slot per query row")
    _gpu(q=q, k_new=k_new, v_new=v_new, out=out, workspace=workspace)
    _qkv(pool, q, k_new, v_new, out)
    lib = _lib.load()
    if out is None:
        out = torch.empty_like(q)
    batch = int(prefix_lens.numel())
    T, hq, d = q.shape
    if dispatch_plan:
        need = paged_prefill_workspace_size(batch, hq, d, T, max_prefix_len)
        workspace = _workspace(need, q.device, workspace)
    else:
        workspace = None
    ps = pool.c_struct()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if slot_mapping is not None:
        _lib.check("kvb_paged_prefill_write", lib.kvb_paged_prefill_write(
            ctypes.byref(ps), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out), _ptr(slot_mapping),
            _ptr(cu_q_lens), _ptr(prefix_lens), _ptr(block_tables), int(block_tables.shape[1]), batch,
            hq, T, int(max_q_len), int(max_prefix_len), float(scale), _ptr(workspace), ws_bytes,
            _stream(stream)))
        return out
    _lib.check("kvb_paged_prefill", lib.kvb_paged_prefill(
        ctypes.byref(ps), _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out), _ptr(cu_q_lens),
        _ptr(prefix_lens), _ptr(block_tables), int(block_tables.shape[1]), batch, hq, T,
        int(max_q_len), int(max_prefix_len), float(scale), _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def paged_prefill_pooled(pool: Pool, q: torch.Tensor, cu_q_lens: torch.Tensor,
                         prefix_lens: torch.Tensor, block_tables: torch.Tensor, scale: float,
                         max_q_len: int, max_prefix_len: int, out: Optional[torch.Tensor] = None,
                         stream=None) -> torch.Tensor:
    """kvb_paged_prefill_pooled: as ``paged_prefill``, with the chunk's own K/V read from
    the pool (written there by ``write_kv`` first) through ``block_tables``."""
    _prefill_index(q, cu_q_lens, prefix_lens, block_tables)
    _gpu(q=q, out=out)
    _qkv(pool, q, out=out)
    lib = _lib.load()
    if out is None:
        out = torch.empty_like(q)
    batch = int(prefix_lens.numel())
    T, hq, d = q.shape
    ps = pool.c_struct()
    _lib.check("kvb_paged_prefill_pooled", lib.kvb_paged_prefill_pooled(
        ctypes.byref(ps), _ptr(q), _ptr(out), _ptr(cu_q_lens), _ptr(prefix_lens),
        _ptr(block_tables), int(block_tables.shape[1]), batch, hq, T, int(max_q_len),
        int(max_prefix_len), float(scale), _stream(stream)))
    return out


def paged_decode(pool: Pool, q: torch.Tensor, context_lens: torch.Tensor,
                 block_tables: torch.Tensor, scale: float, max_context_len: int,
                 split_blocks: int = 0, out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """kvb_paged_decode.  ``q [B][Hq][d]``, ``context_lens`` int32 [B] (including the current
    token), ``block_tables`` int32 [B][stride]."""
    _index(q.device, torch.int32, q.shape[0], context_lens=context_lens, block_tables=block_tables)
    _gpu(q=q, out=out, workspace=workspace)
    _qkv(pool, q, out=out)
    lib = _lib.load()
    if out is None:
        out = torch.empty_like(q)
    B, hq, d = q.shape
    need = paged_decode_workspace_size(B, pool.num_kv_heads, hq, d, max_context_len, split_blocks)
    workspace = _workspace(need, q.device, workspace)
    ps = pool.c_struct()
    _lib.check("kvb_paged_decode", lib.kvb_paged_decode(
        ctypes.byref(ps), _ptr(q), _ptr(out), _ptr(context_lens), _ptr(block_tables),
        int(block_tables.shape[1]), B, hq, int(max_context_len), int(split_blocks), float(scale),
        _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return out


def paged_decode_noalloc(pool: Pool, q: torch.Tensor, context_lens: torch.Tensor,
                         block_tables: torch.Tensor, scale: float, max_context_len: int,
                         out: torch.Tensor, split_blocks: int = 0, stream=None) -> torch.Tensor:
    """kvb_paged_decode_noalloc: ``paged_decode`` with the split partials in the library's
    static device scratch instead of a workspace.  ``out`` is required: this call allocates
    nothing.  Calls that overlap on one GPU share the scratch and race."""
    _index(q.device, torch.int32, q.shape[0], context_lens=context_lens, block_tables=block_tables)
    _gpu(q=q, out=out)
    _qkv(pool, q, out=out)
    lib = _lib.load()
    B, hq, d = q.shape
    ps = pool.c_struct()
    _lib.check("kvb_paged_decode_noalloc", lib.kvb_paged_decode_noalloc(
        ctypes.byref(ps), _ptr(q), _ptr(out), _ptr(context_lens), _ptr(block_tables),
        int(block_tables.shape[1]), B, hq, int(max_context_len), int(split_blocks), float(scale),
        _stream(stream)))
    return out


def gather_kv(pool: Pool, block_tables: torch.Tensor, seq_lens: torch.Tensor,
              cu_seq_lens: torch.Tensor, max_len: int, k_out: torch.Tensor, v_out: torch.Tensor,
              stream=None) -> None:
    """kvb_gather_kv (indexing check): logical tokens of every sequence, contiguous."""
    _index(k_out.device, torch.int32, seq_lens.numel(), block_tables=block_tables, seq_lens=seq_lens)
    _index(k_out.device, torch.int32, seq_lens.numel() + 1, cu_seq_lens=cu_seq_lens)
    _gpu(k_out=k_out, v_out=v_out)
    lib = _lib.load()
    ps = pool.c_struct()
    _lib.check("kvb_gather_kv", lib.kvb_gather_kv(
        ctypes.byref(ps), _ptr(block_tables), int(block_tables.shape[1]), _ptr(seq_lens),
        _ptr(cu_seq_lens), _ptr(k_out), _ptr(v_out), int(seq_lens.numel()), int(max_len),
        _stream(stream)))


def paged_decode_cascade(pool: Pool, q: torch.Tensor, context_lens: torch.Tensor,
                         block_tables: torch.Tensor, shared_blocks: Optional[torch.Tensor],
                         shared_len: int, scale: float, max_context_len: int,
                         split_blocks: int = 0, out: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """kvb_paged_decode_cascade.  As ``paged_decode``; the first ``shared_len`` tokens of
    every sequence are the blocks ``shared_blocks`` (int32), read once for all queries."""
    _index(q.device, torch.int32, q.shape[0], context_lens=context_lens, block_tables=block_tables)
    _index(q.device, torch.int32, (max(int(shared_len), 0) + 15) // 16, shared_blocks=shared_blocks)
    _gpu(q=q, out=out, workspace=workspace)
    _qkv(pool, q, out=out)
    lib = _lib.load()
    if out is None:
        out = torch.empty_like(q)
    B, hq, d = q.shape
    need = paged_decode_cascade_workspace_size(B, pool.num_kv_heads, hq, d, max_context_len,
                                               shared_len, split_blocks)
    workspace = _workspace(need, q.device, workspace)
    ps = pool.c_struct()
    _lib.check("kvb_paged_decode_cascade", lib.kvb_paged_decode_cascade(
        ctypes.byref(ps), _ptr(q), _ptr(out), _ptr(context_lens), _ptr(block_tables),
        int(block_tables.shape[1]), _ptr(shared_blocks), int(shared_len), B, hq,
        int(max_context_len), int(split_blocks), float(scale), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


def copy_blocks(src: Pool, dst: Pool, src_ids: torch.Tensor, dst_ids: torch.Tensor,
                stream=None) -> None:
    """kvb_copy_blocks: block dst_ids[i] of ``dst`` becomes a copy of block src_ids[i] of
    ``src`` (K and V, every head).  ``src_ids``/``dst_ids``: int32 device tensors."""
    _index(None, torch.int32, src_ids.numel(), src_ids=src_ids, dst_ids=dst_ids)
    lib = _lib.load()
    a, b = src.c_struct(), dst.c_struct()
    _lib.check("kvb_copy_blocks", lib.kvb_copy_blocks(
        ctypes.byref(a), ctypes.byref(b), _ptr(src_ids), _ptr(dst_ids), int(src_ids.numel()),
        _stream(stream)))


@dataclass
class PoolQ8:
    """Quantised K/V pool (kvb_pool_q8, or kvb_pool_q4 with ``bits=4``): codes ``k``/``v``
    ``[num_blocks][num_kv_heads][16][head_dim]`` int8 (8 bits) or ``[..][head_dim/2]`` uint8
    holding two 4-bit codes per byte (even channel in the low nibble), per-token V scales
    ``v_scale`` float32 ``[num_blocks][num_kv_heads][16]`` and the pool's per-channel K
    scales ``k_scale`` float32 ``[num_kv_heads][head_dim]``.  A code c stands for c * scale
    (kvboost 0.6.0, "Optional: KV quantization")."""
    k: torch.Tensor
    v: torch.Tensor
    v_scale: torch.Tensor
    k_scale: torch.Tensor
    bits: int = 8

    @classmethod
    def empty(cls, num_blocks: int, num_kv_heads: int, head_dim: int, k_scale: torch.Tensor,
              device="cuda", bits: int = 8) -> "PoolQ8":
        if bits not in (8, 4):
            raise ValueError("bits must be 8 or 4")
        shape = (num_blocks, num_kv_heads, BLOCK_SIZE, head_dim * bits // 8)
        dt = torch.int8 if bits == 8 else torch.uint8
        return cls(torch.zeros(shape, dtype=dt, device=device),
                   torch.zeros(shape, dtype=dt, device=device),
                   torch.zeros(shape[:3], dtype=torch.float32, device=device),
                   k_scale.to(device=device, dtype=torch.float32).contiguous(), bits)

    @property
    def num_blocks(self) -> int:
        return int(self.k.shape[0])

    @property
    def num_kv_heads(self) -> int:
        return int(self.k.shape[1])

    @property
    def head_dim(self) -> int:
        return int(self.k.shape[3]) * 8 // self.bits

    def c_struct(self) -> KvbPoolQ8:
        nb, hkv, bs, row_bytes = self.k.shape
        d = self.head_dim
        code_dt = torch.int8 if self.bits == 8 else torch.uint8
        for t, dt in ((self.k, code_dt), (self.v, code_dt), (self.v_scale, torch.float32),
                      (self.k_scale, torch.float32)):
            if t.dtype != dt or not t.is_contiguous():
                raise ValueError("quantised pool tensors: contiguous codes and float32 scales")
        if self.v.shape != self.k.shape or self.v_scale.shape != (nb, hkv, bs) or \
                self.k_scale.shape != (hkv, d):
            raise ValueError("quantised pool tensor shapes do not match")
        _pool_memory(self.k, self.v, self.v_scale, self.k_scale)
        return KvbPoolQ8(self.k.data_ptr(), self.v.data_ptr(), self.v_scale.data_ptr(),
                         self.k_scale.data_ptr(), hkv * bs * row_bytes, nb, bs, hkv, d)


def PoolQ4(k: torch.Tensor, v: torch.Tensor, v_scale: torch.Tensor, k_scale: torch.Tensor) -> PoolQ8:
    """4-bit pool (kvb_pool_q4): ``k``/``v`` uint8 ``[num_blocks][num_kv_heads][16][head_dim/2]``."""
    return PoolQ8(k, v, v_scale, k_scale, 4)


def _qfn(lib, name: str, pool: PoolQ8):
    return getattr(lib, name.replace("_q8", "_q4") if pool.bits == 4 else name)


def write_kv_q8(pool: PoolQ8, k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
                stream=None) -> None:
    """kvb_write_kv_q8: code ``k_new/v_new [T][Hkv][d]`` (fp16/bf16) into the 8-bit pool's
    slots ``slot_mapping`` (int64), writing each token's V scale."""
    _index(k_new.device, torch.int64, 0, slot_mapping=slot_mapping)
    if min(k_new.shape[0], v_new.shape[0]) < slot_mapping.numel():
        raise ValueError("k_new/v_new need a row for every entry of slot_mapping")
    _gpu(k_new=k_new, v_new=v_new)
    _shaped((k_new.shape[0], pool.num_kv_heads, pool.head_dim),
            (pool.k.dtype,) if isinstance(pool, Pool) else tuple(_DT), k_new=k_new)
    _shaped(k_new.shape, (k_new.dtype,), v_new=v_new)
    lib = _lib.load()
    if k_new.dtype not in _DT or v_new.dtype != k_new.dtype:
        raise ValueError("k_new/v_new must both be float16 or bfloat16")
    ps = pool.c_struct()
    _lib.check("kvb_write_kv_q8", _qfn(lib, "kvb_write_kv_q8", pool)(
        ctypes.byref(ps), _ptr(k_new), _ptr(v_new), _DT[k_new.dtype], _ptr(slot_mapping),
        int(slot_mapping.numel()), _stream(stream)))


def paged_decode_q8(pool: PoolQ8, q: torch.Tensor, context_lens: torch.Tensor,
                    block_tables: torch.Tensor, scale: float, max_context_len: int,
                    split_blocks: int = 0, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """kvb_paged_decode_q8: ``paged_decode`` over the 8-bit pool; ``q``/``out`` fp16 or bf16."""
    _index(q.device, torch.int32, q.shape[0], context_lens=context_lens, block_tables=block_tables)
    _gpu(q=q, out=out, workspace=workspace)
    _qkv(pool, q, out=out)
    lib = _lib.load()
    if q.dtype not in _DT:
        raise ValueError("q must be float16 or bfloat16")
    if out is None:
        out = torch.empty_like(q)
    B, hq, d = q.shape
    need = paged_decode_workspace_size(B, pool.num_kv_heads, hq, d, max_context_len, split_blocks)
    workspace = _workspace(need, q.device, workspace)
    ps = pool.c_struct()
    _lib.check("kvb_paged_decode_q8", _qfn(lib, "kvb_paged_decode_q8", pool)(
        ctypes.byref(ps), _DT[q.dtype], _ptr(q), _ptr(out), _ptr(context_lens), _ptr(block_tables),
        int(block_tables.shape[1]), B, hq, int(max_context_len), int(split_blocks), float(scale),
        _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream(stream)))
    return out


def paged_prefill_q8_workspace_size(batch: int, num_kv_heads: int, num_q_heads: int, head_dim: int,
                                    total_q: int, max_prefix_len: int) -> int:
    return int(_lib.load().kvb_paged_prefill_q8_workspace_size(batch, num_kv_heads, num_q_heads,
                                                               head_dim, total_q, max_prefix_len))


def paged_prefill_q8(pool: PoolQ8, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                     cu_q_lens: torch.Tensor, prefix_lens: torch.Tensor, block_tables: torch.Tensor,
                     scale: float, max_q_len: int, max_prefix_len: int,
                     out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """kvb_paged_prefill_q8: ``paged_prefill`` with the cached prefix in the 8-bit pool;
    ``q``, ``k_new``, ``v_new``, ``out`` fp16 or bf16."""
    _prefill_index(q, cu_q_lens, prefix_lens, block_tables)
    _gpu(q=q, k_new=k_new, v_new=v_new, out=out, workspace=workspace)
    _qkv(pool, q, k_new, v_new, out)
    lib = _lib.load()
    if q.dtype not in _DT:
        raise ValueError("q must be float16 or bfloat16")
    if out is None:
        out = torch.empty_like(q)
    batch = int(prefix_lens.numel())
    T, hq, d = q.shape
    need = paged_prefill_q8_workspace_size(batch, pool.num_kv_heads, hq, d, T, max_prefix_len)
    workspace = _workspace(need, q.device, workspace)
    ps = pool.c_struct()
    _lib.check("kvb_paged_prefill_q8", _qfn(lib, "kvb_paged_prefill_q8", pool)(
        ctypes.byref(ps), _DT[q.dtype], _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out),
        _ptr(cu_q_lens), _ptr(prefix_lens), _ptr(block_tables), int(block_tables.shape[1]), batch,
        hq, T, int(max_q_len), int(max_prefix_len), float(scale), _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream)))
    return out


# The same calls on a 4-bit pool (PoolQ4); the functions above dispatch on ``pool.bits``.
write_kv_q4 = write_kv_q8
paged_decode_q4 = paged_decode_q8
paged_prefill_q4 = paged_prefill_q8
