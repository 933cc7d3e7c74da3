"""Helpers for the GPU parity tests: upload a seeded workload, call the HIP path through
the binding, bring results back as 16-bit payloads, and compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import attention_paged_prefix_amd as kvb
import oracle

TOL = {"fp16": 1e-2, "bf16": 2e-2}
TDT = {"fp16": torch.float16, "bf16": torch.bfloat16}
DEV = "cuda:0"


def to_dev(bits: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(DEV).view(TDT[dtype])


def to_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def idev(a, dtype=torch.int32) -> torch.Tensor:
    return torch.as_tensor(np.ascontiguousarray(a)).to(dtype).to(DEV)


class Dev:
    """Device copies of one workload."""

    def __init__(self, w, pool_layout: str = "split"):
        self.w = w
        dt = w.dtype
        if pool_layout == "interleaved":
            kv = np.stack([w.k_pool, w.v_pool], axis=1)
            self.kv = to_dev(kv, dt)
            self.pool = kvb.Pool.interleaved(self.kv)
        else:
            self.k = to_dev(w.k_pool, dt)
            self.v = to_dev(w.v_pool, dt)
            self.pool = kvb.Pool.from_tensors(self.k, self.v)
        self.bt = idev(w.block_tables)
        self.q = to_dev(w.q, dt)
        if w.kind == "prefill":
            self.k_new = to_dev(w.k_new, dt)
            self.v_new = to_dev(w.v_new, dt)
            self.cu = idev(w.cu_q_lens)
            self.pl = idev(w.prefix_lens)
            self.slots = idev(w.slot_mapping, torch.int64)
        else:
            self.ctx = idev(w.context_lens)

    def prefill(self, out=None):
        w = self.w
        return kvb.paged_prefill(self.pool, self.q, self.k_new, self.v_new, self.cu, self.pl, self.bt,
                                 w.scale, int(w.q_lens.max()) if w.batch else 0,
                                 int(w.prefix_lens.max()) if w.batch else 0, out=out)

    def decode(self, split_blocks=0, out=None):
        w = self.w
        return kvb.paged_decode(self.pool, self.q, self.ctx, self.bt, w.scale,
                                int(w.context_lens.max()), split_blocks=split_blocks, out=out)


def oracle_prefill(w, select=None):
    return oracle.paged_prefill(w.k_pool, w.v_pool, w.q, w.k_new, w.v_new, w.cu_q_lens, w.prefix_lens,
                                w.block_tables, w.num_q_heads, w.scale, w.dtype, select=select)


def oracle_decode(w, seqs=None):
    return oracle.paged_decode(w.k_pool, w.v_pool, w.q, w.context_lens, w.block_tables, w.scale,
                               w.dtype, seqs=seqs)


def max_err(got_bits: np.ndarray, ref: np.ndarray, dtype: str) -> float:
    got = oracle.decode_bits(got_bits, dtype)
    return float(np.max(np.abs(got - ref))) if got.size else 0.0
