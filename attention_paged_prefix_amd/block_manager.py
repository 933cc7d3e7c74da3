"""Host bookkeeping of a paged K/V pool: which physical blocks are free, how many block
tables reference each one, and the block table of every sequence.

It follows the pages' pool operations: a fixed pool of 16-token blocks whose shared
prefixes share physical blocks copy-on-write (kvboost 0.6.0, "CPU paged attention";
kvstream 0.1.0, "Request lifecycle" steps 2-4: one slot per generated token, a shared
prefix's block table forked copy-on-write, pages returned to the pool when a request
ends) and low-priority sequences spilled to a CPU page pool (kvstream 0.1.0, "Why
KVStream?", swap & preemption; "Configuration", num_cpu_blocks).  ``stats()`` reports the
fields of kvboost's ``paged_stats``.

The manager does no device work.  Operations that need data moved return the block
pairs to copy, which the caller runs with ``copy_blocks`` (kvb_copy_blocks) before it
writes the next token (``write_kv``) or attends to the sequence.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Tuple

BLOCK = 16


class OutOfBlocks(RuntimeError):
    pass


class BlockManager:
    def __init__(self, num_gpu_blocks: int, num_cpu_blocks: int = 0, block_size: int = BLOCK):
        if block_size != BLOCK:
            raise ValueError("the kernels use 16-token blocks")
        self.num_gpu_blocks = int(num_gpu_blocks)
        self.num_cpu_blocks = int(num_cpu_blocks)
        # lowest ids first, so tables are easy to read in tests
        self._free = list(range(self.num_gpu_blocks - 1, -1, -1))
        self._cpu_free = list(range(self.num_cpu_blocks - 1, -1, -1))
        self._ref = [0] * self.num_gpu_blocks
        self._tables: Dict[object, List[int]] = {}
        self._lens: Dict[object, int] = {}
        self._swapped: Dict[object, List[int]] = {}     # sequence -> CPU blocks

    # ------------------------------------------------------------------ queries
    def block_table(self, seq) -> List[int]:
        return list(self._tables[seq])

    def num_tokens(self, seq) -> int:
        return self._lens[seq]

    def refcount(self, block: int) -> int:
        return self._ref[block]

    def stats(self) -> dict:
        used = sum(1 for r in self._ref if r > 0)
        return {
            "block_utilization": used / self.num_gpu_blocks if self.num_gpu_blocks else 0.0,
            "free_blocks": len(self._free),
            "used_blocks": used,
            "shared_blocks": sum(1 for r in self._ref if r > 1),
            "sequences": len(self._tables),
            "swapped_sequences": len(self._swapped),
            "cpu_free_blocks": len(self._cpu_free),
        }

    # ------------------------------------------------------------------ allocation
    def _take(self) -> int:
        if not self._free:
            raise OutOfBlocks("no free GPU block")
        b = self._free.pop()
        self._ref[b] = 1
        return b

    def _release(self, b: int) -> None:
        self._ref[b] -= 1
        if self._ref[b] == 0:
            self._free.append(b)

    def allocate(self, seq, num_tokens: int) -> List[int]:
        """A new sequence with ``num_tokens`` token slots; returns its block table."""
        if seq in self._tables or seq in self._swapped:
            raise ValueError(f"sequence {seq!r} exists")
        need = (int(num_tokens) + BLOCK - 1) // BLOCK
        if need > len(self._free):
            raise OutOfBlocks(f"{need} blocks needed, {len(self._free)} free")
        self._tables[seq] = [self._take() for _ in range(need)]
        self._lens[seq] = int(num_tokens)
        return self.block_table(seq)

    def fork(self, parent, child) -> List[int]:
        """``child`` shares every block of ``parent`` (copy-on-write)."""
        if child in self._tables or child in self._swapped:
            raise ValueError(f"sequence {child!r} exists")
        table = self._tables[parent]
        for b in table:
            self._ref[b] += 1
        self._tables[child] = list(table)
        self._lens[child] = self._lens[parent]
        return self.block_table(child)

    def slots(self, seq, start: int, count: int) -> List[int]:
        """Pool slots (block * 16 + row) of tokens start..start+count-1 of ``seq``."""
        t = self._tables[seq]
        return [t[p // BLOCK] * BLOCK + p % BLOCK for p in range(start, start + count)]

    def append_slot(self, seq) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Room for one more token.  Returns its slot and, when the block it lands in was
        shared, the (source, destination) block copy that makes it private: run it
        before writing the token."""
        t = self._tables[seq]
        p = self._lens[seq]
        copy = None
        if p % BLOCK == 0:
            t.append(self._take())
        elif self._ref[t[-1]] > 1:
            new = self._take()
            copy = (t[-1], new)
            self._release(t[-1])
            t[-1] = new
        self._lens[seq] = p + 1
        return t[p // BLOCK] * BLOCK + p % BLOCK, copy

    def free(self, seq) -> None:
        """The sequence ends: its references return to the pool."""
        if seq in self._swapped:
            self._cpu_free.extend(self._swapped.pop(seq))
            del self._lens[seq]
            return
        for b in self._tables.pop(seq):
            self._release(b)
        del self._lens[seq]

    # ------------------------------------------------------------------ swap
    def swap_out(self, seq) -> List[Tuple[int, int]]:
        """Move ``seq`` to the CPU pool.  Returns (GPU block, CPU block) pairs to copy
        (GPU pool -> CPU pool) before any of its GPU blocks are reused."""
        t = self._tables[seq]
        if len(t) > len(self._cpu_free):
            raise OutOfBlocks(f"{len(t)} CPU blocks needed, {len(self._cpu_free)} free")
        cpu = [self._cpu_free.pop() for _ in t]
        pairs = list(zip(t, cpu))
        del self._tables[seq]
        for b in t:
            self._release(b)
        self._swapped[seq] = cpu
        return pairs

    def swap_in(self, seq) -> List[Tuple[int, int]]:
        """Bring ``seq`` back.  Returns (CPU block, GPU block) pairs to copy (CPU pool ->
        GPU pool) before the sequence is used."""
        cpu = self._swapped[seq]
        if len(cpu) > len(self._free):
            raise OutOfBlocks(f"{len(cpu)} GPU blocks needed, {len(self._free)} free")
        gpu = [self._take() for _ in cpu]
        del self._swapped[seq]
        self._cpu_free.extend(cpu)
        self._tables[seq] = gpu
        return list(zip(cpu, gpu))
