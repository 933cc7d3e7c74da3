"""A random script of block-manager operations (allocate, fork, append one token, free,
swap out / in) applied to K/V pools through pluggable write / copy functions, so the same
script drives the oracle (numpy) and the HIP path and their pools can be compared."""
import numpy as np

from attention_paged_prefix_amd.block_manager import BlockManager, OutOfBlocks


def run(backend, nb, ncpu, steps, seed, kv_shape):
    """backend: write(slots, k_rows, v_rows), copy(src_pool, dst_pool, src_ids, dst_ids)
    with pool names "gpu" / "cpu".  Returns (manager, expected tokens per sequence)."""
    rng = np.random.default_rng(seed)
    m = BlockManager(nb, ncpu)
    expect = {}

    def new_toks(n):
        return (rng.integers(0, 1 << 16, size=(n,) + kv_shape).astype(np.uint16),
                rng.integers(0, 1 << 16, size=(n,) + kv_shape).astype(np.uint16))

    nid = 0
    for _ in range(steps):
        live = [s for s in expect if s not in m._swapped]
        op = int(rng.integers(0, 6))
        if op == 0 or not live:
            n = int(rng.integers(1, 40))
            try:
                m.allocate(nid, n)
            except OutOfBlocks:
                continue
            kr, vr = new_toks(n)
            backend.write(m.slots(nid, 0, n), kr, vr)
            expect[nid] = (list(kr), list(vr))
            nid += 1
        elif op == 1:
            p = live[int(rng.integers(len(live)))]
            m.fork(p, nid)
            expect[nid] = (list(expect[p][0]), list(expect[p][1]))
            nid += 1
        elif op in (2, 3):
            sq = live[int(rng.integers(len(live)))]
            try:
                slot, copy = m.append_slot(sq)
            except OutOfBlocks:
                continue
            if copy is not None:
                backend.copy("gpu", "gpu", [copy[0]], [copy[1]])
            kr, vr = new_toks(1)
            backend.write([slot], kr, vr)
            expect[sq][0].append(kr[0])
            expect[sq][1].append(vr[0])
        elif op == 4:
            sq = live[int(rng.integers(len(live)))]
            m.free(sq)
            del expect[sq]
        else:
            sq = list(expect)[int(rng.integers(len(expect)))]
            try:
                if sq in m._swapped:
                    pairs = m.swap_in(sq)
                    backend.copy("cpu", "gpu", [c for c, _ in pairs], [g for _, g in pairs])
                else:
                    pairs = m.swap_out(sq)
                    backend.copy("gpu", "cpu", [g for g, _ in pairs], [c for _, c in pairs])
            except OutOfBlocks:
                continue
    return m, expect
