"""GPU parity at the full benchmark sizes, in the launch configuration the benchmark
times (default split plan for decode), on sampled outputs the oracle computes one row
at a time: first and last rows, rows on tile and block edges, and a few random rows,
for query heads at GQA group edges."""
import numpy as np
import pytest

from workloads import make_config

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _util():
    import gpu_util
    return gpu_util


def _rows(C, rng):
    cand = {0, 1, 15, 16, 31, 32, 63, 64, 127, 128, C // 2, C - 2, C - 1}
    cand |= set(int(x) for x in rng.integers(0, C, size=4))
    return sorted(r for r in cand if 0 <= r < C)


def _heads(hq, hkv, rng):
    G = hq // hkv
    cand = {0, G - 1, G, hq - 1, int(rng.integers(0, hq))}
    return sorted(h for h in cand if 0 <= h < hq)


@pytest.mark.parametrize("name", ["shared_prompt", "long_prefix", "ragged_d96", "ragged_d64"])
def test_prefill_full_size_sampled(name):
    u = _util()
    w = make_config(name, poison=True)
    dev = u.Dev(w)
    got = u.to_bits(dev.prefill())
    torch.cuda.synchronize()
    import oracle
    vals = oracle.decode_bits(got, w.dtype)
    assert np.isfinite(vals).all()
    rng = np.random.default_rng(99)
    B = w.batch
    seqs = sorted(set([0, B - 1] + [int(x) for x in rng.integers(0, B, size=min(B, 4))]))
    select = []
    for b in seqs:
        C = int(w.q_lens[b])
        if C == 0:
            continue
        rows = _rows(C, rng)
        for h in _heads(w.num_q_heads, w.num_kv_heads, rng):
            select.append((b, h, rows))
    ref = oracle.paged_prefill(w.k_pool, w.v_pool, w.q, w.k_new, w.v_new, w.cu_q_lens, w.prefix_lens,
                               w.block_tables, w.num_q_heads, w.scale, w.dtype, select=select)
    worst = 0.0
    for (b, h, rows) in select:
        g = vals[w.cu_q_lens[b] + np.asarray(rows), h]
        worst = max(worst, float(np.max(np.abs(g - ref[(b, h)]))))
    assert worst <= u.TOL[w.dtype], f"max abs err {worst}"


def test_decode_full_size_sampled():
    u = _util()
    w = make_config("decode", poison=True)
    dev = u.Dev(w)
    got = u.to_bits(dev.decode(split_blocks=0))
    torch.cuda.synchronize()
    import oracle
    vals = oracle.decode_bits(got, w.dtype)
    assert np.isfinite(vals).all()
    rng = np.random.default_rng(98)
    seqs = sorted(set([0, w.batch - 1] + [int(x) for x in rng.integers(0, w.batch, size=10)]))
    ref = oracle.paged_decode(w.k_pool, w.v_pool, w.q, w.context_lens, w.block_tables, w.scale,
                              w.dtype, seqs=seqs)
    err = float(np.max(np.abs(vals[seqs] - ref[seqs])))
    assert err <= u.TOL[w.dtype], f"max abs err {err}"


def test_decode_step_full_size_sampled():
    """The decode call of the benchmark step on the ragged mix at head dim 96 (32 contexts
    of up to ~17K tokens, the chunk's and the decode token's K/V scattered into the pool
    first): the balanced form at about 62 blocks per wave, one range per resident wave."""
    import attention_paged_prefix_amd as kvb
    import oracle
    u = _util()
    w = make_config("ragged_d96", poison=True, with_decode=True)
    dev = u.Dev(w)
    kvb.write_kv(dev.pool, dev.k_new, dev.v_new, dev.slots)
    dk, dv = u.to_dev(w.dec_k, w.dtype), u.to_dev(w.dec_v, w.dtype)
    kvb.write_kv(dev.pool, dk, dv, u.idev(w.dec_slots, torch.int64))
    dq = u.to_dev(w.dec_q, w.dtype)
    ctx = w.dec_context_lens
    got = u.to_bits(kvb.paged_decode(dev.pool, dq, u.idev(ctx), dev.bt, w.scale, int(ctx.max())))
    torch.cuda.synchronize()
    ek, ev = oracle.write_kv(w.k_pool, w.v_pool, w.k_new, w.v_new, w.slot_mapping)
    ek, ev = oracle.write_kv(ek, ev, w.dec_k, w.dec_v, w.dec_slots)
    rng = np.random.default_rng(96)
    seqs = sorted(set([0, w.batch - 1, int(np.argmax(ctx))] + [int(x) for x in rng.integers(0, w.batch, size=6)]))
    ref = oracle.paged_decode(ek, ev, w.dec_q, ctx, w.block_tables, w.scale, w.dtype, seqs=seqs)
    vals = oracle.decode_bits(got, w.dtype)
    assert np.isfinite(vals).all()
    err = float(np.max(np.abs(vals[seqs] - ref[seqs])))
    assert err <= u.TOL[w.dtype], f"max abs err {err}"


def test_cascade_decode_full_size_sampled():
    """The decode workload's first 1024 tokens (64 blocks) are one shared prefix; the
    cascade form reads them once for all 64 sequences."""
    import attention_paged_prefix_amd as kvb
    u = _util()
    w = make_config("decode", poison=True)
    dev = u.Dev(w)
    members, ids = w.notes["first_group"]
    assert len(members) == w.batch and len(ids) == 64
    got = u.to_bits(kvb.paged_decode_cascade(dev.pool, dev.q, dev.ctx, dev.bt, u.idev(ids), 1024,
                                             w.scale, int(w.context_lens.max())))
    torch.cuda.synchronize()
    import oracle
    vals = oracle.decode_bits(got, w.dtype)
    assert np.isfinite(vals).all()
    rng = np.random.default_rng(97)
    seqs = sorted(set([0, w.batch - 1] + [int(x) for x in rng.integers(0, w.batch, size=10)]))
    ref = oracle.paged_decode(w.k_pool, w.v_pool, w.q, w.context_lens, w.block_tables, w.scale,
                              w.dtype, seqs=seqs)
    err = float(np.max(np.abs(vals[seqs] - ref[seqs])))
    assert err <= u.TOL[w.dtype], f"max abs err {err}"


@pytest.mark.parametrize("name", ["shared_prompt", "long_prefix"])
def test_prefill_write_full_size(name):
    """kvb_paged_prefill_write as the benchmark step runs it: the output bits of the plain
    prefill (checked against the oracle above) and the whole pool as the oracle's slot
    scatter leaves it."""
    import attention_paged_prefix_amd as kvb
    import oracle
    u = _util()
    w = make_config(name, poison=True)
    dev = u.Dev(w)
    ref = u.to_bits(dev.prefill())
    out = kvb.paged_prefill(dev.pool, dev.q, dev.k_new, dev.v_new, dev.cu, dev.pl, dev.bt, w.scale,
                            int(w.q_lens.max()), int(w.prefix_lens.max()), slot_mapping=dev.slots)
    torch.cuda.synchronize()
    assert np.array_equal(u.to_bits(out), ref)
    ek, ev = oracle.write_kv(w.k_pool, w.v_pool, w.k_new, w.v_new, w.slot_mapping)
    assert np.array_equal(u.to_bits(dev.k), ek)
    assert np.array_equal(u.to_bits(dev.v), ev)


def _tile_edge_rows(C, G, tile_rows=128):
    """First and last virtual row (v = i*G + g) of every tile of `tile_rows` virtual rows
    of one (sequence, KV head): the prefill's work items."""
    n = C * G
    rows = set()
    for t0 in range(0, n, tile_rows):
        rows.add(t0)
        rows.add(min(n, t0 + tile_rows) - 1)
    return sorted(rows)


@pytest.mark.parametrize("name", ["ragged_d96", "long_prefix", "ragged_d64", "shared_prompt"])
def test_prefill_full_size_every_work_item(name):
    """Every (sequence, KV head, 128-row tile) work item that the dispatch plan orders is
    checked at its first and last row, with the fused slot scatter and the dispatch plan
    as the benchmark step runs them (ragged_d96 with the benchmark's decode-step layout)."""
    import attention_paged_prefix_amd as kvb
    import oracle
    u = _util()
    w = make_config(name, poison=True, with_decode=(name == "ragged_d96"))
    dev = u.Dev(w)
    out = kvb.paged_prefill(dev.pool, dev.q, dev.k_new, dev.v_new, dev.cu, dev.pl, dev.bt, w.scale,
                            int(w.q_lens.max()), int(w.prefix_lens.max()), slot_mapping=dev.slots)
    torch.cuda.synchronize()
    vals = oracle.decode_bits(u.to_bits(out), w.dtype)
    assert np.isfinite(vals).all()
    G = w.num_q_heads // w.num_kv_heads
    worst, checked = 0.0, 0
    for b in range(w.batch):
        C, P = int(w.q_lens[b]), int(w.prefix_lens[b])
        if C == 0:
            continue
        c0 = int(w.cu_q_lens[b])
        for kvh in range(w.num_kv_heads):
            # the sequence's keys for this KV head: cached prefix through the table, then
            # the chunk's own rows
            K = np.concatenate([oracle.decode_bits(oracle.gather_kv(w.k_pool, w.block_tables[b], P)[:, kvh], w.dtype),
                                oracle.decode_bits(w.k_new[c0:c0 + C, kvh], w.dtype)])
            V = np.concatenate([oracle.decode_bits(oracle.gather_kv(w.v_pool, w.block_tables[b], P)[:, kvh], w.dtype),
                                oracle.decode_bits(w.v_new[c0:c0 + C, kvh], w.dtype)])
            by_head = {}
            for v in _tile_edge_rows(C, G):
                by_head.setdefault(kvh * G + v % G, []).append(v // G)
            for h, rows in by_head.items():
                rows = np.asarray(rows)
                ref, _ = oracle.attend(oracle.decode_bits(w.q[c0 + rows, h], w.dtype), K, V, P + rows,
                                       w.scale)
                worst = max(worst, float(np.max(np.abs(vals[c0 + rows, h] - ref))))
                checked += len(rows)
    assert checked > 0
    assert worst <= u.TOL[w.dtype], f"max abs err {worst} over {checked} rows"
