"""GPU parity of the 8-bit K/V pool (kvb_write_kv_q8, kvb_paged_decode_q8) against the
oracle (oracle/quant.py): the quantising scatter bit-exact (codes and V scales), decode
over the 8-bit pool within the decode tolerance (max abs error <= 1e-2 fp16, 2e-2 bf16).
Every expected value comes from the oracle's own quantisation of the 16-bit inputs."""
import numpy as np
import pytest

from workloads import make_config, make_custom, channel_scales
from workloads.gen import round_to_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _util():
    import gpu_util
    return gpu_util


def _pool_q8(kc, vc, vs, ks):
    import attention_paged_prefix_amd as kvb
    dev = "cuda:0"
    return kvb.PoolQ8(torch.from_numpy(np.ascontiguousarray(kc)).to(dev),
                      torch.from_numpy(np.ascontiguousarray(vc)).to(dev),
                      torch.from_numpy(np.ascontiguousarray(vs)).to(dev),
                      torch.from_numpy(np.ascontiguousarray(ks)).to(dev))


def _poisoned(nb, hkv, d):
    """Unwritten slots: codes at the extremes and NaN V scales, so a read of one shows."""
    return (np.full((nb, hkv, 16, d), 127, np.int8), np.full((nb, hkv, 16, d), -127, np.int8),
            np.full((nb, hkv, 16), np.nan, np.float32))


def _context_slots(w, seqs=None):
    """Distinct pool slots of the contexts of a decode workload (shared blocks once)."""
    slots = []
    for b in (range(w.batch) if seqs is None else seqs):
        n = int(w.context_lens[b])
        j = np.arange(n)
        slots.append(w.block_tables[b][j // 16].astype(np.int64) * 16 + j % 16)
    return np.unique(np.concatenate(slots)) if slots else np.zeros(0, np.int64)


def _tokens_at(pool_bits, slots):
    return np.ascontiguousarray(pool_bits[slots // 16, :, slots % 16, :])


@pytest.mark.parametrize("dt,d,hkv", [("bf16", 128, 8), ("fp16", 96, 2), ("bf16", 64, 1),
                                      ("fp16", 128, 4)])
def test_write_kv_q8_bit_exact(dt, d, hkv):
    from oracle import quant
    u = _util()
    rng = np.random.default_rng(801 + d + hkv)
    nb, T = 12, 150
    mag = rng.uniform(0.05, 20.0, size=(T, hkv, 1))
    K = rng.standard_normal((T, hkv, d)) * mag
    V = rng.standard_normal((T, hkv, d)) * mag
    V[7] = 0.0                                            # a zero token: scale 0, codes 0
    kb, vb = round_to_bits(K, dt), round_to_bits(V, dt)
    k_scale = channel_scales(oracle_f32(kb, dt)) * np.float32(0.8)   # some codes clamp
    k_scale[0, 3] = 0.0                                   # a zero channel scale
    slots = rng.permutation(nb * 16)[:T].astype(np.int64)
    slots[[2, 50]] = -1
    slots[60] = nb * 16 + 5                               # outside the pool: skipped
    kc0 = rng.integers(-127, 128, size=(nb, hkv, 16, d)).astype(np.int8)
    vc0 = rng.integers(-127, 128, size=(nb, hkv, 16, d)).astype(np.int8)
    vs0 = rng.uniform(0, 1, size=(nb, hkv, 16)).astype(np.float32)
    ref = quant.write_kv_q8(kc0, vc0, vs0, k_scale, kb, vb, np.where(slots < nb * 16, slots, -1), dt)
    pool = _pool_q8(kc0, vc0, vs0, k_scale)
    import attention_paged_prefix_amd as kvb
    kvb.write_kv_q8(pool, u.to_dev(kb, dt), u.to_dev(vb, dt), u.idev(slots, torch.int64))
    torch.cuda.synchronize()
    assert np.array_equal(pool.k.cpu().numpy(), ref[0])
    assert np.array_equal(pool.v.cpu().numpy(), ref[1])
    assert np.array_equal(pool.v_scale.cpu().numpy().view(np.uint32), ref[2].view(np.uint32))


def oracle_f32(bits, dt):
    import oracle
    return oracle.decode_bits(bits, dt).astype(np.float32)


Q8_DECODE_CASES = [
    (811, "bf16", 32, 8, 128, [517, 1, 16, 17, 4001, 2048]),
    (812, "fp16", 8, 8, 64, [3, 64, 100, 0]),
    (813, "fp16", 40, 8, 96, [1000, 33]),
    (814, "bf16", 16, 2, 128, [300, 2000, 15]),
]


def _oracle_q8_pool(w, slots):
    """The oracle's 8-bit pool of a decode workload: K scales from the context tokens,
    every context slot written by the oracle, the other slots poisoned."""
    from oracle import quant
    kt, vt = _tokens_at(w.k_pool, slots), _tokens_at(w.v_pool, slots)
    k_scale = channel_scales(oracle_f32(kt, w.dtype)) if len(slots) \
        else np.full((w.num_kv_heads, w.head_dim), 0.01, np.float32)
    kc, vc, vs = _poisoned(w.k_pool.shape[0], w.num_kv_heads, w.head_dim)
    kc, vc, vs = quant.write_kv_q8(kc, vc, vs, k_scale, kt, vt, slots, w.dtype)
    return kc, vc, vs, k_scale, kt, vt


@pytest.mark.parametrize("case", Q8_DECODE_CASES, ids=lambda c: f"seed{c[0]}_{c[1]}_d{c[4]}")
@pytest.mark.parametrize("split", [0, 3])
def test_decode_q8_matches_oracle(case, split):
    """Decode over an 8-bit pool the oracle wrote, against the oracle's decode over it."""
    import attention_paged_prefix_amd as kvb
    from oracle import quant
    u = _util()
    seed, dt, hq, hkv, d, ctx = case
    w = make_custom(seed, dt, hq, hkv, d, ctx, kind="decode", share="all", poison=False)
    kc, vc, vs, ks, _, _ = _oracle_q8_pool(w, _context_slots(w))
    pool = _pool_q8(kc, vc, vs, ks)
    got = u.to_bits(kvb.paged_decode_q8(pool, u.to_dev(w.q, dt), u.idev(w.context_lens),
                                        u.idev(w.block_tables), w.scale, int(max(ctx)),
                                        split_blocks=split))
    torch.cuda.synchronize()
    ref = quant.paged_decode_q8(kc, vc, vs, ks, w.q, w.context_lens, w.block_tables, w.scale, dt)
    import oracle
    assert np.isfinite(oracle.decode_bits(got, dt)).all()
    for b, n in enumerate(ctx):
        if n <= 0:
            assert (got[b] == 0).all()
    err = u.max_err(got, ref, dt)
    assert err <= u.TOL[dt], f"max abs err {err}"


def test_decode_q8_fp16_large_values_growing_scores():
    """An fp16 8-bit pool whose V values reach a few times 10^4 (V scales above 256) under
    scores that grow along the context, so that probabilities come close to 2^8 before
    each rescale: probability times V scale would leave the fp16 range, code times V
    scale does not.  Outputs finite and within 2e-3 of the largest reference value."""
    import attention_paged_prefix_amd as kvb
    import oracle
    from oracle import quant
    u = _util()
    rng = np.random.default_rng(817)
    w = make_custom(817, "fp16", 8, 2, 64, [600, 333, 17], kind="decode", share="none", poison=False)
    G = w.num_q_heads // w.num_kv_heads
    q = oracle.decode_bits(w.q, "fp16")
    k = oracle.decode_bits(w.k_pool, "fp16")
    v = oracle.decode_bits(w.v_pool, "fp16")
    for b, n in enumerate(w.context_lens):
        for j in range(int(n)):
            blk, row = int(w.block_tables[b][j // 16]), j % 16
            for h in range(w.num_kv_heads):
                k[blk, h, row, :] = q[b, h * G, :] * (6.0 * j / max(1, int(n))) + 0.1 * k[blk, h, row, :]
    v = np.clip(v * 3.0e4, -6.0e4, 6.0e4)
    w.k_pool, w.v_pool = round_to_bits(k, "fp16"), round_to_bits(v, "fp16")
    kc, vc, vs, ks, _, _ = _oracle_q8_pool(w, _context_slots(w))
    assert float(np.nanmax(vs)) > 256.0
    pool = _pool_q8(kc, vc, vs, ks)
    got = u.to_bits(kvb.paged_decode_q8(pool, u.to_dev(w.q, "fp16"), u.idev(w.context_lens),
                                        u.idev(w.block_tables), w.scale, int(w.context_lens.max())))
    torch.cuda.synchronize()
    ref = quant.paged_decode_q8(kc, vc, vs, ks, w.q, w.context_lens, w.block_tables, w.scale, "fp16")
    vals = oracle.decode_bits(got, "fp16")
    assert np.isfinite(vals).all()
    err = float(np.max(np.abs(vals - ref)))
    assert err <= 2e-3 * float(np.max(np.abs(ref))), f"max abs err {err} of {float(np.max(np.abs(ref)))}"


@pytest.mark.parametrize("bits", [8, 4])
def test_decode_quant_every_context_empty_gives_zero_rows(bits):
    """max_context_len 0 over the 8-bit and 4-bit pools: zero rows, through the workspace
    the size query reports."""
    import attention_paged_prefix_amd as kvb
    u = _util()
    w = make_custom(818, "bf16", 8, 2, 128, [0, 0], kind="decode", poison=False)
    nb = w.k_pool.shape[0]
    kc, vc, vs = _poisoned(nb, 2, 128) if bits == 8 else _poisoned4(nb, 2, 128)
    ks = np.full((2, 128), 0.01, np.float32)
    pool = _pool_q8(kc, vc, vs, ks) if bits == 8 else _pool_q4(kc, vc, vs, ks)
    fn = kvb.paged_decode_q8 if bits == 8 else kvb.paged_decode_q4
    out = torch.full_like(u.to_dev(w.q, "bf16"), 7.0)
    fn(pool, u.to_dev(w.q, "bf16"), u.idev(w.context_lens), u.idev(w.block_tables), w.scale, 0, out=out)
    torch.cuda.synchronize()
    assert (u.to_bits(out) == 0).all()


def test_write_then_decode_q8_end_to_end():
    """Every context token written by the GPU's quantising scatter, then decoded on the
    GPU; the oracle writes and decodes the same tokens itself."""
    import attention_paged_prefix_amd as kvb
    from oracle import quant
    u = _util()
    w = make_custom(815, "bf16", 32, 8, 128, [700, 2049, 16, 1333], kind="decode", share="pairs",
                    poison=False)
    slots = _context_slots(w)
    kc, vc, vs, ks, kt, vt = _oracle_q8_pool(w, slots)
    pk, pv, ps = _poisoned(w.k_pool.shape[0], 8, 128)
    pool = _pool_q8(pk, pv, ps, ks)
    kvb.write_kv_q8(pool, u.to_dev(kt, "bf16"), u.to_dev(vt, "bf16"), u.idev(slots, torch.int64))
    got = u.to_bits(kvb.paged_decode_q8(pool, u.to_dev(w.q, "bf16"), u.idev(w.context_lens),
                                        u.idev(w.block_tables), w.scale, int(w.context_lens.max())))
    torch.cuda.synchronize()
    assert np.array_equal(pool.k.cpu().numpy(), kc) and np.array_equal(pool.v.cpu().numpy(), vc)
    ref = quant.paged_decode_q8(kc, vc, vs, ks, w.q, w.context_lens, w.block_tables, w.scale, "bf16")
    assert u.max_err(got, ref, "bf16") <= u.TOL["bf16"]


def test_decode_q8_full_size_sampled():
    """The paged-decode workload (64 sequences, contexts 512..4096, 1024 shared tokens,
    32/8 heads, d=128, bf16) through the 8-bit pool, in the benchmark's launch
    configuration; eight sequences checked against the oracle, which quantises and
    decodes their tokens itself."""
    import attention_paged_prefix_amd as kvb
    from oracle import quant
    u = _util()
    w = make_config("decode")
    slots = _context_slots(w)
    kt, vt = _tokens_at(w.k_pool, slots), _tokens_at(w.v_pool, slots)
    ks = channel_scales(oracle_f32(kt, "bf16"))
    pk, pv, ps = _poisoned(w.k_pool.shape[0], 8, 128)
    pool = _pool_q8(pk, pv, ps, ks)
    kvb.write_kv_q8(pool, u.to_dev(kt, "bf16"), u.to_dev(vt, "bf16"), u.idev(slots, torch.int64))
    got = u.to_bits(kvb.paged_decode_q8(pool, u.to_dev(w.q, "bf16"), u.idev(w.context_lens),
                                        u.idev(w.block_tables), w.scale, int(w.context_lens.max())))
    torch.cuda.synchronize()
    seqs = [0, 5, 17, 31, 40, 47, 58, 63]
    sl = _context_slots(w, seqs)
    kc, vc, vs = _poisoned(w.k_pool.shape[0], 8, 128)
    kc, vc, vs = quant.write_kv_q8(kc, vc, vs, ks, _tokens_at(w.k_pool, sl), _tokens_at(w.v_pool, sl),
                                   sl, "bf16")
    ref = quant.paged_decode_q8(kc, vc, vs, ks, w.q[seqs], w.context_lens[seqs],
                                w.block_tables[seqs], w.scale, "bf16")
    assert u.max_err(got[seqs], ref, "bf16") <= u.TOL["bf16"]


Q8_PREFILL_CASES = [
    # seed, dtype, Hq, Hkv, d, prefix lengths, chunk lengths, sharing
    (821, "bf16", 16, 2, 128, [0, 100, 513, 2048], [37, 200, 1, 64], "pairs"),
    (822, "fp16", 40, 8, 96, [700, 33], [129, 300], "none"),
    (823, "bf16", 8, 8, 64, [17, 1000, 256], [16, 50, 99], "all"),
    # several rounds of work-groups (dispatch plan; a prefix past 64 tiles refills the
    # per-wave tile table, whose codes are staged one tile ahead)
    (824, "fp16", 32, 8, 128, [4500, 100, 0, 2047], [512, 480, 300, 511], "pairs"),
]


def _prefix_slots(w):
    slots = []
    for b in range(w.batch):
        j = np.arange(int(w.prefix_lens[b]))
        slots.append(w.block_tables[b][j // 16].astype(np.int64) * 16 + j % 16)
    return np.unique(np.concatenate(slots)) if slots else np.zeros(0, np.int64)


@pytest.mark.parametrize("case", Q8_PREFILL_CASES, ids=lambda c: f"seed{c[0]}_{c[1]}_d{c[4]}")
def test_prefill_q8_matches_oracle(case):
    """Prefill with the cached prefix in an 8-bit pool the oracle wrote (unwritten slots
    poisoned, NaN V scales included), against the oracle's prefill over that pool."""
    import attention_paged_prefix_amd as kvb
    from oracle import quant
    u = _util()
    seed, dt, hq, hkv, d, P, C, share = case
    w = make_custom(seed, dt, hq, hkv, d, P, C, share=share, poison=False)
    slots = _prefix_slots(w)
    kt, vt = _tokens_at(w.k_pool, slots), _tokens_at(w.v_pool, slots)
    ks = channel_scales(oracle_f32(kt, dt)) if len(slots) else np.full((hkv, d), 0.01, np.float32)
    kc, vc, vs = _poisoned(w.k_pool.shape[0], hkv, d)
    kc, vc, vs = quant.write_kv_q8(kc, vc, vs, ks, kt, vt, slots, dt)
    pool = _pool_q8(kc, vc, vs, ks)
    mq, mp = int(w.q_lens.max()), int(w.prefix_lens.max())
    got = u.to_bits(kvb.paged_prefill_q8(pool, u.to_dev(w.q, dt), u.to_dev(w.k_new, dt),
                                         u.to_dev(w.v_new, dt), u.idev(w.cu_q_lens),
                                         u.idev(w.prefix_lens), u.idev(w.block_tables), w.scale, mq, mp))
    torch.cuda.synchronize()
    import oracle
    assert np.isfinite(oracle.decode_bits(got, dt)).all()
    ref = quant.paged_prefill_q8(kc, vc, vs, ks, w.q, w.k_new, w.v_new, w.cu_q_lens, w.prefix_lens,
                                 w.block_tables, hq, w.scale, dt)
    err = u.max_err(got, ref, dt)
    assert err <= u.TOL[dt], f"max abs err {err}"


@pytest.mark.parametrize("name,bits", [("ragged_d96", 8), ("ragged_d96", 4), ("long_prefix", 8)])
def test_prefill_quant_full_size_sampled(name, bits):
    """The benchmark's quantised-pool prefill at full size, in its launch configuration:
    the prefix tokens written by kvb_write_kv_q8/_q4 into a poisoned pool (K scales from
    their per-channel maxima), then sampled rows (first/last, tile and block edges, random;
    heads at GQA group edges) of a few sequences against the oracle, which quantises those
    sequences' tokens itself."""
    import attention_paged_prefix_amd as kvb
    import oracle
    from oracle import quant
    u = _util()
    w = make_config(name)
    dt, hq, hkv, d = w.dtype, w.num_q_heads, w.num_kv_heads, w.head_dim
    cmax = 127 if bits == 8 else 7
    slots = _prefix_slots(w)
    kt, vt = _tokens_at(w.k_pool, slots), _tokens_at(w.v_pool, slots)
    ks = channel_scales(oracle_f32(kt, dt), cmax)
    nb = w.k_pool.shape[0]
    pool = kvb.PoolQ8.empty(nb, hkv, d, torch.from_numpy(ks), device="cuda:0", bits=bits)
    pool.k.fill_(127 if bits == 8 else 0x77)          # unwritten codes at the extremes
    pool.v.fill_(-127 if bits == 8 else 0x99)
    pool.v_scale.fill_(float("nan"))                  # and NaN V scales
    kvb.write_kv_q8(pool, u.to_dev(kt, dt), u.to_dev(vt, dt), u.idev(slots, torch.int64))
    del kt, vt
    got = u.to_bits(kvb.paged_prefill_q8(pool, u.to_dev(w.q, dt), u.to_dev(w.k_new, dt),
                                         u.to_dev(w.v_new, dt), u.idev(w.cu_q_lens),
                                         u.idev(w.prefix_lens), u.idev(w.block_tables), w.scale,
                                         int(w.q_lens.max()), int(w.prefix_lens.max())))
    torch.cuda.synchronize()
    vals = oracle.decode_bits(got, dt)
    assert np.isfinite(vals).all()
    rng = np.random.default_rng(97)
    B = w.batch
    seqs = sorted(set([0, B - 1] + [int(x) for x in rng.integers(0, B, size=min(B, 4))]))
    select = []
    for b in seqs:
        C = int(w.q_lens[b])
        if C == 0:
            continue
        cand = {0, 1, 15, 16, 31, 32, 63, 64, 127, 128, C // 2, C - 2, C - 1}
        cand |= set(int(x) for x in rng.integers(0, C, size=4))
        rows = sorted(r for r in cand if 0 <= r < C)
        G = hq // hkv
        heads = sorted(h for h in {0, G - 1, G, hq - 1, int(rng.integers(0, hq))} if 0 <= h < hq)
        for h in heads:
            select.append((b, h, rows))
    sl = []
    for b in seqs:
        j = np.arange(int(w.prefix_lens[b]))
        sl.append(w.block_tables[b][j // 16].astype(np.int64) * 16 + j % 16)
    sl = np.unique(np.concatenate(sl))
    kc = np.full((nb, hkv, 16, d), 127, np.int8)
    vc = np.full((nb, hkv, 16, d), -127, np.int8)
    vs = np.full((nb, hkv, 16), np.nan, np.float32)
    kc, vc, vs = quant.write_kv_q8(kc, vc, vs, ks, _tokens_at(w.k_pool, sl), _tokens_at(w.v_pool, sl),
                                   sl, dt, cmax)
    ref = quant.paged_prefill_q8(kc, vc, vs, ks, w.q, w.k_new, w.v_new, w.cu_q_lens, w.prefix_lens,
                                 w.block_tables, hq, w.scale, dt, select=select)
    worst = 0.0
    for (b, h, rows) in select:
        g = vals[w.cu_q_lens[b] + np.asarray(rows), h]
        worst = max(worst, float(np.max(np.abs(g - ref[(b, h)]))))
    assert worst <= u.TOL[dt], f"max abs err {worst}"


# ------------------------------------------------------------------ 4-bit pool

def _pool_q4(kc, vc, vs, ks):
    """Upload the oracle's (unpacked) 4-bit codes as stored bytes."""
    import attention_paged_prefix_amd as kvb
    from oracle import quant
    dev = "cuda:0"
    return kvb.PoolQ4(torch.from_numpy(np.ascontiguousarray(quant.pack_nibbles(kc))).to(dev),
                      torch.from_numpy(np.ascontiguousarray(quant.pack_nibbles(vc))).to(dev),
                      torch.from_numpy(np.ascontiguousarray(vs)).to(dev),
                      torch.from_numpy(np.ascontiguousarray(ks)).to(dev))


def _poisoned4(nb, hkv, d):
    return (np.full((nb, hkv, 16, d), 7, np.int8), np.full((nb, hkv, 16, d), -7, np.int8),
            np.full((nb, hkv, 16), np.nan, np.float32))


@pytest.mark.parametrize("dt,d,hkv", [("bf16", 128, 8), ("fp16", 96, 2), ("bf16", 64, 1)])
def test_write_kv_q4_bit_exact(dt, d, hkv):
    import attention_paged_prefix_amd as kvb
    from oracle import quant
    u = _util()
    rng = np.random.default_rng(831 + d)
    nb, T = 12, 150
    mag = rng.uniform(0.05, 20.0, size=(T, hkv, 1))
    kb = round_to_bits(rng.standard_normal((T, hkv, d)) * mag, dt)
    V = rng.standard_normal((T, hkv, d)) * mag
    V[9] = 0.0
    vb = round_to_bits(V, dt)
    ks = channel_scales(oracle_f32(kb, dt), quant.CODE_MAX4) * np.float32(0.7)
    ks[0, 5] = 0.0
    slots = rng.permutation(nb * 16)[:T].astype(np.int64)
    slots[[3, 40]] = -1
    kc0 = rng.integers(-7, 8, size=(nb, hkv, 16, d)).astype(np.int8)
    vc0 = rng.integers(-7, 8, size=(nb, hkv, 16, d)).astype(np.int8)
    vs0 = rng.uniform(0, 1, size=(nb, hkv, 16)).astype(np.float32)
    ref = quant.write_kv_q8(kc0, vc0, vs0, ks, kb, vb, slots, dt, quant.CODE_MAX4)
    pool = _pool_q4(kc0, vc0, vs0, ks)
    kvb.write_kv_q4(pool, u.to_dev(kb, dt), u.to_dev(vb, dt), u.idev(slots, torch.int64))
    torch.cuda.synchronize()
    assert np.array_equal(pool.k.cpu().numpy(), quant.pack_nibbles(ref[0]))
    assert np.array_equal(pool.v.cpu().numpy(), quant.pack_nibbles(ref[1]))
    assert np.array_equal(pool.v_scale.cpu().numpy().view(np.uint32), ref[2].view(np.uint32))


def _oracle_q4_pool(w, slots):
    from oracle import quant
    kt, vt = _tokens_at(w.k_pool, slots), _tokens_at(w.v_pool, slots)
    ks = channel_scales(oracle_f32(kt, w.dtype), quant.CODE_MAX4) if len(slots) \
        else np.full((w.num_kv_heads, w.head_dim), 0.1, np.float32)
    kc, vc, vs = _poisoned4(w.k_pool.shape[0], w.num_kv_heads, w.head_dim)
    kc, vc, vs = quant.write_kv_q8(kc, vc, vs, ks, kt, vt, slots, w.dtype, quant.CODE_MAX4)
    return kc, vc, vs, ks, kt, vt


@pytest.mark.parametrize("case", Q8_DECODE_CASES, ids=lambda c: f"seed{c[0]}_{c[1]}_d{c[4]}")
@pytest.mark.parametrize("split", [0, 3])
def test_decode_q4_matches_oracle(case, split):
    import attention_paged_prefix_amd as kvb
    from oracle import quant
    u = _util()
    seed, dt, hq, hkv, d, ctx = case
    w = make_custom(seed, dt, hq, hkv, d, ctx, kind="decode", share="all", poison=False)
    kc, vc, vs, ks, _, _ = _oracle_q4_pool(w, _context_slots(w))
    pool = _pool_q4(kc, vc, vs, ks)
    got = u.to_bits(kvb.paged_decode_q4(pool, u.to_dev(w.q, dt), u.idev(w.context_lens),
                                        u.idev(w.block_tables), w.scale, int(max(ctx)),
                                        split_blocks=split))
    torch.cuda.synchronize()
    ref = quant.paged_decode_q8(kc, vc, vs, ks, w.q, w.context_lens, w.block_tables, w.scale, dt)
    err = u.max_err(got, ref, dt)
    assert err <= u.TOL[dt], f"max abs err {err}"


@pytest.mark.parametrize("case", Q8_PREFILL_CASES, ids=lambda c: f"seed{c[0]}_{c[1]}_d{c[4]}")
def test_prefill_q4_matches_oracle(case):
    import attention_paged_prefix_amd as kvb
    from oracle import quant
    u = _util()
    seed, dt, hq, hkv, d, P, C, share = case
    w = make_custom(seed, dt, hq, hkv, d, P, C, share=share, poison=False)
    kc, vc, vs, ks, _, _ = _oracle_q4_pool(w, _prefix_slots(w))
    pool = _pool_q4(kc, vc, vs, ks)
    got = u.to_bits(kvb.paged_prefill_q4(pool, u.to_dev(w.q, dt), u.to_dev(w.k_new, dt),
                                         u.to_dev(w.v_new, dt), u.idev(w.cu_q_lens),
                                         u.idev(w.prefix_lens), u.idev(w.block_tables), w.scale,
                                         int(w.q_lens.max()), int(w.prefix_lens.max())))
    torch.cuda.synchronize()
    ref = quant.paged_prefill_q8(kc, vc, vs, ks, w.q, w.k_new, w.v_new, w.cu_q_lens, w.prefix_lens,
                                 w.block_tables, hq, w.scale, dt)
    err = u.max_err(got, ref, dt)
    assert err <= u.TOL[dt], f"max abs err {err}"


def test_write_then_decode_q4_end_to_end():
    import attention_paged_prefix_amd as kvb
    from oracle import quant
    u = _util()
    w = make_custom(835, "fp16", 32, 8, 128, [700, 2049, 16, 1333], kind="decode", share="pairs",
                    poison=False)
    slots = _context_slots(w)
    kc, vc, vs, ks, kt, vt = _oracle_q4_pool(w, slots)
    pk, pv, ps = _poisoned4(w.k_pool.shape[0], 8, 128)
    pool = _pool_q4(pk, pv, ps, ks)
    kvb.write_kv_q4(pool, u.to_dev(kt, "fp16"), u.to_dev(vt, "fp16"), u.idev(slots, torch.int64))
    got = u.to_bits(kvb.paged_decode_q4(pool, u.to_dev(w.q, "fp16"), u.idev(w.context_lens),
                                        u.idev(w.block_tables), w.scale, int(w.context_lens.max())))
    torch.cuda.synchronize()
    assert np.array_equal(pool.k.cpu().numpy(), quant.pack_nibbles(kc))
    ref = quant.paged_decode_q8(kc, vc, vs, ks, w.q, w.context_lens, w.block_tables, w.scale, "fp16")
    assert u.max_err(got, ref, "fp16") <= u.TOL["fp16"]


@pytest.mark.parametrize("bits,dt", [(8, "fp16"), (4, "fp16"), (8, "bf16")])
def test_prefill_quant_eight_row_waves_matches_oracle(bits, dt):
    """Head dim 96 through a quantised pool on a grid of at least four rounds of 256-row
    work-groups, the form with 8 row waves (K blocks staged by waves 0-3, V blocks by 4-7),
    every output row against the oracle: prefixes of 0, 1, 63, 64 and 65 tokens, one past
    64 tiles (table refill with codes staged a tile ahead), chunks of 1 to 200 tokens."""
    import attention_paged_prefix_amd as kvb
    from oracle import quant
    u = _util()
    rng = np.random.default_rng(860 + bits)
    batch, hq, hkv, d = 32, 32, 8, 96
    P = [0, 1, 63, 64, 65, 4500] + [int(x) for x in rng.integers(0, 3000, size=batch - 6)]
    C = [200, 1, 17, 64, 129, 150] + [int(x) for x in rng.integers(1, 201, size=batch - 6)]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert batch * hkv * ((max(C) * (hq // hkv) + 255) // 256) >= 4 * cus
    w = make_custom(870 + bits, dt, hq, hkv, d, P, C, share="pairs", poison=False)
    slots = _prefix_slots(w)
    if bits == 8:
        kt, vt = _tokens_at(w.k_pool, slots), _tokens_at(w.v_pool, slots)
        ks = channel_scales(oracle_f32(kt, dt))
        kc, vc, vs = _poisoned(w.k_pool.shape[0], hkv, d)
        kc, vc, vs = quant.write_kv_q8(kc, vc, vs, ks, kt, vt, slots, dt)
        pool = _pool_q8(kc, vc, vs, ks)
        fn = kvb.paged_prefill_q8
    else:
        kc, vc, vs, ks, _, _ = _oracle_q4_pool(w, slots)
        pool = _pool_q4(kc, vc, vs, ks)
        fn = kvb.paged_prefill_q4
    got = u.to_bits(fn(pool, u.to_dev(w.q, dt), u.to_dev(w.k_new, dt), u.to_dev(w.v_new, dt),
                       u.idev(w.cu_q_lens), u.idev(w.prefix_lens), u.idev(w.block_tables), w.scale,
                       int(w.q_lens.max()), int(w.prefix_lens.max())))
    torch.cuda.synchronize()
    ref = quant.paged_prefill_q8(kc, vc, vs, ks, w.q, w.k_new, w.v_new, w.cu_q_lens, w.prefix_lens,
                                 w.block_tables, hq, w.scale, dt)
    err = u.max_err(got, ref, dt)
    assert err <= u.TOL[dt], f"max abs err {err}"
