"""Seeded random GPU parity sweep: random shapes (dtype, head dim, KV heads, GQA group up to 32,
batch, prefix and chunk lengths with a bias toward block and tile edges, sharing) through
the prefill (plain, with the fused slot scatter, pooled; empty chunks inside a batch; both
pool layouts; block-table rows longer than needed; host bounds above the batch's), the
decode (split plans forced at random, both pool layouts), the cascade decode and the 8-bit
and 4-bit pools, each against the oracle within the decode/prefill tolerance.  Every
failing case is reported with its parameters."""
import numpy as np
import pytest

from workloads import make_custom

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

EDGE = [0, 1, 15, 16, 17, 63, 64, 65, 127, 128, 129]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


class Sweep:
    def __init__(self, seed):
        import gpu_util
        self.u = gpu_util
        self.rng = np.random.default_rng(seed)
        self.bad = []

    def lens(self, k, lo, hi):
        r = self.rng
        return [int(r.choice(EDGE)) if r.random() < 0.35 else int(r.integers(lo, hi)) for _ in range(k)]

    def shape(self):
        r = self.rng
        dt = str(r.choice(["fp16", "bf16"]))
        d = int(r.choice([64, 96, 128]))
        hkv = int(r.choice([1, 2, 4, 8]))
        if r.random() < 0.2:                        # groups at and past 16 query heads
            return dt, d, min(hkv, 2), min(hkv, 2) * int(r.choice([16, 17, 20, 32]))
        return dt, d, hkv, hkv * int(r.choice([1, 2, 3, 4, 5, 8]))

    def check(self, kind, got_bits, ref, dt, case):
        import oracle
        vals = oracle.decode_bits(got_bits, dt)
        err = float(np.max(np.abs(vals - ref))) if vals.size else 0.0
        if not np.isfinite(vals).all() or not err <= self.u.TOL[dt]:
            self.bad.append((kind, err, case))


@pytest.mark.parametrize("seed", [31, 32])
def test_random_prefill(seed):
    import attention_paged_prefix_amd as kvb
    import oracle
    s = Sweep(seed)
    u, r = s.u, s.rng
    for i in range(24):
        dt, d, hkv, hq = s.shape()
        B = int(r.integers(1, 6))
        P = s.lens(B, 0, 1500)
        C = [0 if r.random() < 0.15 else max(1, c) for c in s.lens(B, 1, 260)]
        if max(C) == 0:
            C[0] = 3
        share = str(r.choice(["none", "pairs", "all"]))
        extra = int(r.choice([0, 0, 3]))            # block-table rows longer than needed
        case = (seed * 1000 + i, dt, hq, hkv, d, P, C, share, extra)
        w = make_custom(case[0], dt, hq, hkv, d, P, C, share=share, poison=True, stride_extra=extra)
        layout = str(r.choice(["split", "interleaved"]))
        dev = u.Dev(w, pool_layout=layout)
        got = u.to_bits(dev.prefill())
        torch.cuda.synchronize()
        ref = u.oracle_prefill(w)
        s.check("prefill", got, ref, dt, case + (layout,))
        # host bounds larger than the batch's (allowed up to total_q: only idle work-groups)
        loose = u.to_bits(kvb.paged_prefill(dev.pool, dev.q, dev.k_new, dev.v_new, dev.cu, dev.pl, dev.bt,
                                            w.scale, min(int(w.q_lens.max()) + 17, int(w.total_q)),
                                            int(w.prefix_lens.max()) + 16 * extra))
        torch.cuda.synchronize()
        if not np.array_equal(loose, got):
            s.bad.append(("prefill_loose_bounds", None, case))
        if layout == "interleaved":                  # the scatter checks below read dev.k / dev.v
            continue
        out = kvb.paged_prefill(dev.pool, dev.q, dev.k_new, dev.v_new, dev.cu, dev.pl, dev.bt, w.scale,
                                int(w.q_lens.max()), int(w.prefix_lens.max()), slot_mapping=dev.slots)
        torch.cuda.synchronize()
        ek, ev = oracle.write_kv(w.k_pool, w.v_pool, w.k_new, w.v_new, w.slot_mapping)
        if not (np.array_equal(u.to_bits(out), got) and np.array_equal(u.to_bits(dev.k), ek)
                and np.array_equal(u.to_bits(dev.v), ev)):
            s.bad.append(("prefill_write", None, case))
        pooled = u.to_bits(kvb.paged_prefill_pooled(dev.pool, dev.q, dev.cu, dev.pl, dev.bt, w.scale,
                                                    int(w.q_lens.max()), int(w.prefix_lens.max())))
        torch.cuda.synchronize()
        s.check("pooled", pooled, ref, dt, case)
    assert not s.bad, s.bad


@pytest.mark.parametrize("seed", [41, 42])
def test_random_decode_and_cascade(seed):
    import attention_paged_prefix_amd as kvb
    s = Sweep(seed)
    u, r = s.u, s.rng
    for i in range(20):
        dt, d, hkv, hq = s.shape()
        B = int(r.integers(1, 40))
        ctx = s.lens(B, 0, 3000)
        share = str(r.choice(["none", "pairs", "all"]))
        sb = int(r.choice([0, 0, 1, 3, 17, 64]))
        extra = int(r.choice([0, 0, 3]))
        layout = str(r.choice(["split", "interleaved"]))
        case = (seed * 1000 + i, dt, hq, hkv, d, ctx, share, sb, extra, layout)
        w = make_custom(case[0], dt, hq, hkv, d, ctx, kind="decode", share=share, poison=True,
                        stride_extra=extra)
        got = u.to_bits(u.Dev(w, pool_layout=layout).decode(split_blocks=sb))
        torch.cuda.synchronize()
        s.check("decode", got, u.oracle_decode(w), dt, case)
    for i in range(8):
        dt, d, hkv, hq = s.shape()
        B = int(r.integers(2, 24))
        nsh = int(r.integers(1, 40))
        ctx = [nsh * 16 + int(x) for x in r.integers(0, 900, size=B)]
        case = (seed * 1000 + 500 + i, dt, hq, hkv, d, ctx, nsh)
        w = make_custom(case[0], dt, hq, hkv, d, ctx, kind="decode", share="all", poison=True)
        tabs = w.block_tables
        if any(not np.array_equal(tabs[b][:nsh], tabs[0][:nsh]) for b in range(B)):
            continue
        dev = u.Dev(w)
        got = u.to_bits(kvb.paged_decode_cascade(dev.pool, dev.q, dev.ctx, dev.bt, u.idev(tabs[0][:nsh]),
                                                 nsh * 16, w.scale, int(max(ctx))))
        torch.cuda.synchronize()
        s.check("cascade", got, u.oracle_decode(w), dt, case)
    assert not s.bad, s.bad


@pytest.mark.parametrize("seed", [51, 52])
def test_random_quantised_pools(seed):
    import attention_paged_prefix_amd as kvb
    from oracle import quant
    import test_gpu_q8 as tq
    s = Sweep(seed)
    u, r = s.u, s.rng
    for i in range(12):
        dt, d, hkv, hq = s.shape()
        bits = 8 if i % 2 == 0 else 4
        B = int(r.integers(1, 12))
        ctx = s.lens(B, 1, 2000)
        case = (seed * 1000 + i, dt, hq, hkv, d, ctx, bits)
        w = make_custom(case[0], dt, hq, hkv, d, ctx, kind="decode", share="all", poison=False)
        slots = tq._context_slots(w)
        make = (tq._oracle_q8_pool, tq._pool_q8, kvb.paged_decode_q8, kvb.paged_prefill_q8) if bits == 8 \
            else (tq._oracle_q4_pool, tq._pool_q4, kvb.paged_decode_q4, kvb.paged_prefill_q4)
        kc, vc, vs, ks, _, _ = make[0](w, slots)
        got = u.to_bits(make[2](make[1](kc, vc, vs, ks), u.to_dev(w.q, dt), u.idev(w.context_lens),
                                u.idev(w.block_tables), w.scale, int(max(ctx))))
        torch.cuda.synchronize()
        ref = quant.paged_decode_q8(kc, vc, vs, ks, w.q, w.context_lens, w.block_tables, w.scale, dt)
        s.check(f"decode_q{bits}", got, ref, dt, case)
        P, C = s.lens(B, 0, 1500), [max(1, c) for c in s.lens(B, 1, 200)]
        case = (seed * 1000 + 100 + i, dt, hq, hkv, d, P, C, bits)
        wp = make_custom(case[0], dt, hq, hkv, d, P, C, share="pairs", poison=False)
        ps = tq._prefix_slots(wp)
        if len(ps) == 0:
            continue
        kc, vc, vs, ks, _, _ = make[0](wp, ps)
        got = u.to_bits(make[3](make[1](kc, vc, vs, ks), u.to_dev(wp.q, dt), u.to_dev(wp.k_new, dt),
                                u.to_dev(wp.v_new, dt), u.idev(wp.cu_q_lens), u.idev(wp.prefix_lens),
                                u.idev(wp.block_tables), wp.scale, int(wp.q_lens.max()),
                                int(wp.prefix_lens.max())))
        torch.cuda.synchronize()
        ref = quant.paged_prefill_q8(kc, vc, vs, ks, wp.q, wp.k_new, wp.v_new, wp.cu_q_lens,
                                     wp.prefix_lens, wp.block_tables, hq, wp.scale, dt)
        s.check(f"prefill_q{bits}", got, ref, dt, case)
    assert not s.bad, s.bad
