"""Pins for the fp64 oracle: each test checks it against something other than itself
(brute force with scalar math, hand-derived closed forms, exact invariants of
softmax attention).  CPU only."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from workloads import make_custom, round_to_bits, blocks_for

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


# ---------------------------------------------------------------- helpers (test side)

def _val(s):
    """Parse an exact expected value: a fraction 'a/b', an integer, or 'lnN'."""
    s = str(s)
    if s.startswith("ln"):
        return math.log(float(s[2:]))
    return float(Fraction(s))


def _brute_rows(q_rows, keys, values, last_visible, scale):
    """Scalar Python attention: no max shift, math.exp and math.fsum only."""
    outs = []
    for r, q in enumerate(q_rows):
        ws = []
        for j in range(last_visible[r] + 1):
            s = scale * math.fsum(float(a) * float(b) for a, b in zip(q, keys[j]))
            ws.append(math.exp(s))
        den = math.fsum(ws)
        d = len(values[0])
        outs.append([math.fsum(ws[j] * float(values[j][k]) for j in range(len(ws))) / den
                     for k in range(d)])
    return np.array(outs)


def _f64(bits, dtype):
    return oracle.decode_bits(bits, dtype)


# ---------------------------------------------------------------- payload decoding

def test_decode_bits_known_payloads():
    # IEEE half: 0x3C00 = 1, 0xC000 = -2, 0x3555 = 0.333251953125; bf16: 0x3F80 = 1, 0xC040 = -3
    assert list(oracle.decode_bits(np.array([0x3C00, 0xC000, 0x3555], np.uint16), "fp16")) == \
        [1.0, -2.0, 0.333251953125]
    assert list(oracle.decode_bits(np.array([0x3F80, 0xC040, 0x0000], np.uint16), "bf16")) == \
        [1.0, -3.0, 0.0]


# ---------------------------------------------------------------- closed forms

def _load_golden_case(c):
    dt = c["dtype"]
    Hkv, Hq, d = c["num_kv_heads"], c["num_q_heads"], c["head_dim"]
    nb = c["num_blocks"]
    kp = np.zeros((nb, Hkv, 16, d), np.float32)
    vp = np.zeros((nb, Hkv, 16, d), np.float32)
    for b in c.get("nan_blocks", []):
        kp[b] = np.nan
        vp[b] = np.nan
    for t in c["pool_tokens"]:
        kp[t["block"], :, t["row"], :] = t["k"]
        vp[t["block"], :, t["row"], :] = t["v"]
    kpb, vpb = round_to_bits(kp, dt), round_to_bits(vp, dt)
    q = round_to_bits(np.array(c["q"], np.float32), dt)
    scale = _val(c["scale"])
    bt = np.array(c["block_tables"], np.int32)
    return dt, Hq, kpb, vpb, q, scale, bt


@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"], ids=lambda c: c["name"])
def test_closed_form_golden(case):
    dt, Hq, kpb, vpb, q, scale, bt = _load_golden_case(case)
    exp_out = np.vectorize(_val)(np.array(case["expected_out"], dtype=object)).astype(np.float64)
    exp_lse = np.vectorize(_val)(np.array(case["expected_lse"], dtype=object)).astype(np.float64)
    if case["kind"] == "prefill":
        kn = round_to_bits(np.array(case["k_new"], np.float32), dt)
        vn = round_to_bits(np.array(case["v_new"], np.float32), dt)
        out, lse = oracle.paged_prefill(kpb, vpb, q, kn, vn, case["cu_q_lens"], case["prefix_lens"],
                                        bt, Hq, scale, dt, want_lse=True)
    else:
        out, lse = oracle.paged_decode(kpb, vpb, q, np.array(case["context_lens"]), bt, scale, dt,
                                       want_lse=True)
    np.testing.assert_allclose(out, exp_out, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, exp_lse, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("seed,dt,P,C,Hq,Hkv,d", [
    (11, "fp16", [5, 0, 17], [3, 4, 2], 2, 1, 4),
    (12, "bf16", [16, 3], [1, 5], 4, 2, 8),
    (13, "fp16", [0], [8], 1, 1, 3),
    (14, "bf16", [33, 1], [2, 1], 3, 3, 5),
])
def test_prefill_vs_brute_force(seed, dt, P, C, Hq, Hkv, d):
    w = make_custom(seed, dt, Hq, Hkv, d, P, C, share="pairs" if len(P) == 2 else "none")
    out = oracle.paged_prefill(w.k_pool, w.v_pool, w.q, w.k_new, w.v_new, w.cu_q_lens,
                               w.prefix_lens, w.block_tables, Hq, w.scale, dt)
    G = Hq // Hkv
    for b in range(len(P)):
        # build the logical sequence with explicit per-token loops
        keys = {g: [] for g in range(Hkv)}
        vals = {g: [] for g in range(Hkv)}
        for j in range(P[b]):
            blk = int(w.block_tables[b][j // 16])
            for g in range(Hkv):
                keys[g].append(_f64(w.k_pool[blk, g, j % 16], dt))
                vals[g].append(_f64(w.v_pool[blk, g, j % 16], dt))
        for i in range(C[b]):
            t = w.cu_q_lens[b] + i
            for g in range(Hkv):
                keys[g].append(_f64(w.k_new[t, g], dt))
                vals[g].append(_f64(w.v_new[t, g], dt))
        for h in range(Hq):
            rows = [_f64(w.q[w.cu_q_lens[b] + i, h], dt) for i in range(C[b])]
            ref = _brute_rows(rows, keys[h // G], vals[h // G], [P[b] + i for i in range(C[b])], w.scale)
            got = out[w.cu_q_lens[b]:w.cu_q_lens[b + 1], h]
            np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("seed,dt,ctx,Hq,Hkv,d", [
    (21, "bf16", [1, 7, 20, 33], 4, 2, 6),
    (22, "fp16", [16, 2], 2, 2, 8),
])
def test_decode_vs_brute_force(seed, dt, ctx, Hq, Hkv, d):
    w = make_custom(seed, dt, Hq, Hkv, d, ctx, kind="decode")
    out = oracle.paged_decode(w.k_pool, w.v_pool, w.q, w.context_lens, w.block_tables, w.scale, dt)
    for b, n in enumerate(ctx):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            keys = [_f64(w.k_pool[w.block_tables[b][j // 16], g, j % 16], dt) for j in range(n)]
            vals = [_f64(w.v_pool[w.block_tables[b][j // 16], g, j % 16], dt) for j in range(n)]
            ref = _brute_rows([_f64(w.q[b, h], dt)], keys, vals, [n - 1], w.scale)
            np.testing.assert_allclose(out[b, h], ref[0], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- invariants

def _prefill(w, **kw):
    return oracle.paged_prefill(w.k_pool, w.v_pool, w.q, w.k_new, w.v_new, w.cu_q_lens,
                                w.prefix_lens, w.block_tables, w.num_q_heads, w.scale, w.dtype, **kw)


def test_softmax_rows_sum_to_one():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((6, 16))
    K = rng.standard_normal((40, 16))
    V = rng.standard_normal((40, 16))
    _, _, wts = oracle.attend(q, K, V, [0, 5, 17, 39, 20, 39], 0.25, want_weights=True)
    np.testing.assert_allclose(wts.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    # weights beyond each row's position are exactly zero
    assert wts[0, 1:].max() == 0.0 and wts[1, 6:].max() == 0.0


def test_single_key_returns_its_value():
    # prefix 0, chunk 1: row 0 sees only itself -> exactly v_new[0] for every head
    w = make_custom(31, "bf16", 8, 2, 64, [0], [1])
    out = _prefill(w)
    for h in range(8):
        np.testing.assert_array_equal(out[0, h], _f64(w.v_new[0, h // 4], "bf16"))
    # row 0 of a longer P=0 chunk too
    w = make_custom(32, "fp16", 2, 1, 96, [0, 0], [37, 5])
    out = _prefill(w)
    np.testing.assert_array_equal(out[0, 1], _f64(w.v_new[0, 0], "fp16"))
    np.testing.assert_array_equal(out[37, 0], _f64(w.v_new[37, 0], "fp16"))


def test_equal_scores_give_mean_of_values():
    w = make_custom(33, "bf16", 4, 2, 64, [45, 16], [7, 3])
    w.q[:] = 0                      # every score is 0
    out = _prefill(w)
    for b in range(2):
        K, V = [], []
        P = int(w.prefix_lens[b])
        for j in range(P):
            V.append(_f64(w.v_pool[w.block_tables[b][j // 16], :, j % 16], "bf16"))
        for i in range(int(w.q_lens[b])):
            V.append(_f64(w.v_new[w.cu_q_lens[b] + i], "bf16"))
        V = np.array(V)                                     # [L][Hkv][d]
        for i in range(int(w.q_lens[b])):
            mean = V[:P + i + 1].mean(axis=0)
            for h in range(4):
                np.testing.assert_allclose(out[w.cu_q_lens[b] + i, h], mean[h // 2],
                                           rtol=0, atol=1e-15 * max(1.0, np.abs(V).max()))


def test_block_permutation_invariance_is_bit_exact():
    w = make_custom(34, "fp16", 4, 2, 32, [50, 20, 0], [9, 4, 6], share="none")
    ref = _prefill(w)
    rng = np.random.default_rng(1)
    perm = rng.permutation(w.num_blocks)          # new physical id of old block i is perm[i]
    kp = np.empty_like(w.k_pool)
    vp = np.empty_like(w.v_pool)
    kp[perm] = w.k_pool
    vp[perm] = w.v_pool
    bt = perm[w.block_tables].astype(np.int32)
    got = oracle.paged_prefill(kp, vp, w.q, w.k_new, w.v_new, w.cu_q_lens, w.prefix_lens, bt,
                               4, w.scale, "fp16")
    assert np.array_equal(got, ref)
    # contiguous layout: logical block j of each sequence stored at consecutive ids
    nb = [blocks_for(int(p)) for p in w.prefix_lens]
    kc = np.zeros((sum(nb) + 1,) + w.k_pool.shape[1:], np.uint16)
    vc = np.zeros_like(kc)
    btc = np.zeros_like(w.block_tables)
    base = 0
    for b in range(3):
        for j in range(nb[b]):
            kc[base + j] = w.k_pool[w.block_tables[b][j]]
            vc[base + j] = w.v_pool[w.block_tables[b][j]]
            btc[b, j] = base + j
        base += nb[b]
    got2 = oracle.paged_prefill(kc, vc, w.q, w.k_new, w.v_new, w.cu_q_lens, w.prefix_lens, btc,
                                4, w.scale, "fp16")
    assert np.array_equal(got2, ref)


def _as_full_sequence(w, b):
    """The same sequence b as a P=0 prefill over its whole logical sequence."""
    P = int(w.prefix_lens[b])
    c0, c1 = int(w.cu_q_lens[b]), int(w.cu_q_lens[b + 1])
    d, Hkv = w.head_dim, w.num_kv_heads
    kpre = np.array([w.k_pool[w.block_tables[b][j // 16], :, j % 16] for j in range(P)],
                    np.uint16).reshape(P, Hkv, d)
    vpre = np.array([w.v_pool[w.block_tables[b][j // 16], :, j % 16] for j in range(P)],
                    np.uint16).reshape(P, Hkv, d)
    rng = np.random.default_rng(99)
    qpre = round_to_bits(rng.standard_normal((P, w.num_q_heads, d), dtype=np.float32), w.dtype)
    q = np.concatenate([qpre, w.q[c0:c1]])
    kn = np.concatenate([kpre, w.k_new[c0:c1]])
    vn = np.concatenate([vpre, w.v_new[c0:c1]])
    L = P + c1 - c0
    return q, kn, vn, np.array([0, L], np.int32), np.array([0], np.int32)


def test_reuse_invariant_prefix_equals_full_causal():
    w = make_custom(35, "bf16", 4, 1, 32, [40, 3], [11, 6])
    out = _prefill(w)
    for b in range(2):
        q, kn, vn, cu, pl = _as_full_sequence(w, b)
        full = oracle.paged_prefill(w.k_pool[:1], w.v_pool[:1], q, kn, vn, cu, pl,
                                    np.zeros((1, 1), np.int32), 4, w.scale, "bf16")
        P = int(w.prefix_lens[b])
        np.testing.assert_allclose(out[w.cu_q_lens[b]:w.cu_q_lens[b + 1]], full[P:], rtol=0, atol=1e-14)


def test_chunk_split_into_two_prefills():
    # processing a chunk as two successive chunks (the first one cached) gives the same rows
    w = make_custom(36, "fp16", 2, 2, 16, [21], [13])
    out = _prefill(w)
    cut = 6
    # second half: prefix = 21 + 6, the first 6 chunk tokens written into the pool
    k2, v2 = oracle.write_kv(w.k_pool, w.v_pool, w.k_new[:cut], w.v_new[:cut], w.slot_mapping[:cut])
    got = oracle.paged_prefill(k2, v2, w.q[cut:], w.k_new[cut:], w.v_new[cut:],
                               np.array([0, 13 - cut]), np.array([21 + cut]), w.block_tables,
                               2, w.scale, "fp16")
    np.testing.assert_allclose(got, out[cut:], rtol=0, atol=1e-14)


def test_decode_is_one_row_prefill():
    w = make_custom(37, "bf16", 4, 2, 64, [30, 16, 1], kind="decode")
    dec = oracle.paged_decode(w.k_pool, w.v_pool, w.q, w.context_lens, w.block_tables, w.scale, "bf16")
    for b in range(3):
        n = int(w.context_lens[b])
        last = n - 1
        blk, row = w.block_tables[b][last // 16], last % 16
        kn = w.k_pool[blk, :, row][None]
        vn = w.v_pool[blk, :, row][None]
        got = oracle.paged_prefill(w.k_pool, w.v_pool, w.q[b:b + 1], kn, vn, [0, 1], [last],
                                   w.block_tables[b:b + 1], 4, w.scale, "bf16")
        np.testing.assert_allclose(got[0], dec[b], rtol=0, atol=1e-14)


def test_gqa_equals_mha_with_repeated_kv():
    w = make_custom(38, "fp16", 6, 2, 32, [19, 32], [5, 2])
    out = _prefill(w)
    G = 3
    kp = np.repeat(w.k_pool, G, axis=1)
    vp = np.repeat(w.v_pool, G, axis=1)
    kn = np.repeat(w.k_new, G, axis=1)
    vn = np.repeat(w.v_new, G, axis=1)
    mha = oracle.paged_prefill(kp, vp, w.q, kn, vn, w.cu_q_lens, w.prefix_lens, w.block_tables,
                               6, w.scale, "fp16")
    assert np.array_equal(out, mha)


def test_causality_future_keys_do_not_matter():
    w = make_custom(39, "bf16", 2, 1, 16, [10], [8])
    out = _prefill(w)
    k2, v2 = w.k_new.copy(), w.v_new.copy()
    k2[5:] = round_to_bits(np.full(k2[5:].shape, 7.0, np.float32), "bf16")
    v2[5:] = round_to_bits(np.full(v2[5:].shape, -3.0, np.float32), "bf16")
    got = oracle.paged_prefill(w.k_pool, w.v_pool, w.q, k2, v2, w.cu_q_lens, w.prefix_lens,
                               w.block_tables, 2, w.scale, "bf16")
    assert np.array_equal(got[:5], out[:5])
    assert not np.allclose(got[5:], out[5:])


def test_poisoned_slots_are_never_read():
    # make_custom poisons unused blocks and prefix tail slots with NaN
    w = make_custom(40, "fp16", 2, 1, 16, [19, 0], [4, 3])
    assert np.isnan(_f64(w.k_pool, "fp16")).any()
    out = _prefill(w)
    assert np.isfinite(out).all()


def test_lse_merge_of_key_partitions():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((3, 8))
    K = rng.standard_normal((37, 8))
    V = rng.standard_normal((37, 8))
    pos = [36, 36, 20]
    full, lse = oracle.attend(q, K, V, pos, 0.3)
    cuts = [0, 5, 16, 17, 30, 37]
    parts = [oracle.attend(q, K, V, pos, 0.3, keys=np.arange(a, b)) for a, b in zip(cuts, cuts[1:])]
    m, l = oracle.lse_merge(parts)
    np.testing.assert_allclose(m, full, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l, lse, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- scatter

def test_write_kv_matches_slot_semantics():
    w = make_custom(41, "bf16", 2, 2, 8, [3, 20], [14, 2])
    slots = w.slot_mapping.copy()
    slots[4] = -1
    kp, vp = oracle.write_kv(w.k_pool, w.v_pool, w.k_new, w.v_new, slots)
    changed = np.argwhere((kp != w.k_pool).any(axis=(1, 3)))
    for t, s in enumerate(slots):
        if s < 0:
            continue
        assert np.array_equal(kp[s // 16, :, s % 16], w.k_new[t])
        assert np.array_equal(vp[s // 16, :, s % 16], w.v_new[t])
    touched = {(int(s) // 16, int(s) % 16) for s in slots if s >= 0}
    assert {(int(a), int(b)) for a, b in changed} <= touched
    assert (int(slots[4 + 1]) // 16, 0) != (-1, 0)
    # the skipped token's would-be slot is untouched
    s4 = int(w.slot_mapping[4])
    assert np.array_equal(kp[s4 // 16, :, s4 % 16], w.k_pool[s4 // 16, :, s4 % 16])


def test_write_kv_skips_slots_outside_the_pool():
    """A slot at or past num_blocks * 16 names no row of the fixed pool: the token is
    skipped and the pool is bit-for-bit unchanged; the other tokens land as usual."""
    w = make_custom(43, "fp16", 2, 1, 8, [5], [6])
    nb = w.k_pool.shape[0]
    slots = w.slot_mapping.copy()
    slots[1] = nb * 16                  # first slot past the pool
    slots[2] = nb * 16 + 17
    slots[3] = 1 << 40
    kp, vp = oracle.write_kv(w.k_pool, w.v_pool, w.k_new, w.v_new, slots)
    keep = [0, 4, 5]
    ek, ev = oracle.write_kv(w.k_pool, w.v_pool, w.k_new[keep], w.v_new[keep], slots[keep])
    assert np.array_equal(kp, ek) and np.array_equal(vp, ev)
    for t in keep:
        s = int(slots[t])
        assert np.array_equal(kp[s // 16, :, s % 16], w.k_new[t])
    # only the three in-pool slots' rows changed
    diff = (kp != w.k_pool).any(axis=(1, 3)) | (vp != w.v_pool).any(axis=(1, 3))
    assert {(int(a), int(b)) for a, b in np.argwhere(diff)} <= {(int(slots[t]) // 16, int(slots[t]) % 16) for t in keep}


def test_selected_rows_equal_full_result():
    w = make_custom(42, "bf16", 8, 2, 32, [40, 0, 17], [9, 12, 3])
    full = _prefill(w)
    sel = [(0, 3, [0, 4, 8]), (1, 7, list(range(12))), (2, 0, [2])]
    got = _prefill(w, select=sel)
    for b, h, rows in sel:
        np.testing.assert_allclose(got[(b, h)], full[w.cu_q_lens[b] + np.array(rows), h], rtol=0, atol=1e-14)
    dec = make_custom(43, "fp16", 4, 2, 16, [33, 5, 70], kind="decode")
    a = oracle.paged_decode(dec.k_pool, dec.v_pool, dec.q, dec.context_lens, dec.block_tables, dec.scale, "fp16")
    b_ = oracle.paged_decode(dec.k_pool, dec.v_pool, dec.q, dec.context_lens, dec.block_tables, dec.scale, "fp16",
                             seqs=[2])
    np.testing.assert_allclose(a[2], b_[2], rtol=0, atol=1e-14)


def test_copy_blocks_preserves_sequences_through_remapped_tables():
    """A sequence whose blocks are copied elsewhere and whose table is remapped to the
    copies gathers to exactly the same tokens; other destination blocks are untouched,
    and pairs with an id outside its pool are skipped."""
    w = make_custom(31, "bf16", 4, 2, 64, [70, 33], poison=True, kind="decode")
    nb = w.num_blocks
    rng = np.random.default_rng(3)
    host_k = rng.integers(0, 1 << 16, size=(nb + 5,) + w.k_pool.shape[1:]).astype(np.uint16)
    host_v = rng.integers(0, 1 << 16, size=(nb + 5,) + w.v_pool.shape[1:]).astype(np.uint16)
    src = list(w.block_tables[0][:5])
    dst = [nb + 4, 0 + 7, 3, 11, 2]
    ids_s = src + [nb + 100, 1]
    ids_d = dst + [5, -1]                             # invalid pairs: skipped
    hk, hv = oracle.copy_blocks(w.k_pool, w.v_pool, host_k, host_v, ids_s, ids_d)
    for a, b in ((hk, host_k), (hv, host_v)):
        keep = np.ones(nb + 5, bool)
        keep[dst] = False
        assert np.array_equal(a[keep], b[keep])
    table = np.asarray(dst, np.int32)
    n = int(w.context_lens[0])
    assert np.array_equal(oracle.gather_kv(hk, table, n), oracle.gather_kv(w.k_pool, w.block_tables[0], n))
    assert np.array_equal(oracle.gather_kv(hv, table, n), oracle.gather_kv(w.v_pool, w.block_tables[0], n))
    # round trip back into a fresh pool: identity on the copied blocks
    bk, bv = oracle.copy_blocks(hk, hv, np.zeros_like(w.k_pool), np.zeros_like(w.v_pool), dst, src)
    assert np.array_equal(bk[src], w.k_pool[src]) and np.array_equal(bv[src], w.v_pool[src])
