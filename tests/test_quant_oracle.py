"""Pins of the 8-bit pool oracle (oracle/quant.py) against what the pages and plain
arithmetic fix, on the CPU.  The pages (kvboost 0.6.0, "Optional: KV quantization")
fix only the axes of the scales: per channel for K, per token for V."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import quant
from workloads.gen import round_to_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quant_codes.json")


def bits(x, dtype):
    return round_to_bits(np.asarray(x, dtype=np.float64), dtype)


def test_codes_of_hand_examples():
    """Hand-derived codes (tests/golden/quant_codes.json): a token whose absolute maximum
    is 127 has scale exactly 1, so its codes are its values rounded half to even; K
    values at given per-channel scales round the same way, clamp at +-127, and a zero
    scale gives code 0."""
    g = json.load(open(GOLDEN))
    for case in g["v_tokens"]:
        x = np.asarray(case["values"], dtype=np.float32)
        s = quant.token_scale(x)
        assert s == np.float32(case["scale"])
        assert quant.quantize(x, s).tolist() == case["codes"]
    for case in g["k_channels"]:
        got = quant.quantize(np.asarray(case["values"], np.float32), np.asarray(case["scales"], np.float32))
        assert got.tolist() == case["codes"]


def test_error_within_half_a_step():
    """|x - s*code| <= s/2 for every value a per-token scale covers (never clamped)."""
    rng = np.random.default_rng(0)
    v = (rng.standard_normal((200, 4, 128)) * rng.uniform(0.01, 50, (200, 4, 1))).astype(np.float32)
    s = quant.token_scale(v)
    c = quant.quantize(v, s[..., None])
    assert np.abs(c).max() <= 127
    assert (np.abs(c).max(axis=-1) == 127).all()        # the largest value maps to +-127
    err = np.abs(v.astype(np.float64) - quant.dequant_v(c, s))
    assert (err <= s.astype(np.float64)[..., None] * (0.5 + 1e-6)).all()


def test_token_scale_equivariance():
    """Scaling a token by a power of two scales its V scale and keeps its codes."""
    rng = np.random.default_rng(1)
    v = rng.standard_normal((16, 2, 64)).astype(np.float32)
    s1 = quant.token_scale(v)
    s2 = quant.token_scale(v * np.float32(8))
    assert np.array_equal(s2, s1 * np.float32(8))
    assert np.array_equal(quant.quantize(v, s1[..., None]), quant.quantize(v * np.float32(8), s2[..., None]))


def test_channel_scale_only_moves_its_channel():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 3, 32)).astype(np.float32)
    s = np.full((3, 32), 0.02, np.float32)
    c1 = quant.quantize(x, s)
    s2 = s.copy()
    s2[1, 7] = 0.05
    c2 = quant.quantize(x, s2)
    diff = np.argwhere(c1 != c2)
    assert len(diff) > 0 and (diff[:, 1] == 1).all() and (diff[:, 2] == 7).all()


def _exact_pool(rng, dtype, nb, hkv, d, n_tok):
    """Tokens whose K is k_scale * integer codes and whose V is 2^e * integer codes with
    a code of +-127 in every (token, head): every value is exact in 16 bits, so writing
    them reproduces those codes and scales exactly."""
    k_scale = (2.0 ** rng.integers(-6, -2, size=(hkv, d))).astype(np.float32)
    kc = rng.integers(-127, 128, size=(n_tok, hkv, d))
    vc = rng.integers(-127, 128, size=(n_tok, hkv, d))
    vc[np.arange(n_tok)[:, None], np.arange(hkv)[None, :], rng.integers(0, d, size=(n_tok, hkv))] = 127
    ve = 2.0 ** rng.integers(-8, -3, size=(n_tok, hkv))
    K = kc * k_scale.astype(np.float64)
    V = vc * ve[..., None]
    return k_scale, kc, vc, ve, bits(K, dtype), bits(V, dtype)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_write_reproduces_exact_codes_and_skips_negative_slots(dtype):
    rng = np.random.default_rng(3)
    nb, hkv, d, n = 6, 2, 64, 40
    k_scale, kc, vc, ve, kb, vb = _exact_pool(rng, dtype, nb, hkv, d, n)
    slots = rng.permutation(nb * 16)[:n].astype(np.int64)
    slots[5] = -1
    K0 = np.full((nb, hkv, 16, d), 99, np.int8)
    V0 = np.full((nb, hkv, 16, d), -99, np.int8)
    S0 = np.full((nb, hkv, 16), 7.0, np.float32)
    K1, V1, S1 = quant.write_kv_q8(K0, V0, S0, k_scale, kb, vb, slots, dtype)
    written = np.zeros((nb, 16), bool)
    for t, s in enumerate(slots):
        if s < 0:
            continue
        blk, row = s // 16, s % 16
        written[blk, row] = True
        assert np.array_equal(K1[blk, :, row], kc[t])
        assert np.array_equal(V1[blk, :, row], vc[t])
        assert np.array_equal(S1[blk, :, row], ve[t].astype(np.float32))
    # [block][row] first, so the mask of written slots selects every head of a slot
    assert (K1.transpose(0, 2, 1, 3)[~written] == 99).all()
    assert (V1.transpose(0, 2, 1, 3)[~written] == -99).all()
    assert (S1.transpose(0, 2, 1)[~written] == 7.0).all()


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_decode_over_exact_pool_equals_plain_decode(dtype):
    """When every K/V value is exactly what its code stands for, decode over the 8-bit
    pool is decode over the 16-bit values: the same float64 result, bit for bit."""
    rng = np.random.default_rng(4)
    nb, hkv, hq, d = 40, 2, 8, 64
    ctx = np.array([1, 17, 100, 333, 0], np.int32)
    n_tok = int(ctx.sum())
    k_scale, kc, vc, ve, kb, vb = _exact_pool(rng, dtype, nb, hkv, d, n_tok)
    perm = rng.permutation(nb)
    stride = 22
    bt = np.full((len(ctx), stride), -1, np.int32)
    slots, used = [], 0
    for b, n in enumerate(ctx):
        nblk = (n + 15) // 16
        bt[b, :nblk] = perm[used:used + nblk]
        used += nblk
        slots += [int(bt[b, j // 16]) * 16 + j % 16 for j in range(n)]
    slots = np.array(slots, np.int64)
    K16 = np.zeros((nb, hkv, 16, d), np.uint16)
    V16 = np.zeros((nb, hkv, 16, d), np.uint16)
    K16, V16 = oracle.write_kv(K16, V16, kb, vb, slots)
    Kc, Vc, Vs = quant.write_kv_q8(np.zeros((nb, hkv, 16, d), np.int8), np.zeros((nb, hkv, 16, d), np.int8),
                                   np.zeros((nb, hkv, 16), np.float32), k_scale, kb, vb, slots, dtype)
    q = bits(rng.standard_normal((len(ctx), hq, d)), dtype)
    ref = oracle.paged_decode(K16, V16, q, ctx, bt, 0.125, dtype)
    got = quant.paged_decode_q8(Kc, Vc, Vs, k_scale, q, ctx, bt, 0.125, dtype)
    assert np.array_equal(got, ref)
    assert (got[ctx == 0] == 0).all()


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_prefill_over_exact_pool_equals_plain_prefill(dtype):
    """Prefill whose cached prefix sits in the 8-bit pool with values exactly code x scale
    equals the 16-bit prefill of the same values, bit for bit."""
    rng = np.random.default_rng(5)
    nb, hkv, hq, d = 30, 2, 6, 64
    P = np.array([0, 40, 129, 16], np.int64)
    C = np.array([5, 17, 3, 30], np.int64)
    n_tok = int(P.sum())
    k_scale, kc, vc, ve, kb, vb = _exact_pool(rng, dtype, nb, hkv, d, n_tok)
    perm = rng.permutation(nb)
    stride = 10
    bt = np.full((len(P), stride), -1, np.int32)
    slots, used = [], 0
    for b, n in enumerate(P):
        nblk = (n + 15) // 16
        bt[b, :nblk] = perm[used:used + nblk]
        used += nblk
        slots += [int(bt[b, j // 16]) * 16 + j % 16 for j in range(n)]
    slots = np.array(slots, np.int64)
    K16, V16 = oracle.write_kv(np.zeros((nb, hkv, 16, d), np.uint16), np.zeros((nb, hkv, 16, d), np.uint16),
                               kb, vb, slots)
    Kc, Vc, Vs = quant.write_kv_q8(np.zeros((nb, hkv, 16, d), np.int8), np.zeros((nb, hkv, 16, d), np.int8),
                                   np.zeros((nb, hkv, 16), np.float32), k_scale, kb, vb, slots, dtype)
    T = int(C.sum())
    cu = np.concatenate([[0], np.cumsum(C)])
    q = bits(rng.standard_normal((T, hq, d)), dtype)
    kn = bits(rng.standard_normal((T, hkv, d)), dtype)
    vn = bits(rng.standard_normal((T, hkv, d)), dtype)
    ref = oracle.paged_prefill(K16, V16, q, kn, vn, cu, P, bt, hq, 0.125, dtype)
    got = quant.paged_prefill_q8(Kc, Vc, Vs, k_scale, q, kn, vn, cu, P, bt, hq, 0.125, dtype)
    assert np.array_equal(got, ref)


def test_4bit_codes_and_nibbles():
    """4-bit codes of hand examples (tests/golden/quant_codes.json) and their packing two
    per byte, even channel in the low nibble."""
    g = json.load(open(GOLDEN))
    for case in g["v_tokens_4bit"]:
        x = np.asarray(case["values"], dtype=np.float32)
        s = quant.token_scale(x, quant.CODE_MAX4)
        assert s == np.float32(case["scale"])
        assert quant.quantize(x, s, quant.CODE_MAX4).tolist() == case["codes"]
    nb = g["nibbles"]
    packed = quant.pack_nibbles(np.asarray(nb["codes"], np.int8))
    assert packed.tolist() == nb["bytes"]
    assert quant.unpack_nibbles(packed).tolist() == nb["codes"]
    rng = np.random.default_rng(9)
    c = rng.integers(-7, 8, size=(5, 3, 64)).astype(np.int8)
    assert np.array_equal(quant.unpack_nibbles(quant.pack_nibbles(c)), c)


def test_4bit_error_bound_and_exact_reduction():
    """4-bit: |x - s*code| <= s/2, and decode over a 4-bit pool whose values are exactly
    code x scale equals the 16-bit decode bit for bit."""
    rng = np.random.default_rng(10)
    v = rng.standard_normal((100, 2, 64)).astype(np.float32)
    s = quant.token_scale(v, quant.CODE_MAX4)
    c = quant.quantize(v, s[..., None], quant.CODE_MAX4)
    assert np.abs(c).max() == 7
    assert (np.abs(v.astype(np.float64) - quant.dequant_v(c, s)) <= s.astype(np.float64)[..., None] * (0.5 + 1e-6)).all()
    nb, hkv, hq, d, dtype = 20, 2, 4, 64, "bf16"
    ctx = np.array([33, 100, 1], np.int32)
    n_tok = int(ctx.sum())
    k_scale = (2.0 ** rng.integers(-4, 0, size=(hkv, d))).astype(np.float32)
    kc = rng.integers(-7, 8, size=(n_tok, hkv, d))
    vc = rng.integers(-7, 8, size=(n_tok, hkv, d))
    vc[np.arange(n_tok)[:, None], np.arange(hkv)[None, :], rng.integers(0, d, size=(n_tok, hkv))] = 7
    ve = 2.0 ** rng.integers(-6, -2, size=(n_tok, hkv))
    kb, vb = bits(kc * k_scale.astype(np.float64), dtype), bits(vc * ve[..., None], dtype)
    perm = rng.permutation(nb)
    bt = np.full((3, 8), -1, np.int32)
    slots, used = [], 0
    for b, n in enumerate(ctx):
        nblk = (n + 15) // 16
        bt[b, :nblk] = perm[used:used + nblk]
        used += nblk
        slots += [int(bt[b, j // 16]) * 16 + j % 16 for j in range(n)]
    slots = np.array(slots, np.int64)
    K16, V16 = oracle.write_kv(np.zeros((nb, hkv, 16, d), np.uint16), np.zeros((nb, hkv, 16, d), np.uint16),
                               kb, vb, slots)
    Kc, Vc, Vs = quant.write_kv_q8(np.zeros((nb, hkv, 16, d), np.int8), np.zeros((nb, hkv, 16, d), np.int8),
                                   np.zeros((nb, hkv, 16), np.float32), k_scale, kb, vb, slots, dtype,
                                   quant.CODE_MAX4)
    q = bits(rng.standard_normal((3, hq, d)), dtype)
    ref = oracle.paged_decode(K16, V16, q, ctx, bt, 0.125, dtype)
    got = quant.paged_decode_q8(Kc, Vc, Vs, k_scale, q, ctx, bt, 0.125, dtype)
    assert np.array_equal(got, ref)


def test_prefill_q8_select_matches_full():
    """The oracle's row selection computes the same values as its full prefill (up to the
    summation order of the matrix products, which depends on the number of rows)."""
    from workloads import make_custom, channel_scales
    w = make_custom(851, "bf16", 8, 2, 64, [40, 0, 90], [17, 5, 33], share="pairs", poison=False)
    slots = []
    for b in range(w.batch):
        j = np.arange(int(w.prefix_lens[b]))
        slots.append(w.block_tables[b][j // 16].astype(np.int64) * 16 + j % 16)
    slots = np.unique(np.concatenate(slots))
    kt = np.ascontiguousarray(w.k_pool[slots // 16, :, slots % 16, :])
    vt = np.ascontiguousarray(w.v_pool[slots // 16, :, slots % 16, :])
    ks = channel_scales(oracle.decode_bits(kt, "bf16").astype(np.float32))
    nb = w.k_pool.shape[0]
    kc, vc, vs = quant.write_kv_q8(np.zeros((nb, 2, 16, 64), np.int8), np.zeros((nb, 2, 16, 64), np.int8),
                                   np.zeros((nb, 2, 16), np.float32), ks, kt, vt, slots, "bf16")
    args = (kc, vc, vs, ks, w.q, w.k_new, w.v_new, w.cu_q_lens, w.prefix_lens, w.block_tables, 8, w.scale, "bf16")
    full = quant.paged_prefill_q8(*args)
    sel = [(0, 3, [0, 16]), (2, 7, [1, 32]), (1, 0, [4])]
    part = quant.paged_prefill_q8(*args, select=sel)
    for (b, h, rows) in sel:
        assert np.allclose(part[(b, h)], full[w.cu_q_lens[b] + np.asarray(rows), h], rtol=0, atol=1e-12)
