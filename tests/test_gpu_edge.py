"""Edge cases of the HIP path against the oracle: empty chunks inside a batch, a 64K-token
prefix (long descriptor refills), scores large enough that the running max moves on
almost every tile, a zero scale (uniform attention), and decode contexts that end exactly
at the end of their block tables."""
import numpy as np
import pytest

from workloads import make_custom, round_to_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _util():
    import gpu_util
    return gpu_util


def test_prefill_empty_chunks_inside_a_batch():
    u = _util()
    w = make_custom(701, "fp16", 16, 4, 128, [100, 50, 0, 300, 7], [0, 70, 0, 33, 0], poison=True)
    assert w.total_q == 103
    dev = u.Dev(w)
    got = u.to_bits(dev.prefill())
    err = u.max_err(got, u.oracle_prefill(w), "fp16")
    assert err <= u.TOL["fp16"], f"max abs err {err}"


@pytest.mark.parametrize("pooled", [False, True])
def test_prefill_64k_token_prefix_sampled(pooled):
    import attention_paged_prefix_amd as kvb
    import oracle
    u = _util()
    w = make_custom(702, "bf16", 8, 1, 128, [65536], [64], poison=True)
    dev = u.Dev(w)
    if pooled:
        kvb.write_kv(dev.pool, dev.k_new, dev.v_new, dev.slots)
        out = kvb.paged_prefill_pooled(dev.pool, dev.q, dev.cu, dev.pl, dev.bt, w.scale, 64, 65536)
    else:
        out = dev.prefill()
    vals = oracle.decode_bits(u.to_bits(out), "bf16")
    assert np.isfinite(vals).all()
    sel = [(0, h, [0, 1, 31, 32, 62, 63]) for h in (0, 3, 7)]
    ref = oracle.paged_prefill(w.k_pool, w.v_pool, w.q, w.k_new, w.v_new, w.cu_q_lens, w.prefix_lens,
                               w.block_tables, w.num_q_heads, w.scale, w.dtype, select=sel)
    for (b, h, rows) in sel:
        assert np.max(np.abs(vals[rows, h] - ref[(b, h)])) <= u.TOL["bf16"]


@pytest.mark.parametrize("gain", [12.0, 40.0])
def test_prefill_large_scores(gain):
    """Queries scaled up: scores span tens of units, the running max is raised on most
    tiles (the lazy rescale path) and the softmax is sharply peaked."""
    import oracle
    u = _util()
    w = make_custom(703, "bf16", 16, 2, 128, [1000, 333], [200, 77], share="pairs", poison=True)
    w.q = round_to_bits(oracle.decode_bits(w.q, "bf16") * gain, "bf16")
    dev = u.Dev(w)
    got = u.to_bits(dev.prefill())
    assert np.isfinite(oracle.decode_bits(got, "bf16")).all()
    err = u.max_err(got, u.oracle_prefill(w), "bf16")
    assert err <= u.TOL["bf16"], f"max abs err {err}"


def test_prefill_increasing_scores_rescale_every_tile():
    """Keys aligned with the query and growing along the sequence: every new tile holds
    the largest scores so far."""
    import oracle
    u = _util()
    w = make_custom(704, "fp16", 4, 4, 64, [700], [40], poison=True)
    q = oracle.decode_bits(w.q, "fp16")
    k = oracle.decode_bits(w.k_pool, "fp16")
    table = w.block_tables[0]
    for j in range(700):
        blk, row = int(table[j // 16]), j % 16
        # scores grow to ~100 in exp2 units: the running max moves by > 8 on most tiles
        k[blk, :, row, :] = q[0, :, :] * (9.0 * j / 700.0) + 0.1 * k[blk, :, row, :]
    w.k_pool = np.where(np.isnan(oracle.decode_bits(w.k_pool, "fp16")), w.k_pool, round_to_bits(k, "fp16"))
    dev = u.Dev(w)
    got = u.to_bits(dev.prefill())
    err = u.max_err(got, u.oracle_prefill(w), "fp16")
    assert err <= u.TOL["fp16"], f"max abs err {err}"


def test_scale_zero_is_uniform_attention():
    import oracle
    u = _util()
    w = make_custom(705, "bf16", 8, 2, 64, [50, 0], [30, 17], poison=True)
    w.scale = 0.0
    dev = u.Dev(w)
    got = u.to_bits(dev.prefill())
    err = u.max_err(got, u.oracle_prefill(w), "bf16")
    assert err <= u.TOL["bf16"], f"max abs err {err}"
    wd = make_custom(706, "fp16", 8, 2, 128, [300, 17], kind="decode", poison=True)
    wd.scale = 0.0
    dd = u.Dev(wd)
    gd = u.to_bits(dd.decode(split_blocks=4))
    assert u.max_err(gd, u.oracle_decode(wd), "fp16") <= u.TOL["fp16"]


def test_decode_contexts_ending_at_the_table_end():
    import attention_paged_prefix_amd as kvb
    u = _util()
    w = make_custom(707, "bf16", 32, 8, 128, [1024, 512, 1023, 1009], kind="decode", poison=True)
    assert w.block_tables.shape[1] * 16 == 1024
    dev = u.Dev(w)
    ref = u.oracle_decode(w)
    for split in (0, 1, 64):
        got = u.to_bits(dev.decode(split_blocks=split))
        assert u.max_err(got, ref, "bf16") <= u.TOL["bf16"]
    # a max_context_len larger than every context changes nothing
    big = u.to_bits(kvb.paged_decode(dev.pool, dev.q, dev.ctx, dev.bt, w.scale, 1024))
    assert u.max_err(big, ref, "bf16") <= u.TOL["bf16"]
