"""kvb_paged_decode_noalloc (split partials in the library's static device scratch, no
allocation) against kvb_paged_decode with a caller workspace: the same kernels and split
plan, so the same bits; and both within tolerance of the fp64 oracle.  Two calls in a
row, the second with a smaller input, so the second reuses scratch the first filled."""
import numpy as np
import pytest

from workloads import make_custom

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _util():
    import gpu_util
    return gpu_util


def _check(w, split_blocks):
    import attention_paged_prefix_amd as kvb
    u = _util()
    dev = u.Dev(w)
    max_ctx = int(w.context_lens.max())
    ref = u.to_bits(dev.decode(split_blocks=split_blocks))
    out = torch.full_like(dev.q, float("nan"))
    kvb.paged_decode_noalloc(dev.pool, dev.q, dev.ctx, dev.bt, w.scale, max_ctx, out=out,
                             split_blocks=split_blocks)
    torch.cuda.synchronize()
    got = u.to_bits(out)
    assert np.array_equal(got, ref)
    err = u.max_err(got, u.oracle_decode(w), w.dtype)
    assert err <= u.TOL[w.dtype], f"max abs err {err}"


@pytest.mark.parametrize("split_blocks", [0, 4])
def test_noalloc_decode_equals_workspace_decode_twice(split_blocks):
    # first call: 12 sequences, long contexts (many splits); second: 3 short sequences
    big = make_custom(301, "bf16", 32, 8, 128, [3000, 17, 1200, 4096, 900, 2500, 64, 1, 777,
                                                 3333, 1600, 2048], kind="decode", poison=True)
    small = make_custom(302, "bf16", 32, 8, 128, [700, 5, 260], kind="decode", poison=True)
    _check(big, split_blocks)
    _check(small, split_blocks)


def test_noalloc_decode_fp16_d96_then_smaller():
    _check(make_custom(303, "fp16", 16, 4, 96, [2000, 1500, 3900, 40], kind="decode",
                       poison=True), 0)
    _check(make_custom(304, "fp16", 16, 4, 96, [100, 33], kind="decode", poison=True), 2)
