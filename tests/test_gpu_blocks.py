"""Block copies on the GPU (kvb_copy_blocks): copy-on-write forks inside the device pool
and swap between the device pool and a pool in pinned host memory, driven by the same
random block-manager script as the oracle; final pools compared bit for bit."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


class _GpuBackend:
    def __init__(self, nb, ncpu, hkv, d):
        import attention_paged_prefix_amd as kvb
        self.kvb = kvb
        # device pool interleaved (K and V of a block side by side), host pool split:
        # copies go between different block strides
        self.kv = torch.zeros((nb, 2, hkv, 16, d), dtype=torch.float16, device="cuda:0")
        self.gpu = kvb.Pool.interleaved(self.kv)
        self.hk = torch.zeros((ncpu, hkv, 16, d), dtype=torch.float16).pin_memory()
        self.hv = torch.zeros((ncpu, hkv, 16, d), dtype=torch.float16).pin_memory()
        self.cpu = kvb.Pool.from_tensors(self.hk, self.hv)

    def write(self, slots, kr, vr):
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda:0").view(torch.float16)
        self.kvb.write_kv(self.gpu, dev(kr), dev(vr),
                          torch.as_tensor(np.asarray(slots, np.int64)).to("cuda:0"))

    def copy(self, src, dst, s_ids, d_ids):
        ids = lambda a: torch.as_tensor(np.asarray(a, np.int32)).to("cuda:0")
        pools = {"gpu": self.gpu, "cpu": self.cpu}
        self.kvb.copy_blocks(pools[src], pools[dst], ids(s_ids), ids(d_ids))
        torch.cuda.synchronize()        # the host pool is read on the host afterwards


def test_block_script_matches_oracle_bit_for_bit():
    import blockscript
    from test_block_manager import _OracleBackend
    nb, ncpu, hkv, d = 48, 24, 2, 64
    ref = _OracleBackend(nb, ncpu, (hkv, 16, d))
    blockscript.run(ref, nb, ncpu, 300, 21, (hkv, d))
    gpu = _GpuBackend(nb, ncpu, hkv, d)
    blockscript.run(gpu, nb, ncpu, 300, 21, (hkv, d))
    torch.cuda.synchronize()
    bits = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(bits(gpu.kv[:, 0]), ref.pools["gpu"][0])
    assert np.array_equal(bits(gpu.kv[:, 1]), ref.pools["gpu"][1])
    assert np.array_equal(bits(gpu.hk), ref.pools["cpu"][0])
    assert np.array_equal(bits(gpu.hv), ref.pools["cpu"][1])


def test_copy_blocks_skips_out_of_pool_pairs():
    import attention_paged_prefix_amd as kvb
    k = torch.arange(4 * 2 * 16 * 64, dtype=torch.int16, device="cuda:0").view(4, 2, 16, 64).view(torch.float16)
    v = (k.view(torch.int16) + 7).view(torch.float16)
    pool = kvb.Pool.from_tensors(k, v)
    before_k, before_v = k.clone(), v.clone()
    ids = lambda a: torch.tensor(a, dtype=torch.int32, device="cuda:0")
    kvb.copy_blocks(pool, pool, ids([0, 9, -1, 2]), ids([3, 1, 1, 4]))
    torch.cuda.synchronize()
    assert torch.equal(k[3].view(torch.int16), before_k[0].view(torch.int16))
    assert torch.equal(v[3].view(torch.int16), before_v[0].view(torch.int16))
    for b in (0, 1, 2):                       # invalid pairs left everything else alone
        assert torch.equal(k[b].view(torch.int16), before_k[b].view(torch.int16))
        assert torch.equal(v[b].view(torch.int16), before_v[b].view(torch.int16))
