"""The hot path captured in a HIP graph (as a serving loop would run it): replays give the
same bits as eager calls.  Replayed several times with the program's own eager work and
synchronisations in between, every replay checked."""
import numpy as np
import pytest

from workloads import make_custom

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("fused", [False, True])
def test_step_graph_replays_match_eager(fused):
    """fused: the chunk's prefill and slot scatter in one launch (kvb_paged_prefill_write),
    as the benchmark step runs it; replays must give the bits of the four-call step."""
    import attention_paged_prefix_amd as kvb
    import gpu_util as u
    w = make_custom(601, "bf16", 16, 2, 128, [300, 64, 1000], [40, 130, 77], share="pairs",
                    poison=True, with_decode=True)
    dev = u.Dev(w)
    dq = u.to_dev(w.dec_q, "bf16")
    dk = u.to_dev(w.dec_k, "bf16")
    dv = u.to_dev(w.dec_v, "bf16")
    dslots = u.idev(w.dec_slots, torch.int64)
    dctx = u.idev(w.dec_context_lens)
    max_ctx = int(w.dec_context_lens.max())
    out = torch.empty_like(dev.q)
    dout = torch.empty_like(dq)
    n = kvb.paged_decode_workspace_size(w.batch, w.num_kv_heads, w.num_q_heads, w.head_dim, max_ctx, 2)
    ws = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda:0")
    k0, v0 = dev.k.clone(), dev.v.clone()

    def step_serial():
        kvb.write_kv(dev.pool, dev.k_new, dev.v_new, dev.slots)
        dev.prefill(out=out)
        kvb.write_kv(dev.pool, dk, dv, dslots)
        kvb.paged_decode(dev.pool, dq, dctx, dev.bt, w.scale, max_ctx, split_blocks=2, out=dout,
                         workspace=ws)

    def step_fused():
        kvb.paged_prefill(dev.pool, dev.q, dev.k_new, dev.v_new, dev.cu, dev.pl, dev.bt, w.scale,
                          int(w.q_lens.max()), int(w.prefix_lens.max()), out=out,
                          slot_mapping=dev.slots)
        kvb.write_kv(dev.pool, dk, dv, dslots)
        kvb.paged_decode(dev.pool, dq, dctx, dev.bt, w.scale, max_ctx, split_blocks=2, out=dout,
                         workspace=ws)

    step = step_fused if fused else step_serial

    def reset():
        dev.k.copy_(k0)
        dev.v.copy_(v0)
        out.zero_()
        dout.zero_()

    step_serial()                                   # the reference: four separate calls
    torch.cuda.synchronize()
    ref = (u.to_bits(out), u.to_bits(dout), u.to_bits(dev.k), u.to_bits(dev.v))

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                      # warm the capture stream
        reset()
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    reset()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        reset()                                     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (u.to_bits(out), u.to_bits(dout), u.to_bits(dev.k), u.to_bits(dev.v))
        for a, b in zip(got, ref):
            assert np.array_equal(a, b), f"replay {rep} differs"
        _ = (out.float() * 2).sum().item()          # unrelated eager kernels
