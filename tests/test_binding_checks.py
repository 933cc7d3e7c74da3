"""The Python binding checks the index tensors it hands to the kernels as raw pointers
(dtype, contiguity, device, length) before any library call, so these run without a GPU:
every call here must raise ValueError on the host."""
import pytest
import torch

import attention_paged_prefix_amd as kvb

B, HQ, HKV, D, NB = 3, 4, 2, 64, 8


def _pool():
    k = torch.zeros(NB, HKV, 16, D, dtype=torch.float16)
    return kvb.Pool.from_tensors(k, torch.zeros_like(k))


def _i32(*shape):
    return torch.zeros(*shape, dtype=torch.int32)


def _prefill_args():
    q = torch.zeros(10, HQ, D, dtype=torch.float16)
    kn = torch.zeros(10, HKV, D, dtype=torch.float16)
    return dict(pool=_pool(), q=q, k_new=kn, v_new=kn.clone(), cu_q_lens=_i32(B + 1),
                prefix_lens=_i32(B), block_tables=_i32(B, 4), scale=0.125, max_q_len=4,
                max_prefix_len=16)


@pytest.mark.parametrize("bad", [
    dict(cu_q_lens=torch.zeros(B + 1, dtype=torch.int64)),      # wrong element type
    dict(cu_q_lens=_i32(B)),                                   # one offset short
    dict(prefix_lens=_i32(2 * B)[::2]),                        # not contiguous
    dict(block_tables=_i32(B - 1, 4)),                         # a row short
    dict(block_tables=_i32(B, 8)[:, :4]),                      # a strided view
])
def test_prefill_rejects_bad_index_tensors(bad):
    a = _prefill_args()
    a.update(bad)
    name = next(iter(bad))
    with pytest.raises(ValueError, match=name):
        kvb.paged_prefill(**a)
    for k in ("k_new", "v_new"):
        a.pop(k)
    with pytest.raises(ValueError, match=name):
        kvb.paged_prefill_pooled(**a)


def test_prefill_write_rejects_a_short_slot_mapping():
    a = _prefill_args()
    with pytest.raises(ValueError, match="slot_mapping"):
        kvb.paged_prefill(**a, slot_mapping=torch.zeros(9, dtype=torch.int64))
    with pytest.raises(ValueError, match="slot_mapping"):
        kvb.paged_prefill(**a, slot_mapping=torch.zeros(11, dtype=torch.int64))
    with pytest.raises(ValueError, match="slot_mapping"):
        kvb.paged_prefill(**a, slot_mapping=_i32(10))


@pytest.mark.parametrize("bad", [
    dict(context_lens=torch.zeros(B, dtype=torch.int64)),
    dict(context_lens=_i32(B - 1)),
    dict(block_tables=_i32(B, 4).to(torch.int16)),
    dict(block_tables=_i32(B, 8)[:, ::2]),
])
def test_decode_rejects_bad_index_tensors(bad):
    a = dict(pool=_pool(), q=torch.zeros(B, HQ, D, dtype=torch.float16), context_lens=_i32(B),
             block_tables=_i32(B, 4), scale=0.125, max_context_len=64)
    a.update(bad)
    name = next(iter(bad))
    with pytest.raises(ValueError, match=name):
        kvb.paged_decode(**a)
    with pytest.raises(ValueError, match=name):
        kvb.paged_decode_noalloc(**a, out=torch.zeros_like(a["q"]))
    with pytest.raises(ValueError, match=name):
        kvb.paged_decode_cascade(**a, shared_blocks=None, shared_len=0)


def test_cascade_rejects_too_few_shared_blocks():
    with pytest.raises(ValueError, match="shared_blocks"):
        kvb.paged_decode_cascade(_pool(), torch.zeros(B, HQ, D, dtype=torch.float16), _i32(B),
                                 _i32(B, 4), _i32(2), 33, 0.125, 64)


def test_write_kv_needs_int64_slots_and_a_row_per_slot():
    kn = torch.zeros(4, HKV, D, dtype=torch.float16)
    with pytest.raises(ValueError, match="slot_mapping must"):
        kvb.write_kv(_pool(), kn, kn, _i32(4))
    with pytest.raises(ValueError, match="a row for every entry"):
        kvb.write_kv(_pool(), kn, kn, torch.zeros(5, dtype=torch.int64))


def test_copy_blocks_needs_block_ids_on_the_gpu():
    with pytest.raises(ValueError, match="src_ids"):
        kvb.copy_blocks(_pool(), _pool(), _i32(2), _i32(2))


def test_gather_kv_rejects_a_short_offset_list():
    k = torch.zeros(16, HKV, D, dtype=torch.float16)
    with pytest.raises(ValueError, match="cu_seq_lens"):
        kvb.gather_kv(_pool(), _i32(B, 4), _i32(B), _i32(B), 8, k, k.clone())



def test_well_formed_index_tensors_pass_their_checks():
    # With every index tensor well formed the calls stop only at the first tensor that is not
    # in GPU memory (all of them here, on the host).
    a = _prefill_args()
    calls = [
        lambda: kvb.paged_prefill(**a),
        lambda: kvb.paged_prefill(**a, slot_mapping=torch.zeros(10, dtype=torch.int64)),
        lambda: kvb.paged_decode_noalloc(_pool(), torch.zeros(B, HQ, D, dtype=torch.float16),
                                         _i32(B), _i32(B, 4), 0.125, 64,
                                         out=torch.zeros(B, HQ, D, dtype=torch.float16)),
        lambda: kvb.write_kv(_pool(), a["k_new"], a["v_new"], torch.zeros(6, dtype=torch.int64)),
    ]
    for call in calls:
        with pytest.raises(ValueError, match="must be a GPU tensor"):
            call()


def test_pools_in_pageable_host_memory_are_rejected():
    with pytest.raises(ValueError, match="pool tensors"):
        _pool().c_struct()
    codes = torch.zeros(NB, HKV, 16, D, dtype=torch.int8)
    q8 = kvb.PoolQ8(codes, codes.clone(), torch.zeros(NB, HKV, 16), torch.zeros(HKV, D))
    with pytest.raises(ValueError, match="pool tensors"):
        q8.c_struct()


def test_data_tensor_shapes_follow_the_pool():
    pool, f16 = _pool(), torch.float16
    q, kn = torch.zeros(5, HQ, D, dtype=f16), torch.zeros(5, HKV, D, dtype=f16)
    kvb._qkv(pool, q, kn, kn.clone(), torch.zeros_like(q))          # well formed: no error
    bad = [
        (dict(q=torch.zeros(5, HQ, D // 2, dtype=f16)), "q must"),   # head dim of another pool
        (dict(q=q.to(torch.bfloat16)), "q must"),                    # not the pool's dtype
        (dict(q=torch.zeros(5, 2 * HQ, D, dtype=f16)[:, ::2]), "q must"),
        (dict(out=torch.zeros(4, HQ, D, dtype=f16)), "out must"),
        (dict(k_new=torch.zeros(5, HKV + 1, D, dtype=f16)), "k_new must"),
        (dict(v_new=torch.zeros(4, HKV, D, dtype=f16)), "v_new must"),
    ]
    for change, msg in bad:
        a = dict(q=q, k_new=kn, v_new=kn, out=None)
        a.update(change)
        with pytest.raises(ValueError, match=msg):
            kvb._qkv(pool, **a)
    codes = torch.zeros(NB, HKV, 16, D, dtype=torch.int8)
    q8 = kvb.PoolQ8(codes, codes.clone(), torch.zeros(NB, HKV, 16), torch.zeros(HKV, D))
    kvb._qkv(q8, q.to(torch.bfloat16))                               # code pools take either
    with pytest.raises(ValueError, match="q must"):
        kvb._qkv(q8, q.float())
