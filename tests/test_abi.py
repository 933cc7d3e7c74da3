"""The C-ABI library loads, exports every symbol include/kvb.h declares, and rejects bad
arguments on the host before any HIP call.  CPU only: the fake device pointers used
here are never dereferenced because validation fails first."""
import ctypes
import os
import re

import pytest

from attention_paged_prefix_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvb.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libkvb.so not built (run __graft_entry__.build())")

FAKE = 0x7F0000000000          # 16-byte aligned, never dereferenced
OK, NULL, INVALID, UNSUP, WS = 0, 1, 2, 3, 4


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvb_[a-z_0-9]+)\s*\(", text)))


def pool(**kw):
    p = dict(k=FAKE, v=FAKE + 4096, block_stride=2 * 16 * 128, num_blocks=8, block_size=16,
             num_kv_heads=2, head_dim=128, dtype=_lib.KVB_BF16)
    p.update(kw)
    return _lib.KvbPool(**p)


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version(lib):
    assert lib.kvb_status_str(0) == b"ok"
    assert lib.kvb_status_str(4).startswith(b"workspace")
    assert lib.kvb_version() == b"0.1.0"


def write(lib, p, n=4, kn=FAKE, vn=FAKE, slots=FAKE):
    return lib.kvb_write_kv(ctypes.byref(p), kn, vn, slots, n, None)


def test_write_kv_validation(lib):
    assert lib.kvb_write_kv(None, FAKE, FAKE, FAKE, 4, None) == NULL
    assert write(lib, pool(k=None)) == NULL
    assert write(lib, pool(block_size=32)) == UNSUP
    assert write(lib, pool(head_dim=80)) == UNSUP
    assert write(lib, pool(dtype=7)) == UNSUP
    assert write(lib, pool(block_stride=100)) == INVALID
    assert write(lib, pool(block_stride=2 * 16 * 128 + 4)) == INVALID
    assert write(lib, pool(block_stride=1 << 31)) == INVALID
    assert write(lib, pool(num_kv_heads=0)) == INVALID
    assert write(lib, pool(k=FAKE + 2)) == INVALID
    assert write(lib, pool(), n=-1) == INVALID
    assert write(lib, pool(), kn=None) == NULL
    assert write(lib, pool(), kn=FAKE + 8) == INVALID
    assert write(lib, pool(), slots=FAKE + 4) == INVALID
    assert write(lib, pool(), n=0) == OK          # nothing to do, no HIP call


def prefill(lib, p, **kw):
    a = dict(q=FAKE, kn=FAKE, vn=FAKE, out=FAKE, cu=FAKE, pl=FAKE, bt=FAKE, stride=4, batch=2,
             hq=4, total=10, maxq=6, maxp=64, scale=0.1, ws=None, wsb=0)
    a.update(kw)
    return lib.kvb_paged_prefill(ctypes.byref(p), a["q"], a["kn"], a["vn"], a["out"], a["cu"],
                                 a["pl"], a["bt"], a["stride"], a["batch"], a["hq"], a["total"],
                                 a["maxq"], a["maxp"], a["scale"], a["ws"], a["wsb"], None)


def test_prefill_validation(lib):
    p = pool()
    assert prefill(lib, p, hq=3) == INVALID           # not a multiple of num_kv_heads
    assert prefill(lib, p, hq=0) == INVALID
    assert prefill(lib, p, batch=-1) == INVALID
    assert prefill(lib, p, scale=float("nan")) == INVALID
    assert prefill(lib, p, scale=-1.0) == INVALID
    assert prefill(lib, p, q=None) == NULL
    assert prefill(lib, p, bt=None) == NULL
    assert prefill(lib, p, out=FAKE + 2) == INVALID
    assert prefill(lib, p, cu=FAKE + 2) == INVALID
    assert prefill(lib, p, maxq=11) == INVALID        # longer than total_q
    assert prefill(lib, p, stride=3) == INVALID       # ceil(64/16) = 4 entries needed
    assert prefill(lib, pool(head_dim=256)) == UNSUP
    assert prefill(lib, p, batch=0) == OK
    assert prefill(lib, p, total=0, maxq=0) == OK


def prefill_write(lib, p, **kw):
    a = dict(q=FAKE, kn=FAKE, vn=FAKE, out=FAKE, slots=FAKE, cu=FAKE, pl=FAKE, bt=FAKE, stride=4,
             batch=2, hq=4, total=10, maxq=6, maxp=64, scale=0.1, ws=None, wsb=0)
    a.update(kw)
    return lib.kvb_paged_prefill_write(ctypes.byref(p), a["q"], a["kn"], a["vn"], a["out"], a["slots"],
                                       a["cu"], a["pl"], a["bt"], a["stride"], a["batch"], a["hq"],
                                       a["total"], a["maxq"], a["maxp"], a["scale"], a["ws"], a["wsb"],
                                       None)


def test_prefill_write_validation(lib):
    p = pool()
    assert prefill_write(lib, p, slots=None) == NULL          # the slot mapping is required
    assert prefill_write(lib, p, slots=FAKE + 4) == INVALID    # int64: 8-byte aligned
    assert prefill_write(lib, p, hq=3) == INVALID
    assert prefill_write(lib, p, q=None) == NULL
    assert prefill_write(lib, p, stride=3) == INVALID
    assert prefill_write(lib, pool(head_dim=256)) == UNSUP
    assert prefill_write(lib, p, batch=0) == OK
    assert prefill_write(lib, p, total=0, maxq=0, slots=None) == OK


def decode(lib, p, **kw):
    a = dict(q=FAKE, out=FAKE, ctx=FAKE, bt=FAKE, stride=256, batch=4, hq=8, maxc=4000, sb=0,
             scale=0.1, ws=None, wsb=0)
    a.update(kw)
    return lib.kvb_paged_decode(ctypes.byref(p), a["q"], a["out"], a["ctx"], a["bt"], a["stride"],
                                a["batch"], a["hq"], a["maxc"], a["sb"], a["scale"], a["ws"],
                                a["wsb"], None)


def test_decode_validation_and_workspace(lib):
    p = pool()
    need = lib.kvb_paged_decode_workspace_size(4, 2, 8, 128, 4000, 0)
    assert need > 0
    assert decode(lib, p) == WS                       # split decode needs a workspace
    assert decode(lib, p, ws=FAKE, wsb=need - 1) == WS
    assert decode(lib, p, ws=FAKE + 8, wsb=need) == INVALID
    assert decode(lib, p, stride=249) == INVALID      # ceil(4000/16) = 250 entries needed
    assert decode(lib, p, hq=5) == INVALID
    assert decode(lib, p, sb=-2) == INVALID
    assert decode(lib, p, q=None) == NULL
    assert decode(lib, p, ctx=FAKE + 1) == INVALID
    assert decode(lib, p, batch=0) == OK
    # the balanced form always needs its header and records, whatever the split size
    assert lib.kvb_paged_decode_workspace_size(4, 2, 8, 128, 4000, 256) > 0
    # forced range of 16 blocks: 2 KV heads x 4 sequences x 250 blocks = 2000 blocks in
    # ranges of 16 -> 125 waves, rounded up to 128 (whole work-groups on all 8 XCDs);
    # records = waves + units (8) of 4 heads: a 256-byte header, then (max, sum) pairs
    # (rounded up to 256 bytes), then d floats per head
    assert lib.kvb_paged_decode_workspace_size(4, 2, 8, 128, 4000, 16) == 256 + 4352 + 136 * 4 * 128 * 4
    # ranges longer than 64 blocks are taken as 64
    assert (lib.kvb_paged_decode_workspace_size(4, 2, 8, 128, 4000, 256)
            == lib.kvb_paged_decode_workspace_size(4, 2, 8, 128, 4000, 64))


def test_decode_workspace_size_matches_the_call_when_every_context_is_empty(lib):
    """max_context_len 0 (every context empty): the call still writes the zero rows through
    its plan, and the size query reports that plan's workspace, so a caller that follows
    the query is not refused."""
    p = pool()
    need = lib.kvb_paged_decode_workspace_size(4, 2, 8, 128, 0, 0)
    assert need > 0
    assert decode(lib, p, maxc=0, stride=1) == WS
    assert decode(lib, p, maxc=0, stride=1, ws=FAKE, wsb=need - 1) == WS
    needc = lib.kvb_paged_decode_cascade_workspace_size(4, 2, 8, 128, 0, 0, 0)
    assert needc > 0


def decode_noalloc(lib, p, **kw):
    a = dict(q=FAKE, out=FAKE, ctx=FAKE, bt=FAKE, stride=256, batch=4, hq=8, maxc=4000, sb=0,
             scale=0.1)
    a.update(kw)
    return lib.kvb_paged_decode_noalloc(ctypes.byref(p), a["q"], a["out"], a["ctx"], a["bt"],
                                        a["stride"], a["batch"], a["hq"], a["maxc"], a["sb"],
                                        a["scale"], None)


def test_decode_noalloc_validation(lib):
    """The allocation-free decode validates like kvb_paged_decode and refuses, before any
    launch, a split plan whose partials exceed its static scratch (16 MiB)."""
    p = pool(num_kv_heads=8, block_stride=8 * 16 * 128)
    assert decode_noalloc(lib, p, hq=5) == INVALID
    assert decode_noalloc(lib, p, q=None) == NULL
    assert decode_noalloc(lib, p, out=FAKE + 2) == INVALID
    assert decode_noalloc(lib, p, stride=249) == INVALID
    assert decode_noalloc(lib, p, sb=-1) == INVALID
    assert decode_noalloc(lib, p, scale=float("inf")) == INVALID
    assert decode_noalloc(lib, pool(head_dim=80)) == UNSUP
    assert decode_noalloc(lib, p, batch=0) == OK
    # one-block ranges: 64 sequences x 8 KV heads x 250 blocks records of 4 heads x
    # (128 + 2) floats > 16 MiB
    need = lib.kvb_paged_decode_workspace_size(64, 8, 32, 128, 4000, 1)
    assert need > 16 << 20
    assert decode_noalloc(lib, p, batch=64, hq=32, sb=1) == 6
    assert lib.kvb_status_str(6).startswith(b"needs more scratch")


def cascade(lib, p, **kw):
    a = dict(q=FAKE, out=FAKE, ctx=FAKE, bt=FAKE, stride=256, shared=FAKE, slen=1024, batch=4,
             hq=8, maxc=4000, sb=0, scale=0.1, ws=None, wsb=0)
    a.update(kw)
    return lib.kvb_paged_decode_cascade(ctypes.byref(p), a["q"], a["out"], a["ctx"], a["bt"],
                                        a["stride"], a["shared"], a["slen"], a["batch"], a["hq"],
                                        a["maxc"], a["sb"], a["scale"], a["ws"], a["wsb"], None)


def test_cascade_decode_validation_and_workspace(lib):
    p = pool()
    need = lib.kvb_paged_decode_cascade_workspace_size(4, 2, 8, 128, 4000, 1024, 0)
    assert need > 0
    assert cascade(lib, p) == WS                      # always needs a workspace
    assert cascade(lib, p, ws=FAKE, wsb=need - 1) == WS
    assert cascade(lib, p, ws=FAKE + 8, wsb=need) == INVALID
    assert cascade(lib, p, slen=1000) == INVALID      # whole blocks only
    assert cascade(lib, p, slen=-16) == INVALID
    assert cascade(lib, p, shared=None) == NULL
    assert cascade(lib, p, shared=FAKE + 2) == INVALID
    assert cascade(lib, p, stride=249) == INVALID
    assert cascade(lib, p, hq=5) == INVALID
    assert cascade(lib, p, batch=0) == OK
    # no shared prefix: the shared block list may be NULL
    need0 = lib.kvb_paged_decode_cascade_workspace_size(4, 2, 8, 128, 4000, 0, 0)
    assert cascade(lib, p, shared=None, slen=0, ws=FAKE + 16, wsb=need0 - 1) == WS
    assert lib.kvb_paged_decode_cascade_workspace_size(4, 2, 8, 128, 4000, 1000, 0) == 0


def test_copy_blocks_validation(lib):
    p = pool()
    c = lambda a, b, **kw: lib.kvb_copy_blocks(ctypes.byref(a), ctypes.byref(b), kw.get("s", FAKE),
                                               kw.get("d", FAKE), kw.get("n", 4), None)
    assert lib.kvb_copy_blocks(None, ctypes.byref(p), FAKE, FAKE, 4, None) == NULL
    assert c(p, pool(head_dim=64)) == INVALID          # shapes must match
    assert c(p, pool(num_kv_heads=4)) == INVALID
    assert c(p, pool(dtype=_lib.KVB_FP16)) == INVALID
    assert c(p, p, n=-1) == INVALID
    assert c(p, p, n=0) == OK
    assert c(p, p, s=None) == NULL
    assert c(p, p, d=FAKE + 2) == INVALID


def pool_q8(**kw):
    p = dict(k=FAKE, v=FAKE + 4096, v_scale=FAKE + 8192, k_scale=FAKE + 12288,
             block_stride=2 * 16 * 128, num_blocks=8, block_size=16, num_kv_heads=2, head_dim=128)
    p.update(kw)
    return _lib.KvbPoolQ8(**p)


def test_q8_validation(lib):
    def w(p, **kw):
        return lib.kvb_write_kv_q8(ctypes.byref(p), kw.get("kn", FAKE), kw.get("vn", FAKE),
                                   kw.get("dt", _lib.KVB_BF16), kw.get("slots", FAKE), kw.get("n", 4), None)
    assert lib.kvb_write_kv_q8(None, FAKE, FAKE, 1, FAKE, 4, None) == NULL
    assert w(pool_q8(k_scale=None)) == NULL
    assert w(pool_q8(v_scale=FAKE + 4)) == INVALID
    assert w(pool_q8(block_stride=2 * 16 * 128 + 8)) == INVALID     # whole 16-byte units
    assert w(pool_q8(block_stride=16 * 128)) == INVALID             # < heads * 16 * head_dim
    assert w(pool_q8(head_dim=80)) == UNSUP
    assert w(pool_q8(block_size=8)) == UNSUP
    assert w(pool_q8(), dt=5) == UNSUP
    assert w(pool_q8(), kn=None) == NULL
    assert w(pool_q8(), slots=FAKE + 4) == INVALID
    assert w(pool_q8(), n=-1) == INVALID
    assert w(pool_q8(), n=0) == OK

    def d(p, **kw):
        return lib.kvb_paged_decode_q8(ctypes.byref(p), kw.get("dt", 1), kw.get("q", FAKE), FAKE, FAKE,
                                       FAKE, kw.get("stride", 256), kw.get("batch", 4), kw.get("hq", 8),
                                       4000, 0, 0.1, kw.get("ws", None), kw.get("wsb", 0), None)
    need = lib.kvb_paged_decode_workspace_size(4, 2, 8, 128, 4000, 0)
    assert d(pool_q8()) == WS                         # the split decode's workspace
    assert d(pool_q8(), ws=FAKE, wsb=need - 1) == WS
    assert d(pool_q8(), ws=FAKE + 8, wsb=need) == INVALID
    assert d(pool_q8(), stride=249) == INVALID
    assert d(pool_q8(), hq=5) == INVALID
    assert d(pool_q8(), dt=9) == UNSUP
    assert d(pool_q8(), q=None) == NULL
    assert d(pool_q8(), batch=0) == OK


def test_prefill_q8_validation(lib):
    def pq(p, **kw):
        a = dict(dt=1, q=FAKE, ws=None, wsb=0, stride=4, batch=2, hq=4, total=10, maxq=6, maxp=64)
        a.update(kw)
        return lib.kvb_paged_prefill_q8(ctypes.byref(p), a["dt"], a["q"], FAKE, FAKE, FAKE, FAKE, FAKE,
                                        FAKE, a["stride"], a["batch"], a["hq"], a["total"], a["maxq"],
                                        a["maxp"], 0.1, a["ws"], a["wsb"], None)
    need = lib.kvb_paged_prefill_q8_workspace_size(2, 2, 4, 128, 10, 64)
    # the codes are widened inside the prefill kernel: only its dispatch plan is needed
    assert need == lib.kvb_paged_prefill_workspace_size(2, 4, 128, 10, 64) > 0
    assert need == lib.kvb_paged_prefill_q8_workspace_size(2, 2, 4, 128, 10, 100000)
    p = pool_q8()
    assert pq(p, ws=FAKE, wsb=need - 1) == WS         # the plan's workspace is optional
    assert pq(p, ws=FAKE + 8, wsb=need) == INVALID
    assert pq(p, ws=FAKE, wsb=need, stride=3) == INVALID
    assert pq(p, ws=FAKE, wsb=need, hq=3) == INVALID
    assert pq(p, ws=FAKE, wsb=need, dt=4) == UNSUP
    assert pq(p, q=None) == NULL
    assert pq(p, batch=0) == OK
    assert lib.kvb_paged_prefill_q8_workspace_size(2, 2, 4, 80, 10, 64) == 0


def test_prefill_pooled_validation(lib):
    p = pool()
    def pp(**kw):
        a = dict(q=FAKE, out=FAKE, cu=FAKE, pl=FAKE, bt=FAKE, stride=200, batch=4, hq=8, T=512,
                 maxq=200, maxp=3000, scale=0.1)
        a.update(kw)
        return lib.kvb_paged_prefill_pooled(ctypes.byref(p), a["q"], a["out"], a["cu"], a["pl"],
                                            a["bt"], a["stride"], a["batch"], a["hq"], a["T"],
                                            a["maxq"], a["maxp"], a["scale"], None)
    assert pp(stride=187) == INVALID                  # ceil(3000 / 16) = 188 entries at least
    assert pp(q=None) == NULL
    assert pp(out=FAKE + 8) == INVALID
    assert pp(hq=5) == INVALID
    assert pp(maxq=600) == INVALID                    # longer than total_q
    assert pp(batch=0) == OK


def test_prefill_workspace_size_and_validation(lib):
    # dispatch plan: one int per work item, items <= batch * (ceil(total_q * hq / 128) + hq),
    # at most 8 x 4096, rounded up to 256 bytes
    assert lib.kvb_paged_prefill_workspace_size(8, 16, 128, 2048, 2048) == 8 * (256 + 16) * 4
    assert lib.kvb_paged_prefill_workspace_size(0, 16, 128, 2048, 2048) == 0
    assert lib.kvb_paged_prefill_workspace_size(64, 64, 128, 1 << 20, 0) == 8 * 4096 * 4
    assert lib.kvb_paged_prefill_workspace_size(1, 1, 64, 1, 0) == 256
    p = pool()
    need = lib.kvb_paged_prefill_workspace_size(2, 4, 128, 10, 64)
    assert prefill(lib, p, ws=FAKE, wsb=need - 1) == WS     # too small (optional, but checked)
    assert prefill(lib, p, ws=FAKE + 8, wsb=need) == INVALID


def test_gather_validation(lib):
    p = pool()
    assert lib.kvb_gather_kv(ctypes.byref(p), FAKE, 1, FAKE, FAKE, FAKE, FAKE, 2, 17, None) == INVALID
    assert lib.kvb_gather_kv(ctypes.byref(p), None, 2, FAKE, FAKE, FAKE, FAKE, 2, 17, None) == NULL
    assert lib.kvb_gather_kv(ctypes.byref(p), FAKE, 2, FAKE, FAKE, FAKE, FAKE, 0, 17, None) == OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        _lib.load()
