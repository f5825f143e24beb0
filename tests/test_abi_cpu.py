"""The C ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before any launch (no GPU needed)."""

import ctypes
import os
import re

import pytest

import paged_kv_cache_316_amd as pkv
from paged_kv_cache_316_amd._lib import PaPool, lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "pagedkv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("pa_cache_write", "pa_decode", "pa_prefill_chunk", "pa_copy_blocks",
                 "pa_alloc_create", "pa_alloc_append_slot", "pa_alloc_fork"):
        assert must in names


def test_library_exports_every_declared_symbol():
    L = lib()
    missing = [n for n in declared_functions() if not hasattr(L, n)]
    assert not missing, missing
    # and the ctypes signatures cover all of them
    assert set(declared_functions()) <= set(pkv.SIGNATURES)


def test_status_strings_and_version():
    L = lib()
    assert L.pa_status_string(0) == b"ok"
    for s in range(-6, 0):
        assert L.pa_status_string(s) not in (b"", b"unknown status")
    assert L.pa_version() >= 10000


def _pool(**kw):
    base = dict(k_pool=16, v_pool=32, num_blocks=4, num_kv_heads=2, block_size=16, head_dim=128,
                dtype=1)
    base.update(kw)
    return PaPool(base["k_pool"], base["v_pool"], base["num_blocks"], base["num_kv_heads"],
                  base["block_size"], base["head_dim"], base["dtype"])


@pytest.mark.parametrize("bad,status", [
    (dict(block_size=12), -1), (dict(block_size=512), -1), (dict(head_dim=96), -2),
    (dict(dtype=7), -2), (dict(num_blocks=0), -1), (dict(k_pool=0), -1)])
def test_pool_validation_rejects_before_launch(bad, status):
    L = lib()
    p = _pool(**bad)
    assert L.pa_cache_write(ctypes.byref(p), 16, 16, 16, 1, None) == status
    assert L.pa_last_error()
    assert L.pa_copy_blocks(ctypes.byref(p), 16, 1, None) == status


def test_decode_argument_checks():
    L = lib()
    p = _pool(num_kv_heads=8)
    # q heads not a multiple of KV heads
    st = L.pa_decode(16, 16, ctypes.byref(p), 16, 4, 16, 2, 12, 0.1, 0, 16, 1 << 20, None)
    assert st == -1 and b"multiple" in L.pa_last_error()
    # negative worker count
    st = L.pa_decode(16, 16, ctypes.byref(p), 16, 4, 16, 2, 8, 0.1, -3, 16, 1 << 20, None)
    assert st == -1
    # workspace missing or too small
    need = L.pa_decode_workspace_bytes(2, 8, 8, 128, 0)
    assert need > 0
    assert L.pa_decode(16, 16, ctypes.byref(p), 16, 4, 16, 2, 8, 0.1, 0, None, 0, None) == -5
    assert L.pa_decode(16, 16, ctypes.byref(p), 16, 4, 16, 2, 8, 0.1, 0, 16, need - 1, None) == -5
    # NULL output
    st = L.pa_decode(None, 16, ctypes.byref(p), 16, 4, 16, 2, 8, 0.1, 0, 16, need, None)
    assert st == -1
    # misaligned q / workspace
    assert L.pa_decode(16, 18, ctypes.byref(p), 16, 4, 16, 2, 8, 0.1, 0, 16, need, None) == -1
    assert L.pa_decode(16, 16, ctypes.byref(p), 16, 4, 16, 2, 8, 0.1, 0, 24, need, None) == -1
    # zero sequences is a no-op
    assert L.pa_decode(None, None, ctypes.byref(p), None, 4, None, 0, 8, 0.1, 0, None, 0, None) == 0


def test_workspace_formula():
    L = lib()
    # MHA, 100 workers: 2*100 slots x 2 heads (FP8 MHA pairs KV heads) x 128 floats,
    # a 128-byte line of (m, l) records per slot, and 100 split records
    assert L.pa_decode_workspace_bytes(64, 40, 40, 128, 100) == 400 * 128 * 4 + 200 * 128 + 100 * 16
    # GQA 64/8: 8 query heads per unit
    n = L.pa_decode_workspace_bytes(256, 64, 8, 128, 10)
    assert n == 20 * 8 * 128 * 4 + 20 * 128 + 10 * 16
    assert L.pa_decode_workspace_bytes(4, 6, 4, 128, 10) == 0  # 6 not a multiple of 4


def test_mixed_workspace_formula():
    L = lib()
    # short chunks (4 rows x 8 query heads per KV head = 32 columns): the
    # multi-row decode, 2 slots per worker of 32 columns, each D bf16 values and
    # an 8-byte (m, l) record, plus 100 split records
    assert (L.pa_attention_mixed_workspace_bytes(0, 256, 64, 8, 128, 4, 100)
            == 2 * 100 * 32 * 128 * 2 + 2 * 100 * 32 * 8 + 100 * 16)
    assert (L.pa_attention_mixed_workspace_bytes(3, 5, 16, 16, 64, 32, 7)
            == 2 * 7 * 32 * 64 * 2 + 2 * 7 * 32 * 8 + 7 * 16)
    # decode rows only: the decode's workspace
    assert (L.pa_attention_mixed_workspace_bytes(64, 0, 64, 8, 128, 0, 10)
            == L.pa_decode_workspace_bytes(64, 64, 8, 128, 10))
    # 5 rows x 8 heads do not fit 32 columns: chunks go to the prefill kernel,
    # which needs no workspace; with no decode rows only the 16-byte minimum
    assert L.pa_attention_mixed_workspace_bytes(0, 8, 64, 8, 128, 5, 10) == 16
    assert (L.pa_attention_mixed_workspace_bytes(4, 8, 64, 8, 128, 512, 10)
            == L.pa_decode_workspace_bytes(4, 64, 8, 128, 10))
    # invalid sizes
    assert L.pa_attention_mixed_workspace_bytes(0, 8, 6, 4, 128, 4, 10) == 0
    assert L.pa_attention_mixed_workspace_bytes(-1, 8, 64, 8, 128, 4, 10) == 0
    assert L.pa_attention_mixed_workspace_bytes(0, 8, 64, 8, 128, -1, 10) == 0


def test_prefill_argument_checks():
    L = lib()
    p = _pool(dtype=0)
    st = L.pa_prefill_chunk(16, 16, 16, 16, ctypes.byref(p), 16, 4, 2, 2, 64, 0.1, None)
    assert st in (-2, -1)
    assert L.pa_prefill_chunk(16, 16, 16, 16, ctypes.byref(_pool()), 16, 4, 0, 2, 64, 0.1, None) == 0


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    from paged_kv_cache_316_amd import _lib
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="no CPU or Python fallback"):
        _lib.lib()


def test_stream_probe_rejects_bad_arguments():
    L = lib()
    assert L.pa_probe_stream_read(None, 0, 0, None, None) == 0  # no bytes: no-op
    assert L.pa_probe_stream_read(None, 16, 0, 16, None) == -1  # NULL buffer
    assert L.pa_probe_stream_read(16, 24, 0, 16, None) == -1  # bytes not a multiple of 16
    assert L.pa_probe_stream_read(8, 16, 0, 16, None) == -1  # unaligned buffer
    assert L.pa_last_error()


def test_fp8_pool_validation():
    L = lib()
    ok = _pool(dtype=2)
    ok.k_scale, ok.v_scale = 0.5, 2.0
    # a valid FP8 pool passes the pool checks (then fails on the NULL arrays)
    assert L.pa_cache_write(ctypes.byref(ok), None, None, None, 1, None) == -1
    assert b"NULL" in L.pa_last_error()
    for ks, vs in ((0.0, 1.0), (1.0, -1.0), (float("inf"), 1.0), (1.0, float("nan"))):
        p = _pool(dtype=2)
        p.k_scale, p.v_scale = ks, vs
        assert L.pa_cache_write(ctypes.byref(p), 16, 16, 16, 1, None) == -1
        assert b"scale" in L.pa_last_error()
    # chunked prefill is built for bf16 pools only
    assert L.pa_prefill_chunk(16, 16, 16, 16, ctypes.byref(ok), 16, 4, 1, 8, 16,
                              ctypes.c_float(0.1), None) == -2


def test_shared_prefix_argument_checks():
    L = lib()
    p = _pool(num_kv_heads=8)
    need = L.pa_decode_shared_prefix_workspace_bytes(2, 8, 8, 128, 16, 3, 0)
    assert need > L.pa_decode_workspace_bytes(2, 8, 8, 128, 0)
    args = lambda **kw: [kw.get("out", 16), kw.get("q", 16), ctypes.byref(kw.get("pool", p)), 16,
                         kw.get("maxb", 4), 16, kw.get("S", 2), kw.get("Hq", 8),
                         ctypes.c_float(0.1), kw.get("P", 3), kw.get("workers", 0),
                         kw.get("ws", 16), kw.get("wsb", need), None]
    call = lambda **kw: L.pa_decode_shared_prefix(*args(**kw))
    assert call(P=5) == -1 and b"num_prefix_blocks" in L.pa_last_error()  # P > max_blocks
    assert call(P=-1) == -1
    assert call(Hq=12) == -1 and b"multiple" in L.pa_last_error()
    assert call(ws=None) == -5
    assert call(wsb=need - 1) == -5
    assert call(out=None) == -1
    assert call(q=18) == -1  # misaligned
    assert call(pool=_pool(num_kv_heads=8, dtype=0)) == -2  # fp32 pools: not built
    assert call(S=0, out=None, q=None) == 0  # no sequences: no-op
    # workspace sizes grow with the prefix partials and are 0 for bad sizes
    assert L.pa_decode_shared_prefix_workspace_bytes(2, 6, 4, 128, 16, 3, 0) == 0
    assert L.pa_decode_shared_prefix_workspace_bytes(2, 8, 8, 128, 16, -1, 0) == 0


def test_shared_prefix_workspace_formula():
    L = lib()
    # 2 seqs, 2 heads (MHA), D 128, 10 workers, 256 blocks of 16: 256 tiles of 16
    # keys, 1 column block per KV head -> 2 waves per key range; about 4 waves
    # per CU on 256 CUs wants 512 ranges, capped at 256/8 = 32 ranges of 8 tiles
    dec = L.pa_decode_workspace_bytes(2, 2, 2, 128, 10)
    assert dec == 2 * 10 * 2 * 128 * 4 + 2 * 10 * 128 + 10 * 16
    n = L.pa_decode_shared_prefix_workspace_bytes(2, 2, 2, 128, 16, 256, 10)
    # tail lse (4 floats), 32 x (m, l) and 32 x 128 bf16 partial sums per row
    assert n == dec + 16 + 32 * 4 * 8 + 32 * 4 * 128 * 2


def test_mixed_argument_checks():
    L = lib()
    p = _pool(num_kv_heads=8)
    need = L.pa_decode_workspace_bytes(3, 8, 8, 128, 0)
    f = ctypes.c_float(0.1)
    call = lambda pool=p, nd=3, npf=2, ws=16, wsb=need, out=16, loc=16, mq=64: \
        L.pa_attention_mixed(out, 16, loc, 16, ctypes.byref(pool), 16, 4, nd, npf, 8, mq, f, 0, ws,
                             wsb, None)
    assert call(nd=0, npf=0, out=None) == 0               # empty batch: no-op
    assert call(nd=-1) == -1
    assert call(mq=-1) == -1
    assert call(out=None) == -1
    assert call(loc=None) == -1                            # chunks need q_start_loc
    assert call(ws=None) == -5                             # decode rows need the workspace
    # beside chunks the decode defaults to 2 waves per CU (256 CUs without a device)
    assert call(wsb=L.pa_decode_workspace_bytes(3, 8, 8, 128, 2 * 256) - 1) == -5
    fp8 = _pool(num_kv_heads=8, dtype=2)
    fp8.k_scale, fp8.v_scale = 1.0, 1.0
    assert call(pool=fp8) == -2 and b"bf16" in L.pa_last_error()  # FP8 chunks: not built


def test_swap_argument_checks():
    L = lib()
    dev = _pool(num_blocks=4)
    host = _pool(num_blocks=6)
    pairs = lambda *ps: (ctypes.c_int32 * (2 * len(ps)))(*[x for p in ps for x in p])
    call = lambda d=dev, h=host, pr=pairs((0, 5), (3, 1)), n=2, dirn=0: \
        L.pa_swap_blocks(ctypes.byref(d), ctypes.byref(h), pr, n, dirn, None)
    assert call(n=0, pr=None) == 0                                  # nothing to move
    assert call(dirn=2) == -1 and b"direction" in L.pa_last_error()
    assert call(h=_pool(num_blocks=6, head_dim=64)) == -1             # geometry differs
    assert call(h=_pool(num_blocks=6, dtype=0)) == -1                 # dtype differs
    assert call(pr=None) == -1
    assert call(pr=pairs((0, 6), (3, 1))) == -1 and b"outside" in L.pa_last_error()  # host id 6
    assert call(pr=pairs((4, 0), (3, 1))) == -1                       # device id 4
    # swap in: sources are host ids (0..5), destinations device ids (0..3)
    assert call(pr=pairs((5, 4)), n=1, dirn=1) == -1 and b"outside" in L.pa_last_error()
    assert call(pr=pairs((5, 3), (4, 1)), dirn=1) == -1 and b"pool memory" in L.pa_last_error()
    assert call(pr=pairs((0, 5), (3, 5))) == -1 and b"twice" in L.pa_last_error()
    # fp8 pools must agree on their scales
    d8, h8 = _pool(dtype=2), _pool(dtype=2, num_blocks=6)
    d8.k_scale = d8.v_scale = h8.k_scale = 1.0
    h8.v_scale = 2.0
    assert call(d=d8, h=h8) == -1 and b"scale" in L.pa_last_error()
    # past the host checks the pointers are looked up: fake addresses are refused
    assert call() == -1 and b"pool memory" in L.pa_last_error()


@pytest.mark.parametrize("scale", [0.0, -0.125, float("inf"), float("-inf"), float("nan")])
def test_every_attention_call_rejects_bad_scales(scale):
    """The softmax scale must be finite and > 0 in every attention entry point."""
    L = lib()
    p = _pool(num_kv_heads=8)
    f = ctypes.c_float(scale)
    need = L.pa_decode_workspace_bytes(2, 8, 8, 128, 0)
    assert L.pa_decode(16, 16, ctypes.byref(p), 16, 4, 16, 2, 8, f, 0, 16, need, None) == -1
    assert b"scale" in L.pa_last_error()
    nsp = L.pa_decode_shared_prefix_workspace_bytes(2, 8, 8, 128, 16, 1, 0)
    assert L.pa_decode_shared_prefix(16, 16, ctypes.byref(p), 16, 4, 16, 2, 8, f, 1, 0, 16, nsp,
                                     None) == -1
    assert b"scale" in L.pa_last_error()
    assert L.pa_prefill_chunk(16, 16, 16, 16, ctypes.byref(p), 16, 4, 2, 8, 64, f, None) == -1
    assert b"scale" in L.pa_last_error()
    assert L.pa_attention_mixed(16, 16, 16, 16, ctypes.byref(p), 16, 4, 1, 1, 8, 64, f, 0, 16,
                                1 << 24, None) == -1
    assert b"scale" in L.pa_last_error()


def test_noalloc_decode_argument_checks():
    """pa_decode_noalloc checks its arguments like pa_decode and refuses a call
    whose workspace would not fit its static scratch array, before any launch."""
    L = lib()
    p = _pool(num_kv_heads=8)
    cap = L.pa_decode_noalloc_scratch_bytes()
    assert cap == 32 << 20
    f = ctypes.c_float(0.1)
    call = lambda out=16, Hq=8, workers=0, scale=f, S=2: L.pa_decode_noalloc(
        out, 16, ctypes.byref(p), 16, 4, 16, S, Hq, scale, workers, None)
    assert call(S=0, out=None) == 0                       # nothing to do
    assert call(Hq=12) == -1 and b"multiple" in L.pa_last_error()
    assert call(out=None) == -1
    assert call(scale=ctypes.c_float(-1.0)) == -1
    assert call(workers=-2) == -1
    # G = 1 MHA: 2 * W * 2 * (128 * 4 + 8) + 16 W bytes; 1 << 14 workers need 34.3 MB
    assert L.pa_decode_workspace_bytes(2, 8, 8, 128, 1 << 14) > cap
    assert call(workers=1 << 14) == -5 and b"scratch" in L.pa_last_error()


def test_grouped_decode_argument_checks():
    L = lib()
    p = _pool(num_kv_heads=8)
    need = L.pa_decode_grouped_workspace_bytes(6, 8, 8, 128, 10)
    # 16 columns per partial slot: 2 * 10 * 16 * (128 * 4 + 8) + 10 * 16
    assert need == 2 * 10 * 16 * (128 * 4 + 8) + 10 * 16
    f = ctypes.c_float(0.1)
    call = lambda S=6, M=3, Hq=8, pool=p, pl=16, ws=16, wsb=need, workers=10, scale=f: \
        L.pa_decode_grouped(16, 16, ctypes.byref(pool), 16, 4, 16, pl, S, M, Hq, scale, workers,
                            ws, wsb, None)
    assert call(S=0) == 0                                     # nothing to do
    assert call(M=4) == -1 and b"multiple of group_size" in L.pa_last_error()
    assert call(M=0) == -1
    assert call(pl=None) == -1 and b"prefix_lens" in L.pa_last_error()
    assert call(pool=_pool(num_kv_heads=8, dtype=0)) == -2   # fp32 pools: not built
    assert call(Hq=8 * 17, pool=_pool(num_kv_heads=8)) == -2 and b"columns" in L.pa_last_error()
    assert call(ws=None) == -5 and call(wsb=need - 1) == -5
    assert call(scale=ctypes.c_float(0.0)) == -1
    assert L.pa_decode_grouped_workspace_bytes(6, 6, 4, 128, 0) == 0  # 6 not a multiple of 4
