"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, and every invalid argument is rejected on the host with the
documented status before anything is launched (no call here reaches a kernel)."""
import ctypes
import os
import re

import pytest

import quantized_routed_moe_router_amd as q
from quantized_routed_moe_router_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ds4moe.h")


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(ds4moe_\w+)\s*\(", txt)))


def test_header_symbols_exported():
    names = declared_functions()
    assert len(names) >= 9
    L = B.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(B.EXPORTED) == set(names)


def test_single_hip_runtime_loaded():
    maps = open("/proc/self/maps").read()
    paths = {l.split()[-1] for l in maps.splitlines() if "libamdhip64" in l}
    assert len(paths) == 1, paths


def test_version_and_status_strings():
    assert B.lib().ds4moe_version() >= 100
    for s in range(9):
        assert B.status_str(s)
    assert B.status_str(99) == "unknown status"


def test_build_keeps_common_code_sinking_off():
    """The prefill GEMMs inline one multiply instance per live n-tile count;
    with common-code sinking on, this compiler merged their final stores and
    then gave part of a loop-carried accumulator to scratch registers (wrong
    values in the down projection, caught by the GPU test that steers tokens
    to every n-tile count).  The build must keep the sinking off."""
    from quantized_routed_moe_router_amd import build
    flags = build.FLAGS
    i = flags.index("-simplifycfg-sink-common=false")
    assert flags[i - 1] == "-mllvm"
    assert "-Xclang" in flags and "-packed-fp32-ops" in flags   # no packed fp32 instructions


def test_read_probe_argument_errors():
    """The streaming-read probe rejects its arguments on the host (fake,
    never dereferenced addresses: every call returns before a launch)."""
    L = B.lib()
    P = ctypes.c_void_p
    ok, sink = P(0x10000), P(0x20000)
    ev = P(0x30000)
    assert L.ds4moe_read_probe(None, 4096, 8, sink, None, None, None) == 1
    assert L.ds4moe_read_probe(ok, 4096, 8, None, None, None, None) == 1
    assert L.ds4moe_read_probe(ok, 0, 8, sink, None, None, None) == 2
    assert L.ds4moe_read_probe(ok, 4104, 8, sink, None, None, None) == 2      # not a multiple of 16
    assert L.ds4moe_read_probe(ok, 4096, 0, sink, None, None, None) == 2
    assert L.ds4moe_read_probe(ok, 4096, (1 << 20) + 1, sink, None, None, None) == 2
    assert L.ds4moe_read_probe(P(0x10008), 4096, 8, sink, None, None, None) == 4
    assert L.ds4moe_read_probe(ok, 4096, 8, P(0x20002), None, None, None) == 4
    assert L.ds4moe_read_probe(ok, 4096, 8, sink, ev, None, None) == 1        # one event without the other
    assert L.ds4moe_read_probe(ok, 4096, 8, sink, None, ev, None) == 1


def test_packed_bytes():
    assert q.ds4moe_packed_bytes(2048, 4096) == 2048 * 4096 // 256 * 84 == 2752512
    assert q.ds4moe_packed_bytes(4096, 2048) == 2752512
    assert q.ds4moe_packed_bytes(256, 128) == 16 * 1 * 1344      # K=128 padded to 256
    assert q.ds4moe_packed_bytes(15, 256) == 0
    assert q.ds4moe_packed_bytes(16, 384) == 0
    assert q.ds4moe_packed_bytes(16, 8) == 0


def test_packed_bytes_bits():
    # 4-bit codes: 148 bytes per 256 weights, 2368 per 16 x 256 unit
    assert q.ds4moe_packed_bytes_bits(2048, 4096, 4) == 2048 * 4096 // 256 * 148 == 4849664
    assert q.ds4moe_packed_bytes_bits(256, 128, 4) == 16 * 2368
    assert q.ds4moe_packed_bytes_bits(2048, 4096, 2) == q.ds4moe_packed_bytes(2048, 4096)
    # 6-bit codes: 212 bytes per 256 weights, 3392 per unit; 5-bit codes share the 6-bit unit
    assert q.ds4moe_packed_bytes_bits(2048, 4096, 6) == 2048 * 4096 // 256 * 212
    assert q.ds4moe_packed_bytes_bits(2048, 4096, 5) == q.ds4moe_packed_bytes_bits(2048, 4096, 6)
    assert q.ds4moe_packed_bytes_bits(256, 128, 6) == 16 * 3392
    for bits in (0, 1, 3, 7, 8, -2):
        assert q.ds4moe_packed_bytes_bits(16, 256, bits) == 0
    assert q.ds4moe_packed_bytes_bits(15, 256, 4) == 0
    assert q.ds4moe_packed_bytes_bits(16, 384, 4) == 0
    assert q.ds4moe_packed_bytes_bits((1 << 31) + 16, 256, 4) == 0


def dims(**kw):
    d = dict(H=4096, I=2048, E=256, k=8, Is=0, x_dtype=B.DS4MOE_BF16, router_dtype=B.DS4MOE_BF16, bits=2)
    d.update(kw)
    return B.make_dims(d["H"], d["I"], d["E"], d["k"], d["Is"], d["x_dtype"], d["router_dtype"], d["bits"])


def test_workspace_bytes():
    d = dims()
    assert B.ds4moe_workspace_bytes(d, 0, B.MODE_PREFILL) == 256
    a = B.ds4moe_workspace_bytes(d, 16, B.MODE_DECODE)
    b = B.ds4moe_workspace_bytes(d, 2048, B.MODE_PREFILL)
    r = B.ds4moe_workspace_bytes(d, 2048, B.MODE_ROUTE)
    assert 0 < r < b and a > 0
    assert b >= 2048 * 8 * 4096 * 4                  # per-assignment outputs
    assert B.ds4moe_workspace_bytes(dims(H=100), 16, 1) == 0
    assert B.ds4moe_workspace_bytes(d, 16, 7) == 0
    assert B.lib().ds4moe_workspace_bytes(None, 16, 1) == 0


def test_workspace_bytes_grow_with_T():
    """A workspace sized for the largest batch serves every smaller one, in
    every mode, across the decode kernel classes and the prefill routing's
    chunk-size switch; decode T >= 5 holds the down projection's partials."""
    for d in (dims(), dims(Is=2048), dims(H=256, I=128, E=8, k=2, x_dtype=B.DS4MOE_F32, router_dtype=B.DS4MOE_F32)):
        for mode, Ts in ((B.MODE_DECODE, range(1, 17)),
                         (B.MODE_PREFILL, [0, 1, 16, 17, 64, 65, 2048, 4095, 4096, 4097, 4160, 8192]),
                         (B.MODE_ROUTE, [1, 16, 17, 4096, 4097, 8192])):
            sizes = [B.ds4moe_workspace_bytes(d, T, mode) for T in Ts]
            assert all(x > 0 for x in sizes), (mode, sizes)
            assert sizes == sorted(sizes), (mode, list(zip(Ts, sizes)))
    d = dims()
    for T in (5, 16):
        assert B.ds4moe_workspace_bytes(d, T, B.MODE_DECODE) >= 4 * T * 4096 * 4


@pytest.mark.parametrize("bad,status", [
    (dict(H=100), B.DS4MOE_ERR_SHAPE), (dict(H=0), B.DS4MOE_ERR_SHAPE), (dict(I=8), B.DS4MOE_ERR_SHAPE),
    (dict(I=384), B.DS4MOE_ERR_SHAPE), (dict(k=0), B.DS4MOE_ERR_SHAPE), (dict(k=17, E=32), B.DS4MOE_ERR_SHAPE),
    (dict(E=4, k=8), B.DS4MOE_ERR_SHAPE), (dict(E=300), B.DS4MOE_ERR_SHAPE), (dict(Is=100), B.DS4MOE_ERR_SHAPE),
    (dict(x_dtype=5), B.DS4MOE_ERR_DTYPE), (dict(router_dtype=-1), B.DS4MOE_ERR_DTYPE),
    (dict(bits=0), B.DS4MOE_ERR_SHAPE), (dict(bits=3), B.DS4MOE_ERR_SHAPE), (dict(bits=8), B.DS4MOE_ERR_SHAPE),
])
def test_bad_dims_rejected(bad, status):
    w = B.make_weights(16, 16, 16, 16)
    y = 16
    assert B.lib().ds4moe_forward_prefill(ctypes.byref(dims(**bad)), ctypes.byref(w), ctypes.c_void_p(16), 4,
                                          ctypes.c_void_p(y), None, ctypes.c_void_p(256), 1 << 40, None) == status


def call(fn, d=None, w=None, x=16, T=4, y=16, r=None, ws=256, ws_bytes=1 << 40):
    d = d or dims()
    w = w if w is not None else B.make_weights(16, 16, 16, 16)
    L = B.lib()
    args = [ctypes.byref(d), ctypes.byref(w) if w is not False else None, ctypes.c_void_p(x), T]
    if fn != "ds4moe_route":
        args.append(ctypes.c_void_p(y))
    args.append(ctypes.byref(r) if r is not None else (None if fn != "ds4moe_route" else None))
    args += [ctypes.c_void_p(ws), ws_bytes, None]
    return getattr(L, fn)(*args)


@pytest.mark.parametrize("fn", ["ds4moe_forward_decode", "ds4moe_forward_prefill"])
def test_forward_argument_errors(fn):
    assert call(fn, w=False) == B.DS4MOE_ERR_NULL
    assert call(fn, w=B.make_weights(None, 16, 16, 16)) == B.DS4MOE_ERR_NULL
    assert call(fn, w=B.make_weights(16, None, 16, 16)) == B.DS4MOE_ERR_NULL
    assert call(fn, w=B.make_weights(17, 16, 16, 16)) == B.DS4MOE_ERR_ALIGN
    assert call(fn, w=B.make_weights(16, 16, 24, 16)) == B.DS4MOE_ERR_ALIGN
    assert call(fn, w=B.make_weights(16, 16, 16, 16, router_bias=18)) == B.DS4MOE_ERR_ALIGN
    assert call(fn, x=0) == B.DS4MOE_ERR_NULL
    assert call(fn, y=0) == B.DS4MOE_ERR_NULL
    assert call(fn, x=8) == B.DS4MOE_ERR_ALIGN
    assert call(fn, ws=0) == B.DS4MOE_ERR_WORKSPACE
    assert call(fn, ws=128) == B.DS4MOE_ERR_ALIGN
    assert call(fn, ws_bytes=1000) == B.DS4MOE_ERR_WORKSPACE
    assert call(fn, T=-1) == B.DS4MOE_ERR_SHAPE
    assert call(fn, r=B.make_routing(topk_idx=18)) == B.DS4MOE_ERR_ALIGN
    # shared expert declared but weights missing
    assert call(fn, d=dims(Is=2048)) == B.DS4MOE_ERR_NULL
    # prefill: T = 0 is a no-op that touches nothing; decode needs 1 <= T <= 16
    expect = B.DS4MOE_OK if fn == "ds4moe_forward_prefill" else B.DS4MOE_ERR_SHAPE
    assert call(fn, T=0, x=0, y=0, ws=0) == expect


def test_decode_token_range():
    assert call("ds4moe_forward_decode", T=17) == B.DS4MOE_ERR_SHAPE
    assert call("ds4moe_forward_decode", T=0) == B.DS4MOE_ERR_SHAPE
    assert call("ds4moe_forward_prefill", T=(1 << 20) + 1) == B.DS4MOE_ERR_SHAPE


def test_route_argument_errors():
    L = B.lib()
    d, w, r = dims(), B.make_weights(16, None, None, None), B.make_routing()
    assert L.ds4moe_route(ctypes.byref(d), ctypes.byref(w), ctypes.c_void_p(16), 4, None, ctypes.c_void_p(256),
                          1 << 40, None) == B.DS4MOE_ERR_NULL
    assert L.ds4moe_route(ctypes.byref(d), ctypes.byref(w), ctypes.c_void_p(16), 4, ctypes.byref(r),
                          ctypes.c_void_p(256), 10, None) == B.DS4MOE_ERR_WORKSPACE
    assert L.ds4moe_route(ctypes.byref(d), ctypes.byref(w), ctypes.c_void_p(16), 0, ctypes.byref(r),
                          None, 0, None) == B.DS4MOE_OK


def test_pack_dequant_argument_errors():
    L = B.lib()
    v = ctypes.c_void_p
    assert L.ds4moe_pack_q2k(v(16), v(16), 1, 15, 256, None) == B.DS4MOE_ERR_SHAPE
    assert L.ds4moe_pack_q2k(v(16), v(16), -1, 16, 256, None) == B.DS4MOE_ERR_SHAPE
    assert L.ds4moe_pack_q2k(None, v(16), 1, 16, 256, None) == B.DS4MOE_ERR_NULL
    assert L.ds4moe_pack_q2k(v(8), v(16), 1, 16, 256, None) == B.DS4MOE_ERR_ALIGN
    assert L.ds4moe_pack_q2k(v(16), v(16), 0, 16, 256, None) == B.DS4MOE_OK
    assert L.ds4moe_dequant_q2k(v(16), None, 1, 16, 256, None) == B.DS4MOE_ERR_NULL
    assert L.ds4moe_dequant_q2k(v(16), v(8), 1, 16, 256, None) == B.DS4MOE_ERR_ALIGN
    assert L.ds4moe_dequant_q2k(v(16), v(16), 1, 16, 100, None) == B.DS4MOE_ERR_SHAPE
    for bits in (2, 4, 5, 6):
        assert L.ds4moe_pack(v(16), v(16), 1, 15, 256, bits, None) == B.DS4MOE_ERR_SHAPE
        assert L.ds4moe_pack(None, v(16), 1, 16, 256, bits, None) == B.DS4MOE_ERR_NULL
        assert L.ds4moe_pack(v(8), v(16), 1, 16, 256, bits, None) == B.DS4MOE_ERR_ALIGN
        assert L.ds4moe_pack(v(16), v(16), 0, 16, 256, bits, None) == B.DS4MOE_OK
        assert L.ds4moe_dequant(v(16), None, 1, 16, 256, bits, None) == B.DS4MOE_ERR_NULL
        assert L.ds4moe_dequant(v(16), v(8), 1, 16, 256, bits, None) == B.DS4MOE_ERR_ALIGN
        # more than 2^39 weights in one call: beyond the launch grids
        assert L.ds4moe_pack(v(16), v(16), 1 << 20, 4096, 4096, bits, None) == B.DS4MOE_ERR_SHAPE
        assert L.ds4moe_dequant(v(16), v(16), 1 << 20, 4096, 4096, bits, None) == B.DS4MOE_ERR_SHAPE
    assert L.ds4moe_pack(v(16), v(16), 1, 16, 256, 3, None) == B.DS4MOE_ERR_SHAPE
    assert L.ds4moe_pack(v(16), v(16), 1, 16, 256, 7, None) == B.DS4MOE_ERR_SHAPE
    assert L.ds4moe_dequant(v(16), v(16), 1, 16, 256, 1, None) == B.DS4MOE_ERR_SHAPE


def test_cache_bytes():
    d = dims()
    per_slot = 3 * q.ds4moe_packed_bytes(2048, 4096)
    b = B.ds4moe_cache_bytes(d, 204)
    assert 204 * per_slot < b < 204 * per_slot + 64 * 1024
    for bad in (0, -1, 257):
        assert B.ds4moe_cache_bytes(d, bad) == 0
    assert B.ds4moe_cache_bytes(dims(E=64), 65) == 0
    assert B.ds4moe_cache_bytes(dims(H=100), 8) == 0
    b4 = B.ds4moe_cache_bytes(dims(bits=4), 8)
    assert b4 > 8 * 3 * q.ds4moe_packed_bytes_bits(2048, 4096, 4)


def test_cache_argument_errors():
    L = B.lib()
    v = ctypes.c_void_p
    d = dims()
    nb = B.ds4moe_cache_bytes(d, 16)
    assert L.ds4moe_cache_reset(ctypes.byref(d), 16, None, nb, None) == B.DS4MOE_ERR_NULL
    assert L.ds4moe_cache_reset(ctypes.byref(d), 16, v(128), nb, None) == B.DS4MOE_ERR_ALIGN
    assert L.ds4moe_cache_reset(ctypes.byref(d), 16, v(256), nb - 1, None) == B.DS4MOE_ERR_WORKSPACE
    assert L.ds4moe_cache_reset(ctypes.byref(d), 0, v(256), nb, None) == B.DS4MOE_ERR_SHAPE
    assert L.ds4moe_cache_reset(ctypes.byref(d), 300, v(256), 1 << 40, None) == B.DS4MOE_ERR_SHAPE
    assert L.ds4moe_cache_reset(ctypes.byref(dims(bits=3)), 16, v(256), nb, None) == B.DS4MOE_ERR_SHAPE
    w = B.make_weights(16, 16, 16, 16)

    def fwd(S=16, T=1, cache=256, cb=1 << 40, wt=w):
        return L.ds4moe_forward_decode_cached(ctypes.byref(d), ctypes.byref(wt), S, v(cache), cb, v(16), T, v(16),
                                              None, v(256), 1 << 40, None, None)
    assert fwd(T=0) == B.DS4MOE_ERR_SHAPE
    assert fwd(T=17) == B.DS4MOE_ERR_SHAPE
    assert fwd(S=7, T=1) == B.DS4MOE_ERR_SHAPE           # fewer slots than the batch's k = 8 experts
    assert fwd(S=16, T=3) == B.DS4MOE_ERR_SHAPE          # 24 experts may be used at once
    assert fwd(cache=0) == B.DS4MOE_ERR_NULL
    assert fwd(cb=100) == B.DS4MOE_ERR_WORKSPACE
    assert fwd(wt=B.make_weights(16, None, 16, 16)) == B.DS4MOE_ERR_NULL
    assert fwd(wt=B.make_weights(16, 24, 16, 16)) == B.DS4MOE_ERR_ALIGN

    def pf(S=16, T=1, cache=256, cb=1 << 40, wt=w, ws=256, wsb=1 << 40):
        return L.ds4moe_forward_prefill_cached(ctypes.byref(d), ctypes.byref(wt), S, v(cache), cb, v(16), T, v(16),
                                               None, v(ws), wsb, None)
    # any slot count 1..E and any T up to 2^20: checks end before the pinned-memory query
    assert pf(T=0, S=1) == B.DS4MOE_OK                   # nothing to do, nothing launched
    assert pf(T=0, S=0) == B.DS4MOE_ERR_SHAPE
    assert pf(T=-1) == B.DS4MOE_ERR_SHAPE
    assert pf(T=(1 << 20) + 1) == B.DS4MOE_ERR_SHAPE
    assert pf(S=257) == B.DS4MOE_ERR_SHAPE
    assert pf(cache=0) == B.DS4MOE_ERR_NULL
    assert pf(cache=128) == B.DS4MOE_ERR_ALIGN
    assert pf(cb=100) == B.DS4MOE_ERR_WORKSPACE
    assert pf(ws=0) == B.DS4MOE_ERR_WORKSPACE
    assert pf(T=2048, wsb=B.ds4moe_workspace_bytes(d, 2048, B.MODE_PREFILL) - 1) == B.DS4MOE_ERR_WORKSPACE
    assert pf(wt=B.make_weights(16, None, 16, 16)) == B.DS4MOE_ERR_NULL
    assert pf(wt=B.make_weights(16, 24, 16, 16)) == B.DS4MOE_ERR_ALIGN
    out = (ctypes.c_uint64 * 3)()
    assert L.ds4moe_cache_stats(ctypes.byref(d), 16, v(256), nb, None, None) == B.DS4MOE_ERR_NULL
    assert L.ds4moe_cache_stats(ctypes.byref(d), 16, None, nb, out, None) == B.DS4MOE_ERR_NULL


def test_decode_noalloc_rejects_on_host():
    """The no-allocation decode checks every argument, and that the call's
    workspace fits the fixed scratch array, before any HIP call."""
    L = B.lib()
    d = dims()
    w = B.make_weights(256, 256, 256, 256)
    f = L.ds4moe_forward_decode_noalloc
    assert f(None, ctypes.byref(w), ctypes.c_void_p(256), 1, ctypes.c_void_p(256), None, None) == B.DS4MOE_ERR_NULL
    for T in (0, 17, -1):
        assert f(ctypes.byref(d), ctypes.byref(w), ctypes.c_void_p(256), T, ctypes.c_void_p(256), None,
                 None) == B.DS4MOE_ERR_SHAPE
    assert f(ctypes.byref(d), ctypes.byref(w), None, 1, ctypes.c_void_p(256), None, None) == B.DS4MOE_ERR_NULL
    assert f(ctypes.byref(d), ctypes.byref(w), ctypes.c_void_p(258), 1, ctypes.c_void_p(256), None,
             None) == B.DS4MOE_ERR_ALIGN
    big = dims(H=65536, I=32768, k=16, bits=4)       # decode workspace far above the scratch array
    assert B.ds4moe_workspace_bytes(big, 16, B.MODE_DECODE) > B.DS4MOE_NOALLOC_SCRATCH_BYTES
    assert f(ctypes.byref(big), ctypes.byref(w), ctypes.c_void_p(256), 16, ctypes.c_void_p(256), None,
             None) == B.DS4MOE_ERR_WORKSPACE
    # the full-size decode shapes fit: T = 16 with k = 16 and 4-bit experts
    full = dims(k=16, Is=2048, bits=4)
    assert B.ds4moe_workspace_bytes(full, 16, B.MODE_DECODE) <= B.DS4MOE_NOALLOC_SCRATCH_BYTES


def test_down_bits_validation():
    assert B.ds4moe_workspace_bytes(dims(), 16, B.MODE_DECODE) > 0
    d = B.make_dims(4096, 2048, 256, 8, 0, B.DS4MOE_BF16, B.DS4MOE_BF16, 2, 4)
    assert B.ds4moe_workspace_bytes(d, 16, B.MODE_DECODE) > 0
    for gu, dn in ((5, 6), (6, 0), (5, 0), (2, 5), (4, 6)):
        d = B.make_dims(4096, 2048, 256, 8, 0, B.DS4MOE_BF16, B.DS4MOE_BF16, gu, dn)
        assert B.ds4moe_workspace_bytes(d, 16, B.MODE_DECODE) > 0
    for gu in (1, 3, 7, 8):
        d = B.make_dims(4096, 2048, 256, 8, 0, B.DS4MOE_BF16, B.DS4MOE_BF16, gu, 0)
        assert B.ds4moe_workspace_bytes(d, 16, B.MODE_DECODE) == 0
    for bad in (1, 3, 7, 8, -2):
        d = B.make_dims(4096, 2048, 256, 8, 0, B.DS4MOE_BF16, B.DS4MOE_BF16, 2, bad)
        assert B.ds4moe_workspace_bytes(d, 16, B.MODE_DECODE) == 0
        w = B.make_weights(256, 256, 256, 256)
        assert B.lib().ds4moe_forward_decode(ctypes.byref(d), ctypes.byref(w), ctypes.c_void_p(256), 1,
                                             ctypes.c_void_p(256), None, ctypes.c_void_p(256), 1 << 30,
                                             None) == B.DS4MOE_ERR_SHAPE
    # a cache slot holds gate and up at expert_bits and down at down_bits
    d2 = B.make_dims(4096, 2048, 256, 8, 0, B.DS4MOE_BF16, B.DS4MOE_BF16, 2, 0)
    d4 = B.make_dims(4096, 2048, 256, 8, 0, B.DS4MOE_BF16, B.DS4MOE_BF16, 2, 4)
    assert B.ds4moe_cache_bytes(d4, 10) - B.ds4moe_cache_bytes(d2, 10) == 10 * (4849664 - 2752512)
    d56 = B.make_dims(4096, 2048, 256, 8, 0, B.DS4MOE_BF16, B.DS4MOE_BF16, 5, 6)
    assert B.ds4moe_cache_bytes(d56, 10) - B.ds4moe_cache_bytes(d2, 10) == 10 * 3 * (6946816 - 2752512)
