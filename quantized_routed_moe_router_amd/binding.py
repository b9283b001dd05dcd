"""ctypes binding of libds4moe.so: the same entry points as include/ds4moe.h.

Argument marshalling only -- every step of the layer runs in the library's
HIP kernels.  Tensors are torch tensors on the GPU (torch provides device
memory and streams); their data pointers are handed to the library.  torch is
imported before the library is loaded so that both share one HIP runtime.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must be loaded before libds4moe.so: one HIP runtime)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libds4moe.so")

DS4MOE_OK = 0
DS4MOE_ERR_NULL = 1
DS4MOE_ERR_SHAPE = 2
DS4MOE_ERR_DTYPE = 3
DS4MOE_ERR_ALIGN = 4
DS4MOE_ERR_WORKSPACE = 5
DS4MOE_ERR_UNSUPPORTED = 6
DS4MOE_ERR_HIP = 7
DS4MOE_ERR_HOSTMEM = 8
DS4MOE_NOALLOC_SCRATCH_BYTES = 32 << 20
DS4MOE_F32 = 0
DS4MOE_BF16 = 1
MODE_ROUTE, MODE_DECODE, MODE_PREFILL = 0, 1, 2

EXPORTED = ("ds4moe_packed_bytes", "ds4moe_packed_bytes_bits", "ds4moe_pack_q2k", "ds4moe_pack",
            "ds4moe_dequant_q2k", "ds4moe_dequant", "ds4moe_workspace_bytes",
            "ds4moe_route", "ds4moe_forward_decode", "ds4moe_forward_prefill", "ds4moe_status_str",
            "ds4moe_version", "ds4moe_forward_timed", "ds4moe_cache_bytes", "ds4moe_cache_reset",
            "ds4moe_forward_decode_cached", "ds4moe_forward_prefill_cached", "ds4moe_cache_stats",
            "ds4moe_forward_decode_noalloc",
            "ds4moe_read_probe")
N_TIMED_KERNELS = 11
KERNEL_SLOTS = ("router", "route", "permute", "gateup", "down", "shared_gateup", "shared_down", "combine",
                "cache_plan", "cache_fill", "shared_convert")


class Dims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("shared_inter", ctypes.c_int32), ("x_dtype", ctypes.c_int32),
                ("router_dtype", ctypes.c_int32), ("expert_bits", ctypes.c_int32), ("down_bits", ctypes.c_int32)]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("router_w", "router_bias", "gate", "up", "down", "sh_gate", "sh_up", "sh_down")]


class Routing(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("topk_idx", "topk_w", "counts", "offsets", "perm", "logits")]


class Ds4MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: status {status} ({status_str(status)})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load the built library; fail loudly if it is missing (no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python quantized_routed_moe_router_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        L.ds4moe_packed_bytes.argtypes = [I64, I64]
        L.ds4moe_packed_bytes.restype = ctypes.c_size_t
        L.ds4moe_packed_bytes_bits.argtypes = [I64, I64, I32]
        L.ds4moe_packed_bytes_bits.restype = ctypes.c_size_t
        L.ds4moe_pack_q2k.argtypes = [P, P, I64, I64, I64, P]
        L.ds4moe_dequant_q2k.argtypes = [P, P, I64, I64, I64, P]
        L.ds4moe_pack.argtypes = [P, P, I64, I64, I64, I32, P]
        L.ds4moe_dequant.argtypes = [P, P, I64, I64, I64, I32, P]
        L.ds4moe_workspace_bytes.argtypes = [P, I32, I32]
        L.ds4moe_workspace_bytes.restype = ctypes.c_size_t
        L.ds4moe_route.argtypes = [P, P, P, I32, P, P, ctypes.c_size_t, P]
        L.ds4moe_forward_decode.argtypes = [P, P, P, I32, P, P, P, ctypes.c_size_t, P]
        L.ds4moe_forward_prefill.argtypes = [P, P, P, I32, P, P, P, ctypes.c_size_t, P]
        L.ds4moe_forward_timed.argtypes = [I32, P, P, P, I32, P, P, P, ctypes.c_size_t, P, P]
        L.ds4moe_cache_bytes.argtypes = [P, I32]
        L.ds4moe_cache_bytes.restype = ctypes.c_size_t
        L.ds4moe_cache_reset.argtypes = [P, I32, P, ctypes.c_size_t, P]
        L.ds4moe_forward_decode_cached.argtypes = [P, P, I32, P, ctypes.c_size_t, P, I32, P, P, P, ctypes.c_size_t,
                                                   P, P]
        L.ds4moe_forward_prefill_cached.argtypes = [P, P, I32, P, ctypes.c_size_t, P, I32, P, P, P, ctypes.c_size_t,
                                                    P]
        L.ds4moe_cache_stats.argtypes = [P, I32, P, ctypes.c_size_t, P, P]
        L.ds4moe_forward_decode_noalloc.argtypes = [P, P, P, I32, P, P, P]
        L.ds4moe_read_probe.argtypes = [P, ctypes.c_size_t, I32, P, P, P, P]
        L.ds4moe_status_str.argtypes = [ctypes.c_int]
        L.ds4moe_status_str.restype = ctypes.c_char_p
        L.ds4moe_version.restype = ctypes.c_int
        for fn in ("ds4moe_pack_q2k", "ds4moe_dequant_q2k", "ds4moe_pack", "ds4moe_dequant", "ds4moe_route",
                   "ds4moe_cache_reset", "ds4moe_forward_decode_cached", "ds4moe_forward_prefill_cached",
                   "ds4moe_cache_stats",
                   "ds4moe_forward_decode", "ds4moe_forward_decode_noalloc", "ds4moe_read_probe",
                   "ds4moe_forward_prefill", "ds4moe_forward_timed"):
            getattr(L, fn).restype = ctypes.c_int
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().ds4moe_status_str(int(status)).decode()


def _ptr(t) -> ctypes.c_void_p | None:
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(status: int, what: str) -> None:
    if status != DS4MOE_OK:
        raise Ds4MoeError(status, what)


def make_dims(H, I, E, k, Is=0, x_dtype=DS4MOE_BF16, router_dtype=DS4MOE_BF16, expert_bits=2, down_bits=0) -> Dims:
    """down_bits = 0: the down matrices use expert_bits too."""
    return Dims(H, I, E, k, Is, x_dtype, router_dtype, expert_bits, down_bits)


def make_weights(router_w, gate, up, down, router_bias=None, sh_gate=None, sh_up=None, sh_down=None) -> Weights:
    return Weights(*(_ptr(t) for t in (router_w, router_bias, gate, up, down, sh_gate, sh_up, sh_down)))


def make_routing(topk_idx=None, topk_w=None, counts=None, offsets=None, perm=None, logits=None) -> Routing:
    return Routing(*(_ptr(t) for t in (topk_idx, topk_w, counts, offsets, perm, logits)))


# ---------------------------------------------------------------- entry points


def ds4moe_packed_bytes(rows: int, cols: int) -> int:
    return int(lib().ds4moe_packed_bytes(rows, cols))


def ds4moe_packed_bytes_bits(rows: int, cols: int, bits: int) -> int:
    return int(lib().ds4moe_packed_bytes_bits(rows, cols, bits))


def ds4moe_pack_q2k(dst, canonical, n_mats: int, rows: int, cols: int, stream=None) -> None:
    _check(lib().ds4moe_pack_q2k(_ptr(dst), _ptr(canonical), n_mats, rows, cols, _stream(stream)), "pack_q2k")


def ds4moe_dequant_q2k(dst, packed, n_mats: int, rows: int, cols: int, stream=None) -> None:
    _check(lib().ds4moe_dequant_q2k(_ptr(dst), _ptr(packed), n_mats, rows, cols, _stream(stream)), "dequant_q2k")


def ds4moe_pack(dst, canonical, n_mats: int, rows: int, cols: int, bits: int, stream=None) -> None:
    _check(lib().ds4moe_pack(_ptr(dst), _ptr(canonical), n_mats, rows, cols, bits, _stream(stream)), "pack")


def ds4moe_dequant(dst, packed, n_mats: int, rows: int, cols: int, bits: int, stream=None) -> None:
    _check(lib().ds4moe_dequant(_ptr(dst), _ptr(packed), n_mats, rows, cols, bits, _stream(stream)), "dequant")


def ds4moe_workspace_bytes(dims: Dims, T: int, mode: int) -> int:
    return int(lib().ds4moe_workspace_bytes(ctypes.byref(dims), T, mode))


def ds4moe_route(dims: Dims, weights: Weights, x, T: int, routing: Routing, ws, ws_bytes: int, stream=None) -> None:
    _check(lib().ds4moe_route(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), T, ctypes.byref(routing),
                              _ptr(ws), ws_bytes, _stream(stream)), "route")


def ds4moe_forward_decode(dims: Dims, weights: Weights, x, T: int, y, routing: Routing | None, ws, ws_bytes: int,
                          stream=None) -> None:
    r = ctypes.byref(routing) if routing is not None else None
    _check(lib().ds4moe_forward_decode(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), T, _ptr(y), r,
                                       _ptr(ws), ws_bytes, _stream(stream)), "forward_decode")


def ds4moe_forward_decode_noalloc(dims: Dims, weights: Weights, x, T: int, y, routing: Routing | None,
                                  stream=None) -> None:
    """ds4moe_forward_decode on the library's fixed per-GPU scratch array (no workspace)."""
    r = ctypes.byref(routing) if routing is not None else None
    _check(lib().ds4moe_forward_decode_noalloc(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), T, _ptr(y), r,
                                               _stream(stream)), "forward_decode_noalloc")


def ds4moe_forward_prefill(dims: Dims, weights: Weights, x, T: int, y, routing: Routing | None, ws, ws_bytes: int,
                           stream=None) -> None:
    r = ctypes.byref(routing) if routing is not None else None
    _check(lib().ds4moe_forward_prefill(ctypes.byref(dims), ctypes.byref(weights), _ptr(x), T, _ptr(y), r,
                                        _ptr(ws), ws_bytes, _stream(stream)), "forward_prefill")


def ds4moe_forward_timed(mode: int, dims: Dims, weights: Weights, x, T: int, y, routing: Routing | None, ws,
                         ws_bytes: int, events, stream=None) -> None:
    """events: 2*N_TIMED_KERNELS torch.cuda.Event objects (already created) or raw
    hipEvent_t ints; pair i times kernel slot KERNEL_SLOTS[i]."""
    arr = _events(events)
    r = ctypes.byref(routing) if routing is not None else None
    _check(lib().ds4moe_forward_timed(mode, ctypes.byref(dims), ctypes.byref(weights), _ptr(x), T, _ptr(y), r,
                                      _ptr(ws), ws_bytes, arr, _stream(stream)), "forward_timed")


def _events(events):
    if events is None:
        return None
    raw = [e.cuda_event if hasattr(e, "cuda_event") else int(e) for e in events]
    assert len(raw) == 2 * N_TIMED_KERNELS
    return (ctypes.c_void_p * (2 * N_TIMED_KERNELS))(*raw)


def ds4moe_cache_bytes(dims: Dims, n_slots: int) -> int:
    return int(lib().ds4moe_cache_bytes(ctypes.byref(dims), n_slots))


def ds4moe_cache_reset(dims: Dims, n_slots: int, cache, cache_bytes: int, stream=None) -> None:
    _check(lib().ds4moe_cache_reset(ctypes.byref(dims), n_slots, _ptr(cache), cache_bytes, _stream(stream)),
           "cache_reset")


def ds4moe_forward_decode_cached(dims: Dims, weights: Weights, n_slots: int, cache, cache_bytes: int, x, T: int, y,
                                 routing: Routing | None, ws, ws_bytes: int, events=None, stream=None) -> None:
    """weights.gate/up/down: pinned host memory; events: None or 2*N_TIMED_KERNELS events."""
    r = ctypes.byref(routing) if routing is not None else None
    _check(lib().ds4moe_forward_decode_cached(ctypes.byref(dims), ctypes.byref(weights), n_slots, _ptr(cache),
                                              cache_bytes, _ptr(x), T, _ptr(y), r, _ptr(ws), ws_bytes,
                                              _events(events), _stream(stream)), "forward_decode_cached")


def ds4moe_forward_prefill_cached(dims: Dims, weights: Weights, n_slots: int, cache, cache_bytes: int, x, T: int,
                                  y, routing: Routing | None, ws, ws_bytes: int, stream=None) -> None:
    """weights.gate/up/down: pinned host memory; ws: the prefill workspace."""
    r = ctypes.byref(routing) if routing is not None else None
    _check(lib().ds4moe_forward_prefill_cached(ctypes.byref(dims), ctypes.byref(weights), n_slots, _ptr(cache),
                                               cache_bytes, _ptr(x), T, _ptr(y), r, _ptr(ws), ws_bytes,
                                               _stream(stream)), "forward_prefill_cached")


def ds4moe_cache_stats(dims: Dims, n_slots: int, cache, cache_bytes: int, stream=None) -> tuple:
    """(calls, hits, misses) since the cache's reset; synchronises the stream."""
    out = (ctypes.c_uint64 * 3)()
    st = _stream(stream)
    _check(lib().ds4moe_cache_stats(ctypes.byref(dims), n_slots, _ptr(cache), cache_bytes, out, st), "cache_stats")
    torch.cuda.synchronize()
    return int(out[0]), int(out[1]), int(out[2])


def ds4moe_read_probe(buf, nbytes: int, n_workgroups: int, sink, events=None, stream=None) -> None:
    """A plain streaming read of nbytes of `buf` (measurement); events: None or a
    (start, stop) pair of torch.cuda.Event stamped by the kernel's dispatch."""
    ev = (None, None) if events is None else tuple(ctypes.c_void_p(e.cuda_event) for e in events)
    _check(lib().ds4moe_read_probe(_ptr(buf), nbytes, n_workgroups, _ptr(sink), ev[0], ev[1], _stream(stream)),
           "read_probe")
