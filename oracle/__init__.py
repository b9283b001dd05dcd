"""CPU oracle for the routed 2-bit MoE layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never calls it and
shares no code with it; its arithmetic is plain fp64 C in ``oracle.c``.

Every function here only marshals numpy arrays into ``liboracle.so``.
Pins (tests that fix the oracle to something other than itself) live in
``tests/test_oracle_pins.py``.  Parity status of each function:

* dequant        pinned (hand-built blocks, exactness brute force, closed form)
* logits         pinned (exact rational recomputation, float64 library matmul)
* score          pinned (high-precision closed forms at chosen logits)
* topk/weights   pinned (brute force over all subsets, invariants, special cases)
* permute        pinned (brute-force sort, invariants)
* layer          pinned (E=1,k=1 equals a library dense SwiGLU FFN; constant-block
                 closed form; zero weights; token independence; shared-expert-only case)
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build_lib(force: bool = False) -> str:
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        cmd = ["gcc", "-O3", "-march=x86-64-v3", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", _SRC,
               "-o", _LIB_PATH + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        build_lib()
        L = ctypes.CDLL(_LIB_PATH)
        P, I64 = ctypes.c_void_p, ctypes.c_int64
        L.oracle_dequant_f64.argtypes = [P, I64, P]
        L.oracle_dequant_f32.argtypes = [P, I64, P]
        L.oracle_logits.argtypes = [P, P, P, I64, I64, I64, P]
        L.oracle_score.argtypes = [ctypes.c_double]
        L.oracle_score.restype = ctypes.c_double
        L.oracle_scores.argtypes = [P, I64, P]
        L.oracle_topk.argtypes = [P, I64, I64, I64, P, P, P]
        L.oracle_permute.argtypes = [P, I64, I64, I64, P, P, P]
        L.oracle_layer.argtypes = [P, I64, I64, I64, I64, I64, P, P, P, P, P, I64, P, P, P, P, P, P]
        L.oracle_dequant_f64_bits.argtypes = [P, I64, ctypes.c_int, P]
        L.oracle_dequant_f32_bits.argtypes = [P, I64, ctypes.c_int, P]
        L.oracle_layer_bits.argtypes = [P, I64, I64, I64, I64, I64, P, P, P, P, P, ctypes.c_int, I64, P, P, P, P,
                                        P, P]
        L.oracle_layer_bits2.argtypes = [P, I64, I64, I64, I64, I64, P, P, P, P, P, ctypes.c_int, ctypes.c_int, I64,
                                         P, P, P, P, P, P]
        L.oracle_layer_bits2.restype = ctypes.c_int
        L.oracle_layer.restype = ctypes.c_int
        L.oracle_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a):
    return ctypes.c_void_p(0) if a is None else ctypes.c_void_p(a.ctypes.data)


def block_bytes(bits: int = 2) -> int:
    """Bytes of one block of 256 weights with 2-, 4-, 5- or 6-bit codes."""
    assert bits in (2, 4, 5, 6)
    return 16 + 32 * bits + 4


def dequant_f64(blocks: np.ndarray, bits: int = 2) -> np.ndarray:
    b = _c(blocks, np.uint8).reshape(-1)
    nb = b.size // block_bytes(bits)
    out = np.empty(nb * 256, dtype=np.float64)
    lib().oracle_dequant_f64_bits(_p(b), nb, bits, _p(out))
    return out


def dequant_f32(blocks: np.ndarray, bits: int = 2) -> np.ndarray:
    b = _c(blocks, np.uint8).reshape(-1)
    nb = b.size // block_bytes(bits)
    out = np.empty(nb * 256, dtype=np.float32)
    lib().oracle_dequant_f32_bits(_p(b), nb, bits, _p(out))
    return out


def logits(x: np.ndarray, wr: np.ndarray, bias: np.ndarray | None = None) -> np.ndarray:
    x = _c(x, np.float32)
    wr = _c(wr, np.float32)
    T, H = x.shape
    E = wr.shape[0]
    b = None if bias is None else _c(bias, np.float32)
    out = np.empty((T, E), dtype=np.float32)
    lib().oracle_logits(_p(x), _p(wr), _p(b), T, E, H, _p(out))
    return out


def score(l: float) -> float:
    return float(lib().oracle_score(float(l)))


def scores(lg: np.ndarray) -> np.ndarray:
    lg = _c(lg, np.float32)
    out = np.empty(lg.shape, dtype=np.float64)
    lib().oracle_scores(_p(lg), lg.size, _p(out))
    return out


def topk(lg: np.ndarray, k: int):
    """Returns (idx int32 [T,k], w fp32 [T,k], w in float64 [T,k])."""
    lg = _c(lg, np.float32)
    T, E = lg.shape
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    wd = np.empty((T, k), dtype=np.float64)
    lib().oracle_topk(_p(lg), T, E, k, _p(idx), _p(w), _p(wd))
    return idx, w, wd


def permute(idx: np.ndarray, E: int):
    """Returns (counts [E], offsets [E+1], perm [T*k]) as int32."""
    idx = _c(idx, np.int32)
    T, k = idx.shape
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    perm = np.empty(T * k, dtype=np.int32)
    lib().oracle_permute(_p(idx), T, k, E, _p(counts), _p(offsets), _p(perm))
    return counts, offsets, perm


def layer(x, wr, bias, gate, up, down, H, I, E, k, sh_gate=None, sh_up=None, sh_down=None, bits=2, down_bits=None):
    """Whole layer.  x [T,H] and wr [E,H] as fp32 values; gate/up/down canonical
    blocks [E, nbytes] (gate/up with `bits`-bit codes, down with `down_bits`,
    default the same); shared weights as fp32 values or None.
    Returns (y fp32 [T,H], idx int32 [T,k], w fp32 [T,k])."""
    x = _c(x, np.float32).reshape(-1, H)
    T = x.shape[0]
    wr = _c(wr, np.float32)
    b = None if bias is None else _c(bias, np.float32)
    g, u, d = _c(gate, np.uint8), _c(up, np.uint8), _c(down, np.uint8)
    Is = 0
    sg = su = sd = None
    if sh_gate is not None:
        sg, su, sd = _c(sh_gate, np.float32), _c(sh_up, np.float32), _c(sh_down, np.float32)
        Is = sg.shape[0]
    y = np.empty((T, H), dtype=np.float32)
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float32)
    rc = lib().oracle_layer_bits2(_p(x), T, H, I, E, k, _p(wr), _p(b), _p(g), _p(u), _p(d), bits,
                                  bits if down_bits is None else down_bits, Is, _p(sg), _p(su), _p(sd), _p(y),
                                  _p(idx), _p(w))
    if rc != 0:
        raise MemoryError("oracle_layer failed to allocate")
    return y, idx, w


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to fp32 values."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def layer_inputs(L, tokens=None):
    """Run the oracle on a synth.LayerInputs, optionally on a subset of tokens."""
    x = L.x if L.wl.x_dtype == "f32" else bf16_to_f32(L.x)
    wr = L.router_w if L.wl.router_dtype == "f32" else bf16_to_f32(L.router_w)
    if tokens is not None:
        x = x[np.asarray(tokens)]
    wl = L.wl
    sh = (None, None, None)
    if L.sh_gate is not None:
        sh = (bf16_to_f32(L.sh_gate), bf16_to_f32(L.sh_up), bf16_to_f32(L.sh_down))
    return layer(x, wr, L.router_bias, L.gate, L.up, L.down, wl.H, wl.I, wl.E, wl.k, *sh, bits=wl.bits,
                 down_bits=getattr(wl, "bits_down", 0) or wl.bits)


def num_threads() -> int:
    return int(lib().oracle_num_threads())
