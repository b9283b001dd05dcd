"""Seeded synthetic inputs for the routed 2-bit MoE layer (inputs only).

Nothing here computes any part of the layer: this module draws Gaussian
tensors with a counter-based generator and quantizes routed-expert weights
into canonical 84-byte super-blocks.  The CPU oracle and the GPU library both
consume what it returns, so neither depends on the other.

Workloads (the five layer shapes the method is measured on):

* ``tiny``     T=16,   H=256,  E=8,   I=128,  k=2, fp32 x N(0,1), fp32 router N(0,0.05)
* ``decode1``  T=1,    H=4096, E=256, I=2048, k=8, bf16 x N(0,1), bf16 router N(0,0.02)
* ``decode16`` T=16,   as decode1, x_t = 0.5*x_s + sqrt(0.75)*z_t (shared component)
* ``prefill``  T=2048, as decode1
* ``skewed``   T=8192, as decode1 plus a Zipf(1.1) router bias and a bf16
  shared expert with intermediate 2048

Routed expert weights are N(0,0.02) before quantization in every workload.
The four H=4096 workloads are one layer (same router and expert weights,
drawn from streams keyed by the layer) fed different activations.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

DEFAULT_SEED = 20261203
BLOCK_BYTES = 84
BLOCK_WEIGHTS = 256

# stream kinds
K_X, K_XSHARED, K_ROUTER, K_BIASPERM, K_GATE, K_UP, K_DOWN, K_SHG, K_SHU, K_SHD = range(1, 11)


def build_lib(force: bool = False) -> str:
    """Compile libsynth.so (plain C, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        cmd = ["gcc", "-O3", "-march=x86-64-v2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
               _SRC, "-o", _LIB_PATH + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        build_lib()
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        L.synth_philox4x32_10.argtypes = [P, P, P]
        L.synth_normal_f32.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_double, ctypes.c_int64, P]
        L.synth_f32_to_bf16.argtypes = [P, ctypes.c_int64, P]
        L.synth_quantize.argtypes = [P, ctypes.c_int64, P]
        L.synth_q2k_matrices.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_int64, ctypes.c_double, P]
        L.synth_qk_matrices.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_double, ctypes.c_int, P]
        L.synth_quantize_bits.argtypes = [P, ctypes.c_int64, ctypes.c_int, P]
        L.synth_u32.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64, P]
        L.synth_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> ctypes.c_void_p:
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


def philox4x32_10(counter, key) -> np.ndarray:
    c = np.asarray(counter, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    out = np.zeros(4, dtype=np.uint32)
    lib().synth_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def stream_id(wl_id: int, kind: int, index: int = 0) -> int:
    assert 0 <= index < (1 << 20) and 0 <= kind < 256 and 0 <= wl_id < 16
    return (wl_id << 28) | (kind << 20) | index


def normal_f32(seed: int, stream: int, sigma: float, shape) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    lib().synth_normal_f32(seed, stream, sigma, n, _ptr(out))
    return out.reshape(shape)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().synth_f32_to_bf16(_ptr(a), a.size, _ptr(out))
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 values."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def block_bytes(bits: int = 2) -> int:
    """Bytes of one canonical block of 256 weights with 2- or 4-bit codes."""
    assert bits in (2, 4, 5, 6)
    return 16 + 32 * bits + 4


def quantize_blocks(w: np.ndarray, bits: int = 2) -> np.ndarray:
    """RTN-quantize fp32 weights (size multiple of 256, row-major) to canonical blocks."""
    w = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
    assert w.size % BLOCK_WEIGHTS == 0
    nb = w.size // BLOCK_WEIGHTS
    out = np.empty(nb * block_bytes(bits), dtype=np.uint8)
    lib().synth_quantize_bits(_ptr(w), nb, bits, _ptr(out))
    return out


def qk_matrices(seed: int, stream_base: int, n_mats: int, rows: int, cols: int, sigma: float,
                bits: int = 2) -> np.ndarray:
    """n_mats matrices [rows, cols] of N(0,sigma) weights quantized to canonical
    blocks with `bits`-bit codes.

    Returns uint8 [n_mats, rows*cols/256*block_bytes(bits)]; matrix e is stream stream_base+e.
    """
    assert (rows * cols) % BLOCK_WEIGHTS == 0
    per = rows * cols // BLOCK_WEIGHTS * block_bytes(bits)
    out = np.empty((n_mats, per), dtype=np.uint8)
    lib().synth_qk_matrices(seed, stream_base, n_mats, rows, cols, sigma, bits, _ptr(out))
    return out


def q2k_matrices(seed: int, stream_base: int, n_mats: int, rows: int, cols: int, sigma: float) -> np.ndarray:
    """2-bit blocks (84 bytes per 256 weights); see qk_matrices."""
    return qk_matrices(seed, stream_base, n_mats, rows, cols, sigma, 2)


def u32(seed: int, stream: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.uint32)
    lib().synth_u32(seed, stream, n, _ptr(out))
    return out


def num_threads() -> int:
    return int(lib().synth_num_threads())


@dataclass(frozen=True)
class Workload:
    name: str
    wl_id: int
    T: int
    H: int
    E: int
    I: int
    k: int
    Is: int = 0
    x_dtype: str = "bf16"          # "f32" or "bf16"
    router_dtype: str = "bf16"
    router_sigma: float = 0.02
    w_sigma: float = 0.02
    x_shared_rho: float = 0.0      # x_t = rho*x_s + sqrt(1-rho^2)*z_t
    zipf_s: float = 0.0            # router bias from a Zipf(s) law, 0 = no bias
    zipf_scale: float = 0.75
    layer_id: int = 1              # weight streams: workloads of one shape share a layer
    description: str = ""
    bits: int = 2                  # routed-expert code width: 2, 4, 5 or 6 (84-, 148-, 180-, 212-byte blocks)
    bits_down: int = 0             # code width of the down matrices (0: the same as `bits`)

    @property
    def down_width(self) -> int:
        return self.bits_down or self.bits


WORKLOADS = {
    "tiny": Workload("tiny", 0, T=16, H=256, E=8, I=128, k=2, x_dtype="f32", router_dtype="f32",
                     router_sigma=0.05, layer_id=0, description="tiny layer, fp32 activations and router"),
    "decode1": Workload("decode1", 1, T=1, H=4096, E=256, I=2048, k=8,
                        description="decode, one token"),
    "decode16": Workload("decode16", 2, T=16, H=4096, E=256, I=2048, k=8, x_shared_rho=0.5,
                         description="decode micro-batch of 16 correlated tokens"),
    "prefill": Workload("prefill", 3, T=2048, H=4096, E=256, I=2048, k=8,
                        description="prefill chunk of 2048 tokens"),
    "skewed": Workload("skewed", 4, T=8192, H=4096, E=256, I=2048, k=8, Is=2048, zipf_s=1.1,
                       description="long prefill, Zipf-skewed routing, bf16 shared expert"),
    # the same decode and prefill shapes with 4-bit routed experts (own layer)
    "decode1_q4": Workload("decode1_q4", 5, T=1, H=4096, E=256, I=2048, k=8, layer_id=2, bits=4,
                           description="decode, one token, 4-bit routed experts"),
    "prefill_q4": Workload("prefill_q4", 6, T=2048, H=4096, E=256, I=2048, k=8, layer_id=2, bits=4,
                           description="prefill chunk of 2048 tokens, 4-bit routed experts"),
    # gate/up with 2-bit codes, down with 4-bit codes (own layer)
    "decode1_mix": Workload("decode1_mix", 7, T=1, H=4096, E=256, I=2048, k=8, layer_id=3, bits=2, bits_down=4,
                            description="decode, one token, 2-bit gate/up and 4-bit down"),
    "prefill_mix": Workload("prefill_mix", 8, T=2048, H=4096, E=256, I=2048, k=8, layer_id=3, bits=2, bits_down=4,
                            description="prefill chunk of 2048 tokens, 2-bit gate/up and 4-bit down"),
    # gate/up with 5-bit codes, down with 6-bit codes, the pages' GLM pairing (own layer)
    "decode1_q56": Workload("decode1_q56", 9, T=1, H=4096, E=256, I=2048, k=8, layer_id=4, bits=5, bits_down=6,
                            description="decode, one token, 5-bit gate/up and 6-bit down"),
    "prefill_q56": Workload("prefill_q56", 10, T=2048, H=4096, E=256, I=2048, k=8, layer_id=4, bits=5, bits_down=6,
                            description="prefill chunk of 2048 tokens, 5-bit gate/up and 6-bit down"),
}


@dataclass
class LayerInputs:
    wl: Workload
    seed: int
    T: int
    x: np.ndarray              # fp32 [T,H] (tiny) or bf16 bits uint16 [T,H]
    router_w: np.ndarray       # fp32 [E,H] or bf16 bits [E,H]
    router_bias: np.ndarray | None  # fp32 [E]
    gate: np.ndarray           # uint8 [E, I*H/256*84] canonical blocks, W[I,H] row-major
    up: np.ndarray             # uint8 [E, I*H/256*84]
    down: np.ndarray           # uint8 [E, H*I/256*84], W[H,I] row-major
    sh_gate: np.ndarray | None = None  # bf16 bits [Is,H]
    sh_up: np.ndarray | None = None    # bf16 bits [Is,H]
    sh_down: np.ndarray | None = None  # bf16 bits [H,Is]
    extra: dict = field(default_factory=dict)

    def x_f32(self) -> np.ndarray:
        return self.x if self.wl.x_dtype == "f32" else bf16_bits_to_f32(self.x)

    def router_f32(self) -> np.ndarray:
        return self.router_w if self.wl.router_dtype == "f32" else bf16_bits_to_f32(self.router_w)


def make_x(wl: Workload, seed: int, T: int, batch: int = 0) -> np.ndarray:
    """Activations for batch number `batch` (fresh tokens per batch)."""
    z = normal_f32(seed, stream_id(wl.wl_id, K_X, batch), 1.0, (T, wl.H))
    if wl.x_shared_rho:
        xs = normal_f32(seed, stream_id(wl.wl_id, K_XSHARED, batch), 1.0, (1, wl.H))
        rho = wl.x_shared_rho
        z = (rho * xs.astype(np.float64) + math.sqrt(1.0 - rho * rho) * z.astype(np.float64)).astype(np.float32)
    return z if wl.x_dtype == "f32" else f32_to_bf16_bits(z)


def zipf_bias(wl: Workload, seed: int) -> np.ndarray:
    """b_e = scale*(ln p_r(e) - mean ln p), p_r ~ r^-s, ranks r assigned by a seeded permutation."""
    E = wl.E
    r = u32(seed, stream_id(wl.wl_id, K_BIASPERM), E)
    perm = list(range(E))
    for i in range(E - 1, 0, -1):  # Fisher-Yates driven by the stream
        j = int(r[i]) % (i + 1)
        perm[i], perm[j] = perm[j], perm[i]
    ranks = np.array(perm, dtype=np.float64) + 1.0   # expert e has rank perm[e]+1
    lnp = -wl.zipf_s * np.log(ranks)
    return (wl.zipf_scale * (lnp - lnp.mean())).astype(np.float32)


def make_layer(wl: Workload | str, seed: int = DEFAULT_SEED, T: int | None = None,
               experts: bool = True) -> LayerInputs:
    """All inputs of one layer.  `T` overrides the workload's token count."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    T = wl.T if T is None else T
    E, H, I = wl.E, wl.H, wl.I
    x = make_x(wl, seed, T)
    lid = wl.layer_id
    rw = normal_f32(seed, stream_id(lid, K_ROUTER), wl.router_sigma, (E, H))
    if wl.router_dtype == "bf16":
        rw = f32_to_bf16_bits(rw)
    bias = zipf_bias(wl, seed) if wl.zipf_s else None
    if experts:
        gate = qk_matrices(seed, stream_id(lid, K_GATE), E, I, H, wl.w_sigma, wl.bits)
        up = qk_matrices(seed, stream_id(lid, K_UP), E, I, H, wl.w_sigma, wl.bits)
        down = qk_matrices(seed, stream_id(lid, K_DOWN), E, H, I, wl.w_sigma, wl.down_width)
    else:
        gate = up = down = None
    shg = shu = shd = None
    if wl.Is:
        shg = f32_to_bf16_bits(normal_f32(seed, stream_id(lid, K_SHG), wl.w_sigma, (wl.Is, H)))
        shu = f32_to_bf16_bits(normal_f32(seed, stream_id(lid, K_SHU), wl.w_sigma, (wl.Is, H)))
        shd = f32_to_bf16_bits(normal_f32(seed, stream_id(lid, K_SHD), wl.w_sigma, (H, wl.Is)))
    return LayerInputs(wl, seed, T, x, rw, bias, gate, up, down, shg, shu, shd)


def derive(base: LayerInputs, wl: Workload | str, T: int | None = None, batch: int = 0) -> LayerInputs:
    """Inputs of workload `wl` reusing `base`'s router and expert weights (the
    workloads of one shape share a layer); x, bias and shared expert follow
    `wl`'s recipe."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    b = base.wl
    assert (wl.H, wl.E, wl.I, wl.layer_id, wl.bits, wl.down_width) == (b.H, b.E, b.I, b.layer_id, b.bits,
                                                                       b.down_width)
    T = wl.T if T is None else T
    shared = make_layer(wl, base.seed, T=1, experts=False) if (wl.Is or wl.zipf_s) else None
    return LayerInputs(wl, base.seed, T, make_x(wl, base.seed, T, batch), base.router_w,
                       shared.router_bias if shared is not None else None, base.gate, base.up, base.down,
                       shared.sh_gate if shared is not None else None, shared.sh_up if shared is not None else None,
                       shared.sh_down if shared is not None else None)
