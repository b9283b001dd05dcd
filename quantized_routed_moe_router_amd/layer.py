"""Device-resident layer: packed expert weights in HBM plus a reusable workspace.

Plumbing around the C ABI only: torch allocates device memory; packing,
routing and the expert FFNs all run in libds4moe.so.
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B


def _dev(a: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def _as_bf16(bits: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


class DeviceLayer:
    def __init__(self, H, I, E, k, Is=0, x_dtype=B.DS4MOE_BF16, router_dtype=B.DS4MOE_BF16, device="cuda:0",
                 bits=2, down_bits=0):
        self.H, self.I, self.E, self.k, self.Is, self.bits = H, I, E, k, Is, bits
        self.down_bits = down_bits or bits
        self.device = torch.device(device)
        self.dims = B.make_dims(H, I, E, k, Is, x_dtype, router_dtype, bits, down_bits)
        self.x_dtype, self.router_dtype = x_dtype, router_dtype
        self.gu_bytes = B.ds4moe_packed_bytes_bits(I, H, bits)
        self.d_bytes = B.ds4moe_packed_bytes_bits(H, I, self.down_bits)
        self._ws = None
        self.router_w = self.router_bias = None
        self.gate = self.up = self.down = None
        self.sh_gate = self.sh_up = self.sh_down = None

    # ------------------------------------------------------------ weights
    def pack(self, canonical: np.ndarray, rows: int, cols: int, stream=None, bits=None) -> torch.Tensor:
        """Upload E canonical-block matrices and repack them on the GPU."""
        bits = self.bits if bits is None else bits
        n = canonical.shape[0]
        src = _dev(canonical.reshape(n, -1), self.device)
        dst = torch.empty(n * B.ds4moe_packed_bytes_bits(rows, cols, bits), dtype=torch.uint8,
                          device=self.device)
        B.ds4moe_pack(dst, src, n, rows, cols, bits, stream)
        torch.cuda.current_stream(self.device).synchronize()
        del src
        return dst

    def set_router(self, router_w: np.ndarray, router_bias: np.ndarray | None = None):
        if self.router_dtype == B.DS4MOE_BF16:
            self.router_w = _as_bf16(router_w, self.device)
        else:
            self.router_w = _dev(router_w.astype(np.float32), self.device)
        self.router_bias = None if router_bias is None else _dev(router_bias.astype(np.float32), self.device)

    def set_experts(self, gate: np.ndarray, up: np.ndarray, down: np.ndarray):
        self.gate = self.pack(gate, self.I, self.H)
        self.up = self.pack(up, self.I, self.H)
        self.down = self.pack(down, self.H, self.I, bits=self.down_bits)

    def set_shared(self, sh_gate, sh_up, sh_down):
        self.sh_gate = _as_bf16(sh_gate, self.device)
        self.sh_up = _as_bf16(sh_up, self.device)
        self.sh_down = _as_bf16(sh_down, self.device)

    def weights(self, gate=None, up=None, down=None) -> B.Weights:
        return B.make_weights(self.router_w, gate if gate is not None else self.gate,
                              up if up is not None else self.up, down if down is not None else self.down,
                              self.router_bias, self.sh_gate, self.sh_up, self.sh_down)

    # ------------------------------------------------------------ activations
    def x_tensor(self, x: np.ndarray) -> torch.Tensor:
        if self.x_dtype == B.DS4MOE_BF16:
            return _as_bf16(x, self.device)
        return _dev(x.astype(np.float32), self.device)

    def workspace(self, T: int, mode: int) -> torch.Tensor:
        need = B.ds4moe_workspace_bytes(self.dims, T, mode)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)
        return self._ws

    def routing_buffers(self, T: int) -> dict:
        d = self.device
        return dict(topk_idx=torch.empty(T, self.k, dtype=torch.int32, device=d),
                    topk_w=torch.empty(T, self.k, dtype=torch.float32, device=d),
                    counts=torch.empty(self.E, dtype=torch.int32, device=d),
                    offsets=torch.empty(self.E + 1, dtype=torch.int32, device=d),
                    perm=torch.empty(T * self.k, dtype=torch.int32, device=d),
                    logits=torch.empty(T, self.E, dtype=torch.float32, device=d))

    def forward(self, x: torch.Tensor, mode: int = B.MODE_PREFILL, y=None, routing: dict | None = None,
                stream=None, weights: B.Weights | None = None) -> torch.Tensor:
        T = x.shape[0]
        if y is None:
            y = torch.empty(T, self.H, dtype=torch.float32, device=self.device)
        ws = self.workspace(T, mode)
        r = B.make_routing(**routing) if routing is not None else None
        w = weights if weights is not None else self.weights()
        fn = B.ds4moe_forward_decode if mode == B.MODE_DECODE else B.ds4moe_forward_prefill
        fn(self.dims, w, x, T, y, r, ws, ws.numel(), stream)
        return y

    def host_experts(self) -> tuple:
        """Pinned host copies of the packed gate, up and down matrices."""
        out = []
        for t in (self.gate, self.up, self.down):
            h = torch.empty(t.numel(), dtype=torch.uint8, pin_memory=True)
            h.copy_(t)
            out.append(h)
        return tuple(out)

    def route(self, x: torch.Tensor, stream=None) -> dict:
        T = x.shape[0]
        bufs = self.routing_buffers(T)
        ws = self.workspace(T, B.MODE_ROUTE)
        B.ds4moe_route(self.dims, self.weights(), x, T, B.make_routing(**bufs), ws, ws.numel(), stream)
        return bufs


def from_layer_inputs(L, device="cuda:0", experts: bool = True) -> DeviceLayer:
    """Build a DeviceLayer from a synth.LayerInputs-like object (duck-typed)."""
    wl = L.wl
    xd = B.DS4MOE_F32 if wl.x_dtype == "f32" else B.DS4MOE_BF16
    rd = B.DS4MOE_F32 if wl.router_dtype == "f32" else B.DS4MOE_BF16
    dl = DeviceLayer(wl.H, wl.I, wl.E, wl.k, wl.Is, xd, rd, device, bits=getattr(wl, "bits", 2),
                     down_bits=getattr(wl, "bits_down", 0))
    dl.set_router(L.router_w, L.router_bias)
    if experts:
        dl.set_experts(L.gate, L.up, L.down)
    if wl.Is:
        dl.set_shared(L.sh_gate, L.sh_up, L.sh_down)
    return dl


class ExpertCache:
    """A bounded routed-expert cache in device memory over experts kept in
    pinned host memory.  `host`: (gate, up, down) pinned uint8 tensors in the
    packed layout, by default copies of `dl`'s.  forward: small batches
    (decode); forward_prefill: any batch, the used experts streamed through
    the slots in batches."""

    def __init__(self, dl: DeviceLayer, n_slots: int, host: tuple | None = None, stream=None):
        self.dl, self.n_slots = dl, n_slots
        self.host = host if host is not None else dl.host_experts()
        self.nbytes = B.ds4moe_cache_bytes(dl.dims, n_slots)
        if self.nbytes == 0:
            raise ValueError(f"invalid cache size: {n_slots} slots")
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device=dl.device)
        self.reset(stream)

    def reset(self, stream=None):
        B.ds4moe_cache_reset(self.dl.dims, self.n_slots, self.buf, self.nbytes, stream)

    def weights(self) -> B.Weights:
        return self.dl.weights(*self.host)

    def forward(self, x: torch.Tensor, y=None, routing: dict | None = None, stream=None, events=None,
                weights: B.Weights | None = None) -> torch.Tensor:
        dl = self.dl
        T = x.shape[0]
        if y is None:
            y = torch.empty(T, dl.H, dtype=torch.float32, device=dl.device)
        ws = dl.workspace(T, B.MODE_DECODE)
        r = B.make_routing(**routing) if routing is not None else None
        w = weights if weights is not None else self.weights()
        B.ds4moe_forward_decode_cached(dl.dims, w, self.n_slots, self.buf, self.nbytes, x, T, y, r, ws, ws.numel(),
                                       events, stream)
        return y

    def forward_prefill(self, x: torch.Tensor, y=None, routing: dict | None = None, stream=None,
                        weights: B.Weights | None = None) -> torch.Tensor:
        dl = self.dl
        T = x.shape[0]
        if y is None:
            y = torch.empty(T, dl.H, dtype=torch.float32, device=dl.device)
        ws = dl.workspace(T, B.MODE_PREFILL)
        r = B.make_routing(**routing) if routing is not None else None
        w = weights if weights is not None else self.weights()
        B.ds4moe_forward_prefill_cached(dl.dims, w, self.n_slots, self.buf, self.nbytes, x, T, y, r, ws, ws.numel(),
                                        stream)
        return y

    def stats(self, stream=None) -> tuple:
        return B.ds4moe_cache_stats(self.dl.dims, self.n_slots, self.buf, self.nbytes, stream)
