"""GPU parity of the layer with 4-bit routed experts (148-byte super-blocks:
the 2-bit block with 4-bit codes) against the oracle, through the C ABI.

Same bars as the 2-bit layer: pack + dequant bit-exact, routing bit-exact,
y within 2e-3 per-token normwise relative error.  The cases reach every
expert kernel at both code widths' shared templates: decode with T <= 4
(routing inside gate/up, activations through LDS) and T > 4, the padded
down projection (I = 128), prefill on the 64-token GEMMs (I = 128) and on
the 96-token wide-tile GEMMs (I a multiple of 256), and the full-size
decode and prefill workloads.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth

from test_gpu_parity import TOL_Y, check_routing, per_token_err

pytestmark = pytest.mark.gpu


def _q():
    import quantized_routed_moe_router_amd as q
    return q


def _wl(name, T, H, I, E=8, k=2, Is=0):
    return synth.Workload(name, 0, T=T, H=H, E=E, I=I, k=k, Is=Is, x_dtype="f32", router_dtype="f32",
                          router_sigma=0.05, layer_id=0, bits=4)


def _run(L, mode, dl=None):
    q = _q()
    dl = dl if dl is not None else q.from_layer_inputs(L)
    assert dl.bits == 4
    bufs = dl.routing_buffers(L.T)
    m = q.MODE_DECODE if mode == "decode" else q.MODE_PREFILL
    y = dl.forward(dl.x_tensor(L.x), m, routing=bufs)
    torch.cuda.synchronize()
    check_routing(bufs, L, label=f"{L.wl.name} {mode} T={L.T}")
    return y, bufs, dl


def _check_all_tokens(L, y, label):
    ref, _, _ = oracle.layer_inputs(L)
    err = per_token_err(y.cpu().numpy(), ref)
    print(f"{label}: per-token rel err {err:.3e}")
    assert err <= TOL_Y


# ------------------------------------------------------------------ pack / dequant


@pytest.mark.parametrize("rows,cols", [(16, 256), (48, 512), (32, 4096), (256, 128), (64, 64), (16, 16)])
def test_q4_dequant_bitwise(rows, cols):
    q = _q()
    dev = torch.device("cuda:0")
    n = 3
    canon = synth.qk_matrices(7, 9100 + rows + cols, n, rows, cols, 0.02, bits=4)
    src = torch.from_numpy(canon).to(dev)
    nb = q.ds4moe_packed_bytes_bits(rows, cols, 4)
    packed = torch.empty(n * nb, dtype=torch.uint8, device=dev)
    q.ds4moe_pack(packed, src, n, rows, cols, 4)
    out = torch.empty(n, rows, cols, dtype=torch.float32, device=dev)
    q.ds4moe_dequant(out, packed, n, rows, cols, 4)
    torch.cuda.synchronize()
    ref = oracle.dequant_f32(canon, bits=4).reshape(n, rows, cols)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_q4_dequant_special_blocks():
    """Hand-built 4-bit blocks (subnormal and negative d, zero block, largest
    finite d and dmin, every code 15) survive pack + dequant bit for bit."""
    q = _q()
    rng = np.random.default_rng(15)
    blk = np.zeros((16, 148), np.uint8)
    blk[:, :144] = rng.integers(0, 256, size=(16, 144))
    blk[0, 144:148] = [0x01, 0x00, 0x00, 0x00]          # subnormal d, zero dmin
    blk[1, 144:148] = [0x00, 0xBC, 0x00, 0x38]          # d = -1, dmin = 0.5
    blk[2, :] = 0                                       # all-zero block
    blk[3, 144:148] = [0xFF, 0x7B, 0xFF, 0x7B]          # largest finite d, dmin
    blk[4, 16:144] = 0xFF                               # every code 15
    canon = blk.reshape(1, -1)
    dev = torch.device("cuda:0")
    packed = torch.empty(q.ds4moe_packed_bytes_bits(16, 256, 4), dtype=torch.uint8, device=dev)
    q.ds4moe_pack(packed, torch.from_numpy(canon).to(dev), 1, 16, 256, 4)
    out = torch.empty(16, 256, dtype=torch.float32, device=dev)
    q.ds4moe_dequant(out, packed, 1, 16, 256, 4)
    ref = oracle.dequant_f32(canon, bits=4).reshape(16, 256)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_pack_bits2_is_pack_q2k():
    """The width-generic entry points with bits = 2 are the 2-bit ones."""
    q = _q()
    dev = torch.device("cuda:0")
    canon = synth.qk_matrices(7, 9300, 2, 48, 512, 0.02, bits=2)
    src = torch.from_numpy(canon).to(dev)
    nb = q.ds4moe_packed_bytes_bits(48, 512, 2)
    assert nb == q.ds4moe_packed_bytes(48, 512)
    a = torch.empty(2 * nb, dtype=torch.uint8, device=dev)
    b = torch.empty(2 * nb, dtype=torch.uint8, device=dev)
    q.ds4moe_pack(a, src, 2, 48, 512, 2)
    q.ds4moe_pack_q2k(b, src, 2, 48, 512)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ------------------------------------------------------------------ small layers


@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 9, 16])
def test_q4_tiny_decode(T):
    """I = 128 (padded down projection), every decode batch-size class."""
    L = synth.make_layer(_wl("tiny_q4", T, 256, 128))
    y, _, _ = _run(L, "decode")
    _check_all_tokens(L, y, f"q4 tiny decode T={T}")


@pytest.mark.parametrize("T", [1, 17, 65, 257])
def test_q4_tiny_prefill(T):
    """I = 128: the 64-token GEMMs, padded down projection."""
    L = synth.make_layer(_wl("tiny_q4", T, 256, 128))
    y, _, _ = _run(L, "prefill")
    _check_all_tokens(L, y, f"q4 tiny prefill T={T}")


@pytest.mark.parametrize("T", [1, 4, 8, 16])
def test_q4_mid_decode(T):
    """I = 256: the LDS-ring decode kernels (T <= 4) and the register ones."""
    L = synth.make_layer(_wl("mid_q4", T, 512, 256))
    y, _, _ = _run(L, "decode")
    _check_all_tokens(L, y, f"q4 mid decode T={T}")


@pytest.mark.parametrize("T", [1, 48, 97, 300, 1000])
def test_q4_mid_prefill_wide(T):
    """I = 256: 96-token wide tiles, partial n-tiles and ragged last tiles."""
    L = synth.make_layer(_wl("mid_q4", T, 512, 256))
    y, _, _ = _run(L, "prefill")
    _check_all_tokens(L, y, f"q4 mid prefill T={T}")


def test_q4_mid_shared_expert():
    """4-bit routed experts beside a bf16 shared expert."""
    wl = dataclasses.replace(_wl("mid_q4_sh", 200, 512, 256, Is=96), x_dtype="bf16", router_dtype="bf16")
    L = synth.make_layer(wl)
    y, _, _ = _run(L, "prefill")
    _check_all_tokens(L, y, "q4 mid shared T=200")


def test_q4_one_expert_all_tokens():
    """Every token's first choice is expert 5 (tiles 96, 96, 96, 12)."""
    q = _q()
    L = synth.make_layer(_wl("mid_q4", 300, 512, 256))
    bias = np.zeros(L.wl.E, np.float32)
    bias[5] = 100.0
    L.router_bias = bias
    dl = q.from_layer_inputs(L)
    y, bufs, _ = _run(L, "prefill", dl)
    assert np.all(bufs["topk_idx"].cpu().numpy()[:, 0] == 5)
    _check_all_tokens(L, y, "q4 one expert")


# ------------------------------------------------------------------ full size


@pytest.fixture(scope="session")
def full4():
    q = _q()
    L = synth.make_layer("prefill_q4")
    return L, q.from_layer_inputs(L)


def test_q4_full_dequant_sample(full4):
    q = _q()
    L, dl = full4
    H, I = L.wl.H, L.wl.I
    for e in (0, 131, 255):
        for packed, canon, rows, cols, nb in ((dl.up, L.up, I, H, dl.gu_bytes), (dl.down, L.down, H, I, dl.d_bytes)):
            out = torch.empty(rows, cols, dtype=torch.float32, device=dl.device)
            q.ds4moe_dequant(out, packed[e * nb:(e + 1) * nb], 1, rows, cols, 4)
            ref = oracle.dequant_f32(canon[e], bits=4).reshape(rows, cols)
            assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32)), (e, rows)


def test_q4_full_decode1(full4):
    L0, dl = full4
    L = synth.derive(L0, "decode1_q4")
    y, _, _ = _run(L, "decode", dl)
    _check_all_tokens(L, y, "q4 decode1")


@pytest.mark.parametrize("T", [4, 16])
def test_q4_full_decode_batches(full4, T):
    L0, dl = full4
    L = synth.derive(L0, "decode1_q4", T=T)
    y, _, _ = _run(L, "decode", dl)
    _check_all_tokens(L, y, f"q4 decode T={T}")


def test_q4_full_prefill_all_tokens(full4):
    """The 2048-token prefill chunk on 4-bit experts, every token."""
    L0, dl = full4
    L = synth.derive(L0, "prefill_q4")
    y, bufs, _ = _run(L, "prefill", dl)
    idx = bufs["topk_idx"].cpu().numpy()
    ref, ridx, _ = oracle.layer_inputs(L)
    assert np.array_equal(ridx, idx)
    err = per_token_err(y.cpu().numpy(), ref)
    print(f"q4 prefill: all {L.T} tokens checked, per-token rel err {err:.3e}")
    assert err <= TOL_Y
