"""GPU parity of the layer with 5- and 6-bit routed experts (the 2-bit
super-block with 5- or 6-bit codes; both packed into the 6-bit unit) against
the oracle, through the C ABI.

Same bars as the 2-bit layer: pack + dequant bit-exact, routing bit-exact,
y within 2e-3 per-token normwise relative error.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

from test_gpu_parity import TOL_Y, check_routing, per_token_err
from test_oracle_pins_q56 import make_block_b, nbytes

pytestmark = pytest.mark.gpu

WIDTHS = (5, 6)


def _q():
    import quantized_routed_moe_router_amd as q
    return q


def _pack_dequant(canon, n, rows, cols, b):
    q = _q()
    dev = torch.device("cuda:0")
    src = torch.from_numpy(np.ascontiguousarray(canon)).to(dev)
    nb = q.ds4moe_packed_bytes_bits(rows, cols, b)
    packed = torch.empty(n * nb, dtype=torch.uint8, device=dev)
    q.ds4moe_pack(packed, src, n, rows, cols, b)
    out = torch.empty(n, rows, cols, dtype=torch.float32, device=dev)
    q.ds4moe_dequant(out, packed, n, rows, cols, b)
    torch.cuda.synchronize()
    return out.cpu().numpy()


# ------------------------------------------------------------------ pack / dequant


@pytest.mark.parametrize("b", WIDTHS)
@pytest.mark.parametrize("rows,cols", [(16, 256), (48, 512), (32, 4096), (256, 128), (64, 64), (16, 16)])
def test_dequant_bitwise(b, rows, cols):
    n = 3
    canon = synth.qk_matrices(7, 9300 + 10 * b + rows + cols, n, rows, cols, 0.02, bits=b)
    out = _pack_dequant(canon, n, rows, cols, b)
    ref = oracle.dequant_f32(canon, bits=b).reshape(n, rows, cols)
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("b", WIDTHS)
def test_dequant_special_blocks(b):
    """Hand-built blocks (every code at its top value, alternating codes,
    subnormal and negative d, the largest finite d and dmin, a zero block)
    survive pack + dequant bit for bit."""
    rng = np.random.default_rng(35 + b)
    top = (1 << b) - 1
    blocks = []
    for hb_d, hb_m, codes in [(0x0001, 0x0000, np.full(256, top)), (0xBC00, 0x3800, np.full(256, top)),
                              (0x7BFF, 0x7BFF, np.arange(256) % (1 << b)), (0x0000, 0x0000, np.zeros(256)),
                              (0x3555, 0x2AAA, np.where(np.arange(256) % 2 == 0, top, 0))]:
        scales = rng.integers(0, 256, 16, dtype=np.uint8)
        blocks.append(make_block_b(scales, codes.astype(np.int64), hb_d, hb_m, b))
    while len(blocks) < 16:   # random bytes with finite d, dmin
        blk = rng.integers(0, 256, nbytes(b), dtype=np.uint8)
        for off in (nbytes(b) - 4, nbytes(b) - 2):
            blk[off + 1] &= 0x7B
        blocks.append(blk)
    canon = np.concatenate(blocks).reshape(1, -1)
    out = _pack_dequant(canon, 1, 16, 256, b)
    ref = oracle.dequant_f32(canon, bits=b).reshape(1, 16, 256)
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("b", WIDTHS)
def test_dequant_full_size_experts(b):
    """Three full-size expert matrices (2048 x 4096 gate, 4096 x 2048 down)."""
    for rows, cols in [(2048, 4096), (4096, 2048)]:
        canon = synth.qk_matrices(9, 9500 + b + rows, 3, rows, cols, 0.02, bits=b)
        out = _pack_dequant(canon, 3, rows, cols, b)
        ref = oracle.dequant_f32(canon, bits=b).reshape(3, rows, cols)
        assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


# ------------------------------------------------------------------ layers

# (gate/up width, down width; 0 = the same)
PAIRS = [(6, 0), (5, 0), (5, 6), (6, 2), (2, 5), (4, 6)]


def _wl(name, T, H, I, bits, bits_down, E=8, k=2, Is=0):
    return synth.Workload(name, 0, T=T, H=H, E=E, I=I, k=k, Is=Is, x_dtype="f32", router_dtype="f32",
                          router_sigma=0.05, layer_id=0, bits=bits, bits_down=bits_down)


def _run(L, mode, dl=None):
    q = _q()
    dl = dl if dl is not None else q.from_layer_inputs(L)
    assert (dl.bits, dl.down_bits) == (L.wl.bits, L.wl.down_width)
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


@pytest.mark.parametrize("bits,bits_down", PAIRS)
@pytest.mark.parametrize("T", [1, 2, 3, 5, 16])
def test_mid_decode(bits, bits_down, T):
    """I = 256: every decode class (routing inside gate/up at T <= 4, the
    LDS-ring and register kernels, the split down of 5..16 tokens)."""
    L = synth.make_layer(_wl("mid_q56", T, 512, 256, bits, bits_down))
    y, _, _ = _run(L, "decode")
    _check_all_tokens(L, y, f"{bits}/{bits_down} mid decode T={T}")


@pytest.mark.parametrize("bits,bits_down", [(6, 0), (5, 6)])
@pytest.mark.parametrize("T", [1, 4, 9])
def test_tiny_decode_padded(bits, bits_down, T):
    """I = 128: the padded down projection of small batches."""
    L = synth.make_layer(_wl("tiny_q56", T, 256, 128, bits, bits_down))
    y, _, _ = _run(L, "decode")
    _check_all_tokens(L, y, f"{bits}/{bits_down} tiny decode T={T}")


@pytest.mark.parametrize("bits,bits_down", [(6, 0), (5, 6), (2, 5)])
@pytest.mark.parametrize("T", [17, 65, 257])
def test_tiny_prefill_64_token_tiles(bits, bits_down, T):
    """I = 128: the 64-token GEMMs with the padded down projection."""
    L = synth.make_layer(_wl("tiny_q56", T, 256, 128, bits, bits_down))
    y, _, _ = _run(L, "prefill")
    _check_all_tokens(L, y, f"{bits}/{bits_down} tiny prefill T={T}")


@pytest.mark.parametrize("bits,bits_down", PAIRS)
@pytest.mark.parametrize("T", [48, 300, 1000])
def test_mid_prefill_wide(bits, bits_down, T):
    """I = 256: 80-token wide tiles, partial n-tiles and ragged last tiles."""
    L = synth.make_layer(_wl("mid_q56", T, 512, 256, bits, bits_down))
    y, _, _ = _run(L, "prefill")
    _check_all_tokens(L, y, f"{bits}/{bits_down} mid prefill T={T}")


def test_mid_shared_expert():
    """5/6-bit routed experts beside a bf16 shared expert (dense GEMMs)."""
    import dataclasses
    wl = dataclasses.replace(_wl("mid_q56_sh", 200, 512, 256, 5, 6, Is=96), x_dtype="bf16", router_dtype="bf16")
    L = synth.make_layer(wl)
    y, _, _ = _run(L, "prefill")
    _check_all_tokens(L, y, "5/6 mid shared T=200")


# ------------------------------------------------------------------ full size


@pytest.fixture(scope="session")
def full56():
    q = _q()
    L = synth.make_layer("prefill_q56")
    return L, q.from_layer_inputs(L)


def test_full_dequant_sample(full56):
    q = _q()
    L, dl = full56
    H, I = L.wl.H, L.wl.I
    for e in (0, 131, 255):
        for packed, canon, rows, cols, nb, b in ((dl.up, L.up, I, H, dl.gu_bytes, 5),
                                                 (dl.down, L.down, H, I, dl.d_bytes, 6)):
            out = torch.empty(rows, cols, dtype=torch.float32, device=dl.device)
            q.ds4moe_dequant(out, packed[e * nb:(e + 1) * nb], 1, rows, cols, b)
            ref = oracle.dequant_f32(canon[e], bits=b).reshape(rows, cols)
            assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32)), (e, rows)


@pytest.mark.parametrize("T", [1, 4, 16])
def test_full_decode(full56, T):
    L0, dl = full56
    L = synth.derive(L0, "decode1_q56", T=T)
    y, _, _ = _run(L, "decode", dl)
    _check_all_tokens(L, y, f"5/6 decode T={T}")


def test_full_prefill_all_tokens(full56):
    """The 2048-token prefill chunk with 5-bit gate/up and 6-bit down, every token."""
    L0, dl = full56
    L = synth.derive(L0, "prefill_q56")
    y, bufs, _ = _run(L, "prefill", dl)
    idx = bufs["topk_idx"].cpu().numpy()
    ref, ridx, _ = oracle.layer_inputs(L)
    assert np.array_equal(ridx, idx)
    err = per_token_err(y.cpu().numpy(), ref)
    print(f"5/6 prefill: all {L.T} tokens checked, per-token rel err {err:.3e}")
    assert err <= TOL_Y
