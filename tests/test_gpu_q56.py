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
