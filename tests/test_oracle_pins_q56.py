"""Pins for the oracle's 5- and 6-bit routed-expert blocks (the 2-bit
super-block with b-bit codes: scales[16] @0, the 256 codes as one bit stream
from byte 16, lowest bits first, weight i at bits b*i .. b*i+b-1, fp16 d and
dmin after the codes: 180 bytes for b = 5, 212 for b = 6; w = d*scale*q -
dmin*min, q in 0..2^b-1).  Each test fixes the oracle to something other than
itself: hand-derived values, single codes at positions that straddle byte
boundaries (the expected bytes written with Python's big integers, not with
the oracle's shifts), exact rationals, the 4-bit block for codes both widths
hold, and a float64 dense FFN for one-expert and mixed-width layers.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

from test_oracle_pins import _dense_swiglu_f64, f32_nearest, half_bits_value
from test_oracle_pins_q4 import make_block4, pack_codes4

WIDTHS = (5, 6)


def nbytes(b):
    return 16 + 32 * b + 4


def pack_stream(q, b):
    """256 codes of b bits -> 32*b bytes: little-endian integer whose bits
    b*i .. b*i+b-1 hold code i."""
    v = 0
    for i, c in enumerate(q):
        assert 0 <= int(c) < (1 << b)
        v |= int(c) << (b * i)
    return np.frombuffer(v.to_bytes(32 * b, "little"), dtype=np.uint8).copy()


def make_block_b(scales, q, d_bits, dmin_bits, b):
    n = nbytes(b)
    blk = np.zeros(n, dtype=np.uint8)
    blk[0:16] = scales
    blk[16:16 + 32 * b] = pack_stream(q, b)
    blk[n - 4], blk[n - 3] = d_bits & 0xFF, d_bits >> 8
    blk[n - 2], blk[n - 1] = dmin_bits & 0xFF, dmin_bits >> 8
    return blk


@pytest.mark.parametrize("b", WIDTHS)
def test_block_sizes(b):
    assert oracle.block_bytes(b) == nbytes(b) == {5: 180, 6: 212}[b]
    assert synth.block_bytes(b) == nbytes(b)


@pytest.mark.parametrize("b", WIDTHS)
def test_dequant_handbuilt_block(b):
    # d = 0.5, dmin = 0.25; sub-block j: scale j, min 15-j; code of weight i = i mod 2^b
    top = (1 << b) - 1
    scales = np.array([((15 - j) << 4) | j for j in range(16)], dtype=np.uint8)
    q = np.arange(256) % (1 << b)
    w = oracle.dequant_f32(make_block_b(scales, q, 0x3800, 0x3400, b), bits=b)
    # by hand: w = 0.5*j*q - 0.25*(15-j)
    assert list(w[0:4]) == [-3.75] * 4                                # sub-block 0: scale 0
    # sub-block 3: 1.5q - 3, q = 48..51 mod 2^b
    assert list(w[48:52]) == {5: [21.0, 22.5, 24.0, 25.5], 6: [69.0, 70.5, 72.0, 73.5]}[b]
    # sub-block 15 (scale 15, min 0): 7.5q; the last weight has q = top (255 mod 2^b)
    assert w[255] == {5: 232.5, 6: 472.5}[b] == 7.5 * top
    assert w[240] == {5: 120.0, 6: 360.0}[b]                           # q = 240 mod 2^b: 16 and 48
    assert w.dtype == np.float32 and w.size == 256


@pytest.mark.parametrize("b", WIDTHS)
def test_code_positions_straddle_bytes(b):
    """One nonzero code at a time, at positions whose bits start mid-byte and
    cross into the next byte; every other weight decodes to zero."""
    top = (1 << b) - 1
    scales = np.full(16, 0x01, np.uint8)       # scale 1, min 0
    for i in (0, 1, 3, 7, 13, 100, 127, 200, 254, 255):
        q = np.zeros(256, np.int64)
        q[i] = top - (i % 3)
        w = oracle.dequant_f32(make_block_b(scales, q, 0x3C00, 0x0000, b), bits=b)   # d = 1
        expect = np.zeros(256, np.float32)
        expect[i] = float(q[i])
        assert np.array_equal(w, expect), i


@pytest.mark.parametrize("b", WIDTHS)
def test_special_blocks(b):
    n = nbytes(b)
    top = (1 << b) - 1
    assert not oracle.dequant_f32(np.zeros(n, np.uint8), bits=b).any()
    q = np.full(256, top)
    w = oracle.dequant_f32(make_block_b(np.full(16, 0x21, np.uint8), q, 0xBC00, 0x3800, b), bits=b)  # d=-1, dmin=.5
    assert np.all(w == np.float32(-top - 1.0))                          # -1*1*top - 0.5*2
    w = oracle.dequant_f32(make_block_b(np.full(16, 0x0F, np.uint8), q, 0x0001, 0x0000, b), bits=b)
    assert np.all(w == np.float32(2.0 ** -24 * 15 * top))               # subnormal d, scale 15


@pytest.mark.parametrize("b", WIDTHS)
def test_matches_q4_for_small_codes(b):
    """Codes 0..15 mean the same in the 4-bit and the b-bit block: equal
    scales, d and dmin give equal weights."""
    rng = np.random.default_rng(21 + b)
    for _ in range(8):
        scales = rng.integers(0, 256, 16, dtype=np.uint8)
        q = rng.integers(0, 16, 256)
        d, dm = int(rng.integers(0x3000, 0x4000)), int(rng.integers(0x3000, 0x4000))
        w4 = oracle.dequant_f32(make_block4(scales, pack_codes4(q), d, dm), bits=4)
        wb = oracle.dequant_f32(make_block_b(scales, q, d, dm, b), bits=b)
        assert np.array_equal(w4, wb)


@pytest.mark.parametrize("b", WIDTHS)
def test_exact_rounding_random(b):
    """fp32 dequant == the correctly rounded exact rational (products of at
    most 21 significant bits), for random blocks with any finite fp16 d, dmin."""
    rng = np.random.default_rng(27 + b)
    n = nbytes(b)
    nb = 32
    blocks = rng.integers(0, 256, size=(nb, n), dtype=np.uint8)
    for k in range(nb):
        for off in (n - 4, n - 2):
            while True:
                hb = int(rng.integers(0, 1 << 16))
                if (hb >> 10) & 0x1F != 31:
                    break
            blocks[k, off], blocks[k, off + 1] = hb & 0xFF, hb >> 8
    w = oracle.dequant_f32(blocks, bits=b)
    for k in range(0, nb, 3):
        blk = blocks[k]
        d = half_bits_value(int(blk[n - 4]) | int(blk[n - 3]) << 8)
        dm = half_bits_value(int(blk[n - 2]) | int(blk[n - 1]) << 8)
        stream = int.from_bytes(bytes(blk[16:16 + 32 * b]), "little")
        for i in range(0, 256, 5):
            j = i // 16
            sc, mn = int(blk[j]) & 15, int(blk[j]) >> 4
            q = (stream >> (b * i)) & ((1 << b) - 1)
            assert w[k * 256 + i] == f32_nearest(d * sc * q - dm * mn)


def test_quantizer_error_falls_with_width():
    """The quantizer of the same draws: each extra code bit lowers the rms
    error (2^b - 1 steps per sub-block; the 4-bit sub-block scales keep the
    step at 6 bits from halving again)."""
    w = synth.normal_f32(3, 99, 0.02, (64, 256))
    ww = w.astype(np.float64)
    rel = {}
    for b in (4, 5, 6):
        dq = oracle.dequant_f64(synth.quantize_blocks(w, bits=b), bits=b).reshape(64, 256)
        rel[b] = np.sqrt(np.mean((dq - ww) ** 2)) / np.sqrt(np.mean(ww ** 2))
    assert rel[5] < rel[4] * 0.7 and rel[6] < rel[5] * 0.8 and rel[6] < 0.035


@pytest.mark.parametrize("b", WIDTHS)
def test_generator_blocks_decode_near_draws(b):
    m = synth.qk_matrices(5, 7100 + b, 2, 32, 256, 0.02, bits=b)
    assert m.shape == (2, 32 * nbytes(b))
    w = oracle.dequant_f64(m, bits=b)
    assert np.all(np.isfinite(w)) and 0.01 < w.std() < 0.03


@pytest.mark.parametrize("b", WIDTHS)
def test_layer_single_expert_equals_dense_ffn(b):
    rng = np.random.default_rng(53 + b)
    T, H, I = 4, 256, 128

    def qb(rows, cols):
        return synth.quantize_blocks((0.02 * rng.standard_normal((rows, cols))).astype(np.float32), bits=b)

    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = np.zeros((1, H), np.float32)
    g, u, d = qb(I, H), qb(I, H), qb(H, I)
    y, idx, w = oracle.layer(x, wr, None, g[None], u[None], d[None], H, I, 1, 1, bits=b)
    assert np.all(idx == 0) and np.all(w == 1.0)
    Wg = torch.from_numpy(oracle.dequant_f64(g, bits=b).reshape(I, H))
    Wu = torch.from_numpy(oracle.dequant_f64(u, bits=b).reshape(I, H))
    Wd = torch.from_numpy(oracle.dequant_f64(d, bits=b).reshape(H, I))
    ref = _dense_swiglu_f64(Wg, Wu, Wd, torch.from_numpy(x).double()).float().numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("gu_bits,dn_bits", [(5, 6), (6, 2), (2, 5)])
def test_mixed_widths_two_experts_equal_dense_ffns(gu_bits, dn_bits):
    """Gate/up in one width and down in another (5-bit gate/up with 6-bit
    down is the pages' GLM pairing), two experts, k = 2, against the float64
    library FFN on each expert's dequantized matrices."""
    rng = np.random.default_rng(64 + gu_bits + 7 * dn_bits)
    T, H, I, E = 5, 256, 256, 2

    def qb(rows, cols, bits):
        return synth.quantize_blocks((0.02 * rng.standard_normal((rows, cols))).astype(np.float32), bits=bits)

    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (0.05 * rng.standard_normal((E, H))).astype(np.float32)
    g = np.stack([qb(I, H, gu_bits) for _ in range(E)])
    u = np.stack([qb(I, H, gu_bits) for _ in range(E)])
    d = np.stack([qb(H, I, dn_bits) for _ in range(E)])
    y, idx, w = oracle.layer(x, wr, None, g, u, d, H, I, E, 2, bits=gu_bits, down_bits=dn_bits)
    _, _, wd = oracle.topk(oracle.logits(x, wr), 2)
    xt = torch.from_numpy(x).double()
    ref = torch.zeros(T, H, dtype=torch.float64)
    for e in range(E):
        Wg = torch.from_numpy(oracle.dequant_f64(g[e], bits=gu_bits).reshape(I, H))
        Wu = torch.from_numpy(oracle.dequant_f64(u[e], bits=gu_bits).reshape(I, H))
        Wd = torch.from_numpy(oracle.dequant_f64(d[e], bits=dn_bits).reshape(H, I))
        ye = _dense_swiglu_f64(Wg, Wu, Wd, xt)
        for t in range(T):
            j = int(np.where(idx[t] == e)[0][0])
            ref[t] += wd[t, j] * ye[t]
    np.testing.assert_allclose(y, ref.float().numpy(), rtol=1e-6, atol=1e-7)
