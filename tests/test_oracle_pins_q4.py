"""Pins for the oracle's 4-bit routed-expert blocks (148 bytes per 256
weights: scales[16] @0, 4-bit codes @16 with weight i at byte 16 + i/2, bits
4*(i%2), fp16 d @144 and dmin @146; w = d*scale*q - dmin*min, q in 0..15).
Each test fixes the oracle to something other than itself: hand-derived
values, single-code positions, exact rationals, the 2-bit block for codes
that both formats can hold, and a float64 dense FFN for the one-expert layer.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

from test_oracle_pins import _dense_swiglu_f64, f32_nearest, half_bits_value, make_block


def make_block4(scales, qs, d_bits, dmin_bits):
    b = np.zeros(148, dtype=np.uint8)
    b[0:16] = scales
    b[16:144] = qs
    b[144], b[145] = d_bits & 0xFF, d_bits >> 8
    b[146], b[147] = dmin_bits & 0xFF, dmin_bits >> 8
    return b


def pack_codes4(q):
    """256 codes 0..15 -> 128 bytes, weight i at byte i/2, low nibble first."""
    q = np.asarray(q, dtype=np.uint8)
    return (q[0::2] | (q[1::2] << 4)).astype(np.uint8)


def test_q4_dequant_handbuilt_block():
    # d = 0.5, dmin = 0.25; sub-block j: scale j, min 15-j; code of weight i = i % 16
    scales = np.array([((15 - j) << 4) | j for j in range(16)], dtype=np.uint8)
    blk = make_block4(scales, pack_codes4(np.arange(256) % 16), 0x3800, 0x3400)
    w = oracle.dequant_f32(blk, bits=4)
    # values derived by hand: w = 0.5*j*q - 0.25*(15-j)
    assert list(w[0:4]) == [-3.75] * 4                              # sub-block 0: scale 0
    assert list(w[48:52]) == [-3.0, -1.5, 0.0, 1.5]                  # sub-block 3: 1.5q - 3
    assert w[63] == 19.5                                             # q = 15
    assert w[241] == 7.5 and w[255] == 112.5                         # sub-block 15: 7.5q
    assert w[128] == -1.75 and w[143] == 58.25                       # sub-block 8: 4q - 1.75
    assert w.dtype == np.float32 and w.size == 256


def test_q4_code_position():
    qs = np.zeros(128, np.uint8)
    qs[10] = 0x90                                   # weight 20: q 0 (low nibble), weight 21: q 9
    scales = np.full(16, 0x01, np.uint8)            # scale 1, min 0
    w = oracle.dequant_f32(make_block4(scales, qs, 0x3C00, 0x0000), bits=4)   # d = 1
    expect = np.zeros(256, np.float32)
    expect[21] = 9.0
    assert np.array_equal(w, expect)
    qs = np.zeros(128, np.uint8)
    qs[127] = 0x0F                                  # weight 254: q 15, weight 255: q 0
    w = oracle.dequant_f32(make_block4(scales, qs, 0x3C00, 0x0000), bits=4)
    expect = np.zeros(256, np.float32)
    expect[254] = 15.0
    assert np.array_equal(w, expect)


def test_q4_special_blocks():
    assert not oracle.dequant_f32(np.zeros(148, np.uint8), bits=4).any()
    scales = np.full(16, 0x21, np.uint8)                            # scale 1, min 2
    qs = np.full(128, 0xFF, np.uint8)                               # q = 15
    w = oracle.dequant_f32(make_block4(scales, qs, 0xBC00, 0x3800), bits=4)   # d = -1, dmin = 0.5
    assert np.all(w == np.float32(-16.0))                           # -1*1*15 - 0.5*2
    w = oracle.dequant_f32(make_block4(np.full(16, 0x0F, np.uint8), qs, 0x0001, 0x0000), bits=4)
    assert np.all(w == np.float32(2.0 ** -24 * 225))                # subnormal d, scale 15, q 15


def test_q4_matches_q2_for_small_codes():
    """Codes 0..3 mean the same in both formats: equal scales, d and dmin give
    equal weights."""
    rng = np.random.default_rng(11)
    for _ in range(8):
        scales = rng.integers(0, 256, 16, dtype=np.uint8)
        q = rng.integers(0, 4, 256)
        q2 = np.zeros(64, np.uint8)
        for i in range(256):
            q2[i // 4] |= np.uint8(q[i] << (2 * (i % 4)))
        d, dm = int(rng.integers(0x3000, 0x4000)), int(rng.integers(0x3000, 0x4000))
        w2 = oracle.dequant_f32(make_block(scales, q2, d, dm))
        w4 = oracle.dequant_f32(make_block4(scales, pack_codes4(q), d, dm), bits=4)
        assert np.array_equal(w2, w4)


def test_q4_exact_rounding_random():
    """fp32 dequant == the correctly rounded exact rational (products of at
    most 19 significant bits), for random blocks with any finite fp16 d, dmin."""
    rng = np.random.default_rng(17)
    nb = 48
    blocks = rng.integers(0, 256, size=(nb, 148), dtype=np.uint8)
    for b in range(nb):
        for off in (144, 146):
            while True:
                bits = int(rng.integers(0, 1 << 16))
                if (bits >> 10) & 0x1F != 31:
                    break
            blocks[b, off], blocks[b, off + 1] = bits & 0xFF, bits >> 8
    w = oracle.dequant_f32(blocks, bits=4)
    for b in range(0, nb, 3):
        blk = blocks[b]
        d = half_bits_value(int(blk[144]) | int(blk[145]) << 8)
        dm = half_bits_value(int(blk[146]) | int(blk[147]) << 8)
        for i in range(0, 256, 5):
            j = i // 16
            sc, mn = int(blk[j]) & 15, int(blk[j]) >> 4
            q = (int(blk[16 + i // 2]) >> (4 * (i % 2))) & 15
            assert w[b * 256 + i] == f32_nearest(d * sc * q - dm * mn)


def test_q4_quantizer_error():
    """The 4-bit quantizer of the same draws is about five times as accurate
    as the 2-bit one (15 steps per sub-block instead of 3)."""
    w = synth.normal_f32(3, 99, 0.02, (64, 256))
    ww = w.astype(np.float64)
    rel = {}
    for bits in (2, 4):
        dq = oracle.dequant_f64(synth.quantize_blocks(w, bits=bits), bits=bits).reshape(64, 256)
        rel[bits] = np.sqrt(np.mean((dq - ww) ** 2)) / np.sqrt(np.mean(ww ** 2))
    assert rel[4] < 0.12 and rel[4] < rel[2] / 3


def test_q4_layer_single_expert_equals_dense_ffn():
    rng = np.random.default_rng(43)
    T, H, I = 4, 256, 128

    def q4(rows, cols):
        return synth.quantize_blocks((0.02 * rng.standard_normal((rows, cols))).astype(np.float32), bits=4)

    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = np.zeros((1, H), np.float32)
    g, u, d = q4(I, H), q4(I, H), q4(H, I)
    y, idx, w = oracle.layer(x, wr, None, g[None], u[None], d[None], H, I, 1, 1, bits=4)
    assert np.all(idx == 0) and np.all(w == 1.0)
    Wg = torch.from_numpy(oracle.dequant_f64(g, bits=4).reshape(I, H))
    Wu = torch.from_numpy(oracle.dequant_f64(u, bits=4).reshape(I, H))
    Wd = torch.from_numpy(oracle.dequant_f64(d, bits=4).reshape(H, I))
    ref = _dense_swiglu_f64(Wg, Wu, Wd, torch.from_numpy(x).double()).float().numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-6, atol=1e-7)


def test_q4_generator_blocks_decode_near_draws():
    """Generated 4-bit expert matrices: the block count and size are right and
    every block decodes to finite weights of the N(0, 0.02) scale."""
    m = synth.qk_matrices(5, 7000, 2, 32, 256, 0.02, bits=4)
    assert m.shape == (2, 32 * 148)
    w = oracle.dequant_f64(m, bits=4)
    assert np.all(np.isfinite(w)) and 0.01 < w.std() < 0.03


@pytest.mark.parametrize("gu_bits,dn_bits", [(2, 4), (4, 2)])
def test_mixed_widths_two_experts_equal_dense_ffns(gu_bits, dn_bits):
    """Gate/up in one code width and down in the other: two experts, k = 2,
    against the float64 library FFN on each expert's dequantized matrices
    (each width's dequantization is pinned above), combined with the routing
    weights.  A slip in which matrix takes which width, or in the down
    matrices' expert stride, fails here."""
    rng = np.random.default_rng(44 + gu_bits)
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
