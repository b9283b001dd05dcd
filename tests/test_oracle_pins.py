"""Pins for the CPU oracle: each test fixes the oracle to something other than
itself -- hand-derived block values, exact rational arithmetic, high-precision
decimal evaluation, brute force over small inputs, a float64 library FFN on
special cases, closed forms and invariants.  A plausible slip anywhere in the
oracle (swapped nibble, byte or code order, a dropped min term, a wrong sign,
a transposed operand, a wrong tie-break, an unstable softplus, a wrong combine
order or weight) makes at least one of these fail.
"""
import decimal
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

# ---------------------------------------------------------------- helpers


def make_block(scales, qs, d_bits, dmin_bits):
    b = np.zeros(84, dtype=np.uint8)
    b[0:16] = scales
    b[16:80] = qs
    b[80], b[81] = d_bits & 0xFF, d_bits >> 8
    b[82], b[83] = dmin_bits & 0xFF, dmin_bits >> 8
    return b


def f32_nearest(fr: Fraction) -> np.float32:
    """Correctly rounded (nearest-even) fp32 value of an exact rational."""
    c = np.float32(float(fr))  # within one fp32 ulp of the answer
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        err = abs(Fraction(float(cand)) - fr)
        key = (err, int(np.frombuffer(np.float32(cand).tobytes(), np.uint32)[0]) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return np.float32(best[1])


def half_bits_value(bits: int) -> Fraction:
    s = -1 if bits & 0x8000 else 1
    e = (bits >> 10) & 0x1F
    m = bits & 0x3FF
    assert e != 31
    if e == 0:
        return s * Fraction(m, 1 << 24)
    return s * Fraction(m + 1024, 1) * (Fraction(2) ** (e - 25))


# ---------------------------------------------------------------- dequant


def test_dequant_handbuilt_block():
    # d = 0.5 (0x3800), dmin = 0.25 (0x3400); sub-block j has scale j (low
    # nibble) and min 15-j (high nibble); every code byte 0xE4 = codes 0,1,2,3.
    scales = np.array([((15 - j) << 4) | j for j in range(16)], dtype=np.uint8)
    blk = make_block(scales, np.full(64, 0xE4, np.uint8), 0x3800, 0x3400)
    w = oracle.dequant_f32(blk)
    # values derived by hand: w = 0.5*j*q - 0.25*(15-j)
    assert list(w[0:4]) == [-3.75, -3.75, -3.75, -3.75]           # sub-block 0: scale 0
    assert list(w[48:52]) == [-3.0, -1.5, 0.0, 1.5]                 # sub-block 3
    assert list(w[52:56]) == [-3.0, -1.5, 0.0, 1.5]
    assert list(w[240:244]) == [0.0, 7.5, 15.0, 22.5]               # sub-block 15: min 0
    assert list(w[128:132]) == [-1.75, 2.25, 6.25, 10.25]           # sub-block 8: 4q - 1.75
    assert w.dtype == np.float32 and w.size == 256


def test_dequant_code_position():
    # only byte 5 of qs holds codes (all 3): weights 20..23 are q=3, rest q=0.
    qs = np.zeros(64, np.uint8)
    qs[5] = 0xFF
    scales = np.full(16, 0x01, np.uint8)                            # scale 1, min 0
    w = oracle.dequant_f32(make_block(scales, qs, 0x3C00, 0x0000))  # d = 1
    expect = np.zeros(256, np.float32)
    expect[20:24] = 3.0
    assert np.array_equal(w, expect)
    # single code in the high bits of byte 0 -> weight 3 only
    qs = np.zeros(64, np.uint8)
    qs[0] = 0x80                                                    # bits 6-7 = 2
    w = oracle.dequant_f32(make_block(scales, qs, 0x3C00, 0x0000))
    expect = np.zeros(256, np.float32)
    expect[3] = 2.0
    assert np.array_equal(w, expect)


def test_dequant_special_blocks():
    assert not oracle.dequant_f32(np.zeros(84, np.uint8)).any()
    scales = np.full(16, 0x21, np.uint8)                            # scale 1, min 2
    qs = np.full(64, 0xFF, np.uint8)                                # q = 3
    w = oracle.dequant_f32(make_block(scales, qs, 0xBC00, 0x3800))  # d=-1, dmin=0.5
    assert np.all(w == np.float32(-4.0))                            # -1*1*3 - 0.5*2
    w = oracle.dequant_f32(make_block(np.full(16, 0x0F, np.uint8), qs, 0x0001, 0x0000))
    assert np.all(w == np.float32(2.0 ** -24 * 45))                 # subnormal d


def test_dequant_exact_rounding_random():
    """oracle fp32 dequant == correctly rounded exact rational, and the fp32
    evaluation order does not matter (products exact, one rounding)."""
    rng = np.random.default_rng(7)
    nb = 64
    blocks = rng.integers(0, 256, size=(nb, 84), dtype=np.uint8)
    # random finite fp16 d, dmin including subnormals and negatives
    for b in range(nb):
        for off in (80, 82):
            while True:
                bits = int(rng.integers(0, 1 << 16))
                if (bits >> 10) & 0x1F != 31:
                    break
            blocks[b, off], blocks[b, off + 1] = bits & 0xFF, bits >> 8
    w = oracle.dequant_f32(blocks)
    for b in range(0, nb, 4):
        blk = blocks[b]
        d = half_bits_value(int(blk[80]) | int(blk[81]) << 8)
        dm = half_bits_value(int(blk[82]) | int(blk[83]) << 8)
        d32, dm32 = np.float32(float(d)), np.float32(float(dm))
        for i in range(0, 256, 7):
            j = i // 16
            sc, mn = int(blk[j]) & 15, int(blk[j]) >> 4
            q = (int(blk[16 + i // 4]) >> (2 * (i % 4))) & 3
            exact = d * sc * q - dm * mn
            assert w[b * 256 + i] == f32_nearest(exact)
            alt = np.float32(np.float32(d32 * np.float32(sc)) * np.float32(q)) - np.float32(dm32 * np.float32(mn))
            assert w[b * 256 + i] == alt


def test_dequant_matches_generated_weights():
    # the quantizer's blocks decode to values close to the N(0,0.02) draws
    w = synth.normal_f32(3, 99, 0.02, (64, 256))
    dq = oracle.dequant_f64(synth.quantize_blocks(w)).reshape(64, 256)
    rel = np.sqrt(np.mean((dq - w) ** 2)) / np.sqrt(np.mean(w.astype(np.float64) ** 2))
    assert 0.15 < rel < 0.45


# ---------------------------------------------------------------- logits


def test_logits_exact_rational_f32_inputs():
    rng = np.random.default_rng(11)
    T, E, H = 6, 8, 256
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (0.05 * rng.standard_normal((E, H))).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    lg = oracle.logits(x, wr, b)
    for t in range(T):
        for e in range(E):
            exact = sum(Fraction(float(x[t, h])) * Fraction(float(wr[e, h])) for h in range(H)) + Fraction(float(b[e]))
            assert lg[t, e] == f32_nearest(exact), (t, e)


def test_logits_match_float64_matmul_bf16():
    rng = np.random.default_rng(12)
    T, E, H = 16, 64, 1024
    xb = synth.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    wb = synth.f32_to_bf16_bits((0.02 * rng.standard_normal((E, H))).astype(np.float32))
    x, wr = oracle.bf16_to_f32(xb), oracle.bf16_to_f32(wb)
    ref = (torch.from_numpy(x).double() @ torch.from_numpy(wr).double().T).float().numpy()
    assert np.array_equal(oracle.logits(x, wr), ref)


# ---------------------------------------------------------------- score


def _score_dec(x: float) -> float:
    with decimal.localcontext() as ctx:
        ctx.prec = 60
        X = decimal.Decimal(x)
        return float((1 + X.exp()).ln().sqrt())


@pytest.mark.parametrize("x", [-12.0, 0.0, -40.0, 20.0, 100.0, -88.0, 5.5, -1e-3, 1e-3, -16.7, -30.0, 89.0])
def test_score_high_precision(x):
    ref = _score_dec(x)
    assert math.isclose(oracle.score(x), ref, rel_tol=4e-16), (x, oracle.score(x), ref)


def test_score_known_values():
    # sqrt(ln 2) at 0; at -12, ln(1+e^-12) = 6.144193...e-6
    assert math.isclose(oracle.score(0.0), math.sqrt(math.log(2.0)), rel_tol=1e-15)
    assert math.isclose(oracle.score(-12.0), 0.0024787483691840, rel_tol=1e-12)
    assert math.isclose(oracle.score(100.0), 10.0, rel_tol=1e-15)


def test_score_naive_fp32_fails_near_minus_12():
    # The failure the router fix addresses: 1 + exp(x) formed in fp32 near
    # logit -12 loses the small term; the oracle keeps it.
    x = np.float32(-12.0)
    naive = np.sqrt(np.log(np.float32(1.0) + np.exp(x, dtype=np.float32), dtype=np.float32), dtype=np.float32)
    ref = _score_dec(-12.0)
    assert abs(float(naive) - ref) / ref > 3e-6
    assert abs(oracle.score(-12.0) - ref) / ref < 1e-15


def test_series_reading_meets_router_tolerance():
    """The reading of the router fix used by the GPU path (fp32: log1p(t) by the
    4-term series t - t^2/2 + t^3/3 - t^4/4 when t = exp(-|l|) < 1/32, with the
    series input clamped; log(1+t) otherwise) stays within 3e-6 of the oracle."""
    l = np.arange(-30.0, 30.0, 0.005).astype(np.float32)
    t = np.exp(-np.abs(l), dtype=np.float32)
    tc = np.minimum(t, np.float32(1.0 / 32.0))
    ser = tc * (np.float32(1) - tc * (np.float32(0.5) - tc * (np.float32(1 / 3.0) - tc * np.float32(0.25))))
    lg = np.where(t < np.float32(1 / 32.0), ser, np.log1p(t, dtype=np.float32)).astype(np.float32)
    s = np.sqrt(np.maximum(l, np.float32(0)) + lg, dtype=np.float32)
    ref = oracle.scores(l)
    assert np.max(np.abs(s - ref) / ref) < 3e-6


# ---------------------------------------------------------------- top-k


def _beats(la, a, lb, b):
    return la > lb or (la == lb and a < b)


def test_topk_bruteforce_subsets():
    rng = np.random.default_rng(21)
    T, E, k = 60, 8, 3
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[::5, 2] = lg[::5, 5]          # exact ties
    lg[::7, :4] = 0.25               # four-way ties
    idx, w, _ = oracle.topk(lg, k)
    for t in range(T):
        winners = [S for S in itertools.combinations(range(E), k)
                   if all(_beats(lg[t, a], a, lg[t, b], b) for a in S for b in range(E) if b not in S)]
        assert len(winners) == 1
        order = sorted(winners[0], key=lambda e: (-lg[t, e], e))
        assert list(idx[t]) == order


def test_topk_ties_and_uniform():
    E, k = 8, 4
    lg = np.zeros((2, E), np.float32)
    idx, w, wd = oracle.topk(lg, k)
    assert idx.tolist() == [[0, 1, 2, 3]] * 2
    assert np.all(w == np.float32(0.25))
    lg = np.array([[1.0, 3.0, 3.0, 2.0, 3.0, -1.0, 0.0, 2.0]], np.float32)
    idx, _, _ = oracle.topk(lg, 5)
    assert idx.tolist() == [[1, 2, 4, 3, 7]]


def test_topk_nan_and_inf_ordering_bruteforce():
    """NaN logits (out of contract) rank below every number, -inf included,
    and among themselves by expert index; +inf ranks first.  Checked against
    a plain Python sort on the key (is NaN, -logit, expert) over random rows
    mixing NaN, +-inf, exact ties and ordinary values, k from 1 to E."""
    rng = np.random.default_rng(23)
    for trial in range(300):
        E = int(rng.integers(2, 20))
        k = int(rng.integers(1, E + 1))
        lg = rng.standard_normal((1, E)).astype(np.float32)
        r = rng.random(E)
        lg[0, r < 0.25] = np.nan
        lg[0, (r >= 0.25) & (r < 0.32)] = -np.inf
        lg[0, (r >= 0.32) & (r < 0.36)] = np.inf
        lg[0, (r >= 0.36) & (r < 0.46)] = 0.5          # exact ties
        idx, _, _ = oracle.topk(lg, k)
        row = [float(v) for v in lg[0]]
        order = sorted(range(E), key=lambda e: (math.isnan(row[e]), 0.0 if math.isnan(row[e]) else -row[e], e))
        assert list(idx[0]) == order[:k], (row, k)
    lg = np.full((1, 6), np.nan, np.float32)
    idx, _, _ = oracle.topk(lg, 4)
    assert idx.tolist() == [[0, 1, 2, 3]]                     # all NaN: experts in index order


def test_topk_weights_invariants():
    rng = np.random.default_rng(22)
    lg = (3 * rng.standard_normal((200, 256))).astype(np.float32)
    idx, w, wd = oracle.topk(lg, 8)
    s = w.astype(np.float32).sum(axis=1, dtype=np.float32)
    assert np.max(np.abs(s - 1.0)) <= 2.0 ** -21
    assert np.allclose(wd.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert np.all(np.diff(wd, axis=1) <= 0)                   # rank order = descending score
    _, w1, _ = oracle.topk(lg, 1)
    assert np.all(w1 == 1.0)
    # weights are s_j / sum s: check one row against the high-precision score
    sc = [_score_dec(float(lg[0, e])) for e in idx[0]]
    assert np.allclose(wd[0], np.array(sc) / sum(sc), rtol=1e-14)


# ---------------------------------------------------------------- permutation


def test_permute_bruteforce():
    rng = np.random.default_rng(31)
    T, E, k = 37, 16, 4
    lg = rng.standard_normal((T, E)).astype(np.float32)
    idx, _, _ = oracle.topk(lg, k)
    counts, offsets, perm = oracle.permute(idx, E)
    flat = idx.reshape(-1)
    ref = sorted(range(T * k), key=lambda a: (flat[a], a // k))
    assert perm.tolist() == ref
    assert counts.tolist() == [int((flat == e).sum()) for e in range(E)]
    assert offsets[0] == 0 and offsets[-1] == T * k
    assert np.array_equal(np.diff(offsets), counts)
    assert sorted(perm.tolist()) == list(range(T * k))


# ---------------------------------------------------------------- layer


def _dense_swiglu_f64(Wg, Wu, Wd, x):
    g = x @ Wg.T
    u = x @ Wu.T
    h = g * torch.sigmoid(g) * u
    return h @ Wd.T


def _q2k(rng, rows, cols, sigma=0.02):
    return synth.quantize_blocks((sigma * rng.standard_normal((rows, cols))).astype(np.float32))


def test_layer_single_expert_equals_dense_ffn():
    rng = np.random.default_rng(41)
    T, H, I = 5, 256, 128
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = np.zeros((1, H), np.float32)
    g, u, d = _q2k(rng, I, H), _q2k(rng, I, H), _q2k(rng, H, I)
    y, idx, w = oracle.layer(x, wr, None, g[None], u[None], d[None], H, I, 1, 1)
    assert np.all(idx == 0) and np.all(w == 1.0)
    Wg = torch.from_numpy(oracle.dequant_f64(g).reshape(I, H))
    Wu = torch.from_numpy(oracle.dequant_f64(u).reshape(I, H))
    Wd = torch.from_numpy(oracle.dequant_f64(d).reshape(H, I))
    ref = _dense_swiglu_f64(Wg, Wu, Wd, torch.from_numpy(x).double()).float().numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-6, atol=1e-7)


def test_layer_two_experts_weighted_combine():
    rng = np.random.default_rng(42)
    T, H, I, E, k = 4, 256, 128, 3, 2
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (0.05 * rng.standard_normal((E, H))).astype(np.float32)
    g = np.stack([_q2k(rng, I, H) for _ in range(E)])
    u = np.stack([_q2k(rng, I, H) for _ in range(E)])
    d = np.stack([_q2k(rng, H, I) for _ in range(E)])
    y, idx, w = oracle.layer(x, wr, None, g, u, d, H, I, E, k)
    lg = (torch.from_numpy(x).double() @ torch.from_numpy(wr).double().T).float().numpy()
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-lg[t, e], e))[:k]
        assert list(idx[t]) == order
        s = [_score_dec(float(lg[t, e])) for e in order]
        acc = torch.zeros(H, dtype=torch.float64)
        for j, e in enumerate(order):
            Wg = torch.from_numpy(oracle.dequant_f64(g[e]).reshape(I, H))
            Wu = torch.from_numpy(oracle.dequant_f64(u[e]).reshape(I, H))
            Wd = torch.from_numpy(oracle.dequant_f64(d[e]).reshape(H, I))
            acc += (s[j] / sum(s)) * _dense_swiglu_f64(Wg, Wu, Wd, torch.from_numpy(x[t]).double())
        np.testing.assert_allclose(y[t], acc.float().numpy(), rtol=1e-6, atol=1e-7)


def test_layer_constant_blocks_closed_form():
    # every block encodes the constant c = 2^-6 (scale 1, min 0, code 1, d = c):
    # g_i = u_i = c*sum(x); h = silu(c*sum x)*(c*sum x); y_j = c*I*h.
    T, H, I, E, k = 3, 256, 128, 4, 2
    c_bits = 0x2400                                   # 2^-6 in binary16
    blk = make_block(np.full(16, 0x01, np.uint8), np.full(64, 0x55, np.uint8), c_bits, 0)
    gate = np.tile(blk, (E, I * H // 256))
    down = np.tile(blk, (E, H * I // 256))
    rng = np.random.default_rng(43)
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = (0.05 * rng.standard_normal((E, H))).astype(np.float32)
    y, _, _ = oracle.layer(x, wr, None, gate, gate, down, H, I, E, k)
    c = 2.0 ** -6
    for t in range(T):
        z = c * float(np.sum(x[t].astype(np.float64)))
        h = z / (1 + math.exp(-z)) * z
        assert np.allclose(y[t], c * I * h, rtol=1e-6, atol=0)


def test_layer_zero_weights_give_zero():
    T, H, I, E, k = 4, 256, 128, 4, 2
    z = np.zeros((E, I * H // 256 * 84), np.uint8)
    rng = np.random.default_rng(44)
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = rng.standard_normal((E, H)).astype(np.float32)
    y, _, _ = oracle.layer(x, wr, None, z, z, z, H, I, E, k)
    assert not y.any()


def test_layer_shared_expert_only():
    rng = np.random.default_rng(45)
    T, H, I, E, k, Is = 3, 256, 128, 4, 2, 64
    z = np.zeros((E, I * H // 256 * 84), np.uint8)
    x = rng.standard_normal((T, H)).astype(np.float32)
    wr = rng.standard_normal((E, H)).astype(np.float32)
    sg = oracle.bf16_to_f32(synth.f32_to_bf16_bits((0.02 * rng.standard_normal((Is, H))).astype(np.float32)))
    su = oracle.bf16_to_f32(synth.f32_to_bf16_bits((0.02 * rng.standard_normal((Is, H))).astype(np.float32)))
    sd = oracle.bf16_to_f32(synth.f32_to_bf16_bits((0.02 * rng.standard_normal((H, Is))).astype(np.float32)))
    y, _, _ = oracle.layer(x, wr, None, z, z, z, H, I, E, k, sg, su, sd)
    ref = _dense_swiglu_f64(*(torch.from_numpy(a).double() for a in (sg, su, sd)), torch.from_numpy(x).double())
    np.testing.assert_allclose(y, ref.float().numpy(), rtol=1e-6, atol=1e-8)


def test_layer_token_independence():
    L = synth.make_layer("tiny")
    y, idx, w = oracle.layer_inputs(L)
    for t in (0, 7, 15):
        y1, idx1, w1 = oracle.layer_inputs(L, tokens=[t])
        assert np.array_equal(y1[0], y[t]) and np.array_equal(idx1[0], idx[t]) and np.array_equal(w1[0], w[t])
