"""GPU parity of the router in the regimes the ds4 router numeric test is about
(opensource-hub.com "antirez/ds4" page, FAQ #1): scores of logits near -12,
where log(1 + exp(x)) in fp32 loses its digits, and across the whole range
the 4-term log1p series and the log(1 + u) branch share; plus bit-equal
logits, where the selection must break ties to the lower expert index.

Every case runs on each routing code path of the library:
* T = 1 decode: the one-token routing inside the gate/up kernel;
* T = 2..4 decode: the small-batch routing inside the gate/up kernel;
* T = 5..16 decode and route-only calls with T <= 16: the routing kernel;
* T > 16 (prefill and route-only): the chunked top-k kernel.

Bars as everywhere: logits, indices, counts, offsets and the permutation
bit-exact, weights within 3e-6 relative, y within 2e-3 per token.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

from test_gpu_parity import TOL_W, TOL_Y, check_routing, per_token_err

pytestmark = pytest.mark.gpu

DECODE_T = [1, 3, 4, 9, 16]
PREFILL_T = [40, 2048]


def _q():
    import quantized_routed_moe_router_amd as q
    return q


def _layer(T, E, k, router_sigma, bias, seed_layer=0, dup=()):
    """Small fp32 layer (H = 256, I = 128) whose logits are bias + a small
    router term; `dup` lists (src, dst) router rows copied so that their
    logits are bit-equal."""
    wl = synth.Workload("edge", 0, T=T, H=256, E=E, I=128, k=k, x_dtype="f32", router_dtype="f32",
                        router_sigma=router_sigma, layer_id=seed_layer)
    L = synth.make_layer(wl)
    rw = L.router_w.copy()
    for src, dst in dup:
        rw[dst] = rw[src]
    L.router_w = rw
    L.router_bias = np.asarray(bias, np.float32)
    return L


def _run(L, mode):
    q = _q()
    dl = q.from_layer_inputs(L)
    bufs = dl.routing_buffers(L.T)
    if mode == "route":
        bufs = dl.route(dl.x_tensor(L.x))
        torch.cuda.synchronize()
        return None, bufs
    m = q.MODE_DECODE if mode == "decode" else q.MODE_PREFILL
    y = dl.forward(dl.x_tensor(L.x), m, routing=bufs)
    torch.cuda.synchronize()
    return y, bufs


def _check(L, y, bufs, label):
    idx = check_routing(bufs, L, label=label)
    if y is not None:
        ref, ridx, _ = oracle.layer_inputs(L)
        assert np.array_equal(ridx, idx)
        err = per_token_err(y.cpu().numpy(), ref)
        assert err <= TOL_Y, f"{label}: {err:.3e}"
    return idx


def _cases():
    return [("decode", T) for T in DECODE_T] + [("route", 9), ("route", 40)] + [("prefill", T) for T in PREFILL_T]


# logits spread over [-30, 30]: both sides of exp(-|l|) = 1/32 (l = -ln 32 =
# -3.4657), the series side down to -30 with five points within 0.5 of -12,
# the point where the naive fp32 score becomes exactly zero (-16.64), and
# large positive logits
SPREAD = [-30.0, -20.0, -16.7, -12.5, -12.2, -12.0, -11.8, -11.5, -8.0, -3.47, -3.46, -1.0, 0.0, 2.5, 15.0, 30.0]


@pytest.mark.parametrize("mode,T", _cases())
def test_scores_across_logit_range(mode, T):
    """k = E = 16: every expert is selected, so every score enters a weight;
    the logits sit within a few 1e-3 of SPREAD."""
    L = _layer(T, 16, 16, 1e-4, SPREAD)
    y, bufs = _run(L, mode)
    idx = _check(L, y, bufs, f"spread {mode} T={T}")
    lg = bufs["logits"].cpu().numpy()
    assert np.all(np.abs(lg - np.asarray(SPREAD, np.float32)) < 0.05)
    # rank order is logit order: expert 15 (l = 30) first, expert 0 (l = -30) last
    assert np.all(idx[:, 0] == 15) and np.all(idx[:, -1] == 0)
    # the weights are those of the stable score: the naive fp32 form would give
    # the experts below -16.64 a weight of exactly zero
    w = bufs["topk_w"].cpu().numpy()
    assert np.all(w[:, -1] > 0.0)


@pytest.mark.parametrize("mode,T", _cases())
def test_selection_near_minus_12(mode, T):
    """E = 64, k = 8, every logit within about 0.5 of -12 (bias -12 +-0.3, a
    router term of standard deviation 0.16): selection and weights entirely
    in the regime where log(1 + exp(l)) in fp32 is inaccurate."""
    rng = np.random.default_rng(12)
    bias = -12.0 + rng.uniform(-0.3, 0.3, size=64)
    L = _layer(T, 64, 8, 0.01, bias)
    y, bufs = _run(L, mode)
    idx = _check(L, y, bufs, f"near -12 {mode} T={T}")
    lg = bufs["logits"].cpu().numpy()
    sel = np.take_along_axis(lg, idx, axis=1)
    assert np.all((sel > -13.0) & (sel < -11.0)), (sel.min(), sel.max())
    # the weights are far from uniform: the scores differ by ~e^(dl/2)
    w = bufs["topk_w"].cpu().numpy()
    assert np.all(w[:, 0] > w[:, -1])


# ties: rows 7, 8 and 30 copy row 3, row 20 copies row 5.  Bias +40 on
# {3, 7, 8, 30} puts them on top, in ascending index order; bias +20 on
# {5, 20} makes them next.  k = 5 splits the pair {5, 20} at the selection
# boundary (5 in, 20 out); k = 6 takes both, 5 before 20.
TIE_DUP = ((3, 7), (3, 8), (3, 30), (5, 20))


def _tie_bias():
    b = np.zeros(32, np.float32)
    b[[3, 7, 8, 30]] = 40.0
    b[[5, 20]] = 20.0
    return b


@pytest.mark.parametrize("k", [5, 6])
@pytest.mark.parametrize("mode,T", _cases())
def test_bit_equal_logits_tie_to_lower_index(mode, T, k):
    L = _layer(T, 32, k, 0.05, _tie_bias(), dup=TIE_DUP)
    y, bufs = _run(L, mode)
    idx = _check(L, y, bufs, f"ties k={k} {mode} T={T}")
    lg = bufs["logits"].cpu().numpy()
    for a, b in ((3, 7), (3, 8), (3, 30), (5, 20)):
        assert np.array_equal(lg[:, a].view(np.uint32), lg[:, b].view(np.uint32))
    expect = [3, 7, 8, 30, 5, 20][:k]
    assert np.all(idx == np.asarray(expect, np.int32)), idx[:3]
    w = bufs["topk_w"].cpu().numpy()
    assert np.all(w[:, 0] == w[:, 1]) and np.all(w[:, 1] == w[:, 3])


@pytest.mark.parametrize("mode,T", _cases())
def test_natural_ties_without_bias(mode, T):
    """Duplicated router rows without a bias: the tied pairs land anywhere in
    the ranking, token by token, including across the top-k boundary."""
    dup = tuple((e, e + 1) for e in range(0, 16, 2))   # rows 2j+1 copy rows 2j
    L = _layer(T, 16, 4, 0.05, np.zeros(16, np.float32), dup=dup)
    y, bufs = _run(L, mode)
    idx = _check(L, y, bufs, f"natural ties {mode} T={T}")
    # a pair straddling the boundary keeps its lower member
    lg = bufs["logits"].cpu().numpy()
    for t in range(L.T):
        for e in range(0, 16, 2):
            if (e + 1) in idx[t]:
                assert e in idx[t]
        assert np.array_equal(lg[t, 0::2].view(np.uint32), lg[t, 1::2].view(np.uint32))
