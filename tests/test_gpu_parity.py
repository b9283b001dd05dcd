"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.

Bars: dequantized weights, logits, top-k indices, counts, offsets and the
permutation bit-exact; top-k weights within 3e-6 relative (the router test
tolerance of the ds4 FAQ); layer output within 2e-3 per-token normwise
relative error, max_t max_j |y-r| / max_j |r|; two runs bitwise equal.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL_Y = 2e-3
TOL_W = 3e-6


def _q():
    import quantized_routed_moe_router_amd as q
    return q


def per_token_err(y, r):
    y = np.asarray(y, np.float64)
    r = np.asarray(r, np.float64)
    num = np.abs(y - r).max(axis=1)
    den = np.abs(r).max(axis=1)
    return float((num / np.maximum(den, 1e-30)).max())


def check_routing(rt, L, tokens=None, label=""):
    """rt: dict of device routing tensors for all T tokens; oracle on tokens."""
    x = L.x if L.wl.x_dtype == "f32" else oracle.bf16_to_f32(L.x)
    wr = L.router_w if L.wl.router_dtype == "f32" else oracle.bf16_to_f32(L.router_w)
    lg = oracle.logits(x, wr, L.router_bias)
    g_lg = rt["logits"].cpu().numpy()
    mism = int((g_lg.view(np.uint32) != lg.view(np.uint32)).sum())
    assert mism == 0, f"{label}: {mism} logits differ"
    idx, w, _ = oracle.topk(lg, L.wl.k)
    assert np.array_equal(rt["topk_idx"].cpu().numpy(), idx), label
    gw = rt["topk_w"].cpu().numpy()
    assert np.max(np.abs(gw - w) / np.abs(w)) <= TOL_W, label
    counts, offsets, perm = oracle.permute(idx, L.wl.E)
    assert np.array_equal(rt["counts"].cpu().numpy(), counts), label
    assert np.array_equal(rt["offsets"].cpu().numpy(), offsets), label
    assert np.array_equal(rt["perm"].cpu().numpy(), perm), label
    return idx


# ------------------------------------------------------------------ fixtures


@pytest.fixture(scope="module")
def tiny():
    q = _q()
    L = synth.make_layer("tiny")
    return L, q.from_layer_inputs(L)


@pytest.fixture(scope="session")
def full():
    q = _q()
    L = synth.make_layer("prefill")
    dl = q.from_layer_inputs(L)
    return L, dl


@pytest.fixture(scope="session")
def full_shared(full):
    q = _q()
    L0, dl0 = full
    Ls = synth.derive(L0, "skewed", T=1)
    dl = q.DeviceLayer(4096, 2048, 256, 8, 2048, q.DS4MOE_BF16, q.DS4MOE_BF16)
    dl.set_router(Ls.router_w, Ls.router_bias)
    dl.gate, dl.up, dl.down = dl0.gate, dl0.up, dl0.down
    dl.set_shared(Ls.sh_gate, Ls.sh_up, Ls.sh_down)
    return L0, dl


# ------------------------------------------------------------------ dequant


def test_dequant_bitwise_tiny(tiny):
    q = _q()
    L, dl = tiny
    E, H, I = L.wl.E, L.wl.H, L.wl.I
    for packed, canon, rows, cols in ((dl.gate, L.gate, I, H), (dl.up, L.up, I, H), (dl.down, L.down, H, I)):
        out = torch.empty(E, rows, cols, dtype=torch.float32, device=dl.device)
        q.ds4moe_dequant_q2k(out, packed, E, rows, cols)
        ref = oracle.dequant_f32(canon).reshape(E, rows, cols)
        assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_dequant_bitwise_full_sample(full):
    q = _q()
    L, dl = full
    H, I = L.wl.H, L.wl.I
    for e in (0, 77, 255):
        for packed, canon, rows, cols, nb in ((dl.gate, L.gate, I, H, dl.gu_bytes), (dl.down, L.down, H, I, dl.d_bytes)):
            out = torch.empty(rows, cols, dtype=torch.float32, device=dl.device)
            q.ds4moe_dequant_q2k(out, packed[e * nb:(e + 1) * nb], 1, rows, cols)
            ref = oracle.dequant_f32(canon[e]).reshape(rows, cols)
            assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32)), (e, rows)


def test_dequant_special_blocks():
    """Hand-built blocks (negative and subnormal d, zero block) survive pack+dequant."""
    q = _q()
    blk = np.zeros((16, 84), np.uint8)
    rng = np.random.default_rng(5)
    blk[:, :80] = rng.integers(0, 256, size=(16, 80))
    blk[0, 80:84] = [0x01, 0x00, 0x00, 0x00]          # subnormal d, zero dmin
    blk[1, 80:84] = [0x00, 0xBC, 0x00, 0x38]          # d = -1, dmin = 0.5
    blk[2, :] = 0                                     # all-zero block
    blk[3, 80:84] = [0xFF, 0x7B, 0xFF, 0x7B]          # largest finite d, dmin
    canon = blk.reshape(1, -1)                        # one matrix 16 x 256
    dev = torch.device("cuda:0")
    src = torch.from_numpy(canon).to(dev)
    packed = torch.empty(q.ds4moe_packed_bytes(16, 256), dtype=torch.uint8, device=dev)
    q.ds4moe_pack_q2k(packed, src, 1, 16, 256)
    out = torch.empty(16, 256, dtype=torch.float32, device=dev)
    q.ds4moe_dequant_q2k(out, packed, 1, 16, 256)
    ref = oracle.dequant_f32(canon).reshape(16, 256)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


# ------------------------------------------------------------------ tiny layer


@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_tiny_layer(tiny, mode):
    q = _q()
    L, dl = tiny
    x = dl.x_tensor(L.x)
    bufs = dl.routing_buffers(L.T)
    m = q.MODE_DECODE if mode == "decode" else q.MODE_PREFILL
    y = dl.forward(x, m, routing=bufs)
    torch.cuda.synchronize()
    check_routing(bufs, L, label=f"tiny/{mode}")
    ref, _, _ = oracle.layer_inputs(L)
    err = per_token_err(y.cpu().numpy(), ref)
    print(f"tiny {mode}: per-token rel err {err:.3e}")
    assert err <= TOL_Y


def test_tiny_route_only(tiny):
    L, dl = tiny
    bufs = dl.route(dl.x_tensor(L.x))
    torch.cuda.synchronize()
    check_routing(bufs, L, label="tiny/route")


@pytest.mark.parametrize("T", [1, 2, 5, 17, 63, 64, 65, 100, 257])
def test_tiny_ragged_prefill(tiny, T):
    q = _q()
    L0, dl = tiny
    L = synth.make_layer("tiny", T=T)
    bufs = dl.routing_buffers(T)
    y = dl.forward(dl.x_tensor(L.x), q.MODE_PREFILL, routing=bufs)
    torch.cuda.synchronize()
    check_routing(bufs, L, label=f"ragged T={T}")
    ref, _, _ = oracle.layer_inputs(L)
    assert per_token_err(y.cpu().numpy(), ref) <= TOL_Y


@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 9, 16])
def test_tiny_ragged_decode(tiny, T):
    """Decode at every batch-size class: T <= 4 routes inside the gate/up
    kernel (one template per T), 5..16 through the routing kernel."""
    q = _q()
    L0, dl = tiny
    L = synth.make_layer("tiny", T=T)
    bufs = dl.routing_buffers(T)
    y = dl.forward(dl.x_tensor(L.x), q.MODE_DECODE, routing=bufs)
    torch.cuda.synchronize()
    check_routing(bufs, L, label=f"ragged decode T={T}")
    ref, _, _ = oracle.layer_inputs(L)
    assert per_token_err(y.cpu().numpy(), ref) <= TOL_Y


@pytest.mark.parametrize("T", [4, 16])
def test_tiny_decode_all_tokens_one_expert(tiny, T):
    """Decode with every token sending its first choice to expert 3."""
    q = _q()
    L0, dl0 = tiny
    L = synth.make_layer("tiny", T=T)
    bias = np.zeros(L.wl.E, np.float32)
    bias[3] = 100.0
    L.router_bias = bias
    dl = q.DeviceLayer(L.wl.H, L.wl.I, L.wl.E, L.wl.k, 0, q.DS4MOE_F32, q.DS4MOE_F32)
    dl.set_router(L.router_w, bias)
    dl.gate, dl.up, dl.down = dl0.gate, dl0.up, dl0.down
    bufs = dl.routing_buffers(T)
    y = dl.forward(dl.x_tensor(L.x), q.MODE_DECODE, routing=bufs)
    torch.cuda.synchronize()
    idx = check_routing(bufs, L, label=f"decode one-expert T={T}")
    assert np.all(idx[:, 0] == 3)
    ref, _, _ = oracle.layer_inputs(L)
    assert per_token_err(y.cpu().numpy(), ref) <= TOL_Y


def test_tiny_all_tokens_one_expert(tiny):
    """A large bias on expert 3 sends every token there (several tiles), most
    experts get none."""
    q = _q()
    L0, dl0 = tiny
    T = 200
    L = synth.make_layer("tiny", T=T)
    bias = np.zeros(L.wl.E, np.float32)
    bias[3] = 100.0
    L.router_bias = bias
    dl = q.DeviceLayer(L.wl.H, L.wl.I, L.wl.E, L.wl.k, 0, q.DS4MOE_F32, q.DS4MOE_F32)
    dl.set_router(L.router_w, bias)
    dl.gate, dl.up, dl.down = dl0.gate, dl0.up, dl0.down
    for m in (q.MODE_PREFILL,):
        bufs = dl.routing_buffers(T)
        y = dl.forward(dl.x_tensor(L.x), m, routing=bufs)
        torch.cuda.synchronize()
        idx = check_routing(bufs, L, label="one-expert")
        assert np.all(idx[:, 0] == 3)
        ref, _, _ = oracle.layer_inputs(L)
        assert per_token_err(y.cpu().numpy(), ref) <= TOL_Y


@pytest.mark.parametrize("k,E,T,mode", [(1, 8, 33, "prefill"), (8, 8, 33, "prefill"), (1, 8, 4, "decode"),
                                          (8, 8, 4, "decode"), (8, 8, 12, "decode")])
def test_tiny_topk_extremes(k, E, T, mode):
    """k = 1 (weight exactly 1) and k = E (every expert selected)."""
    q = _q()
    wl = synth.Workload("tiny_k", 0, T=T, H=256, E=E, I=128, k=k, x_dtype="f32", router_dtype="f32",
                        router_sigma=0.05, layer_id=0)
    L = synth.make_layer(wl)
    dl = q.from_layer_inputs(L)
    bufs = dl.routing_buffers(L.T)
    y = dl.forward(dl.x_tensor(L.x), q.MODE_DECODE if mode == "decode" else q.MODE_PREFILL, routing=bufs)
    torch.cuda.synchronize()
    check_routing(bufs, L, label=f"k={k}")
    if k == 1:
        assert np.all(bufs["topk_w"].cpu().numpy() == 1.0)
    ref, _, _ = oracle.layer_inputs(L)
    assert per_token_err(y.cpu().numpy(), ref) <= TOL_Y


def _mid_workload(T, E=8, k=2):
    # I a multiple of 256: the prefill GEMMs take 96-token tiles
    return synth.Workload("mid", 0, T=T, H=512, E=E, I=256, k=k, x_dtype="f32", router_dtype="f32",
                          router_sigma=0.05, layer_id=0)


@pytest.mark.parametrize("T", [1, 17, 48, 97, 300, 1000])
def test_mid_wide_tiles_prefill(T):
    """Prefill with 96-token tiles: one partial n-tile, several tiles per
    expert and ragged last tiles."""
    q = _q()
    L = synth.make_layer(_mid_workload(T))
    dl = q.from_layer_inputs(L)
    bufs = dl.routing_buffers(T)
    y = dl.forward(dl.x_tensor(L.x), q.MODE_PREFILL, routing=bufs)
    torch.cuda.synchronize()
    check_routing(bufs, L, label=f"mid T={T}")
    ref, _, _ = oracle.layer_inputs(L)
    err = per_token_err(y.cpu().numpy(), ref)
    print(f"mid T={T}: per-token rel err {err:.3e}")
    assert err <= TOL_Y


# tokens per expert: tiles of 80 tokens with every live n-tile count 1..5, the
# last n-tile partial and full, and experts with one and with two tiles
FORCED_COUNTS = ([1, 16, 17, 40, 64, 79, 80, 113], [2, 15, 31, 33, 48, 65, 81, 160])


@pytest.mark.parametrize("I", [256, 512])
@pytest.mark.parametrize("counts", FORCED_COUNTS)
def test_wide_tiles_every_ntile_count(counts, I):
    """Each token is steered to a chosen expert (one-hot router rows, the
    token's own coordinate raised), so the prefill GEMMs see tiles of every
    live n-tile count on both projections, with one and with two down
    super-blocks; every token against the oracle.  A build whose instances
    miscompiled the last n-tile of the down projection's second row tile
    failed exactly this check."""
    q = _q()
    E, H = 8, 512
    T = int(sum(counts))
    wl = synth.Workload("forced", 0, T=T, H=H, E=E, I=I, k=1, x_dtype="f32", router_dtype="f32",
                        router_sigma=0.05, layer_id=0)
    L = synth.make_layer(wl)
    rng = np.random.default_rng(7000 + T + I)
    owner = rng.permutation(np.repeat(np.arange(E), counts))
    x = L.x.copy()
    x[:, :E] = 0.0
    x[np.arange(T), owner] = 6.0
    wr = np.zeros((E, H), np.float32)
    wr[np.arange(E), np.arange(E)] = 8.0
    L.x, L.router_w = np.ascontiguousarray(x), wr
    dl = q.from_layer_inputs(L)
    bufs = dl.routing_buffers(T)
    y = dl.forward(dl.x_tensor(L.x), q.MODE_PREFILL, routing=bufs)
    torch.cuda.synchronize()
    idx = check_routing(bufs, L, label=f"forced I={I}")
    assert np.array_equal(np.bincount(idx[:, 0], minlength=E), counts)
    ref, _, _ = oracle.layer_inputs(L)
    err = per_token_err(y.cpu().numpy(), ref)
    print(f"forced counts {counts} I={I}: all {T} tokens, per-token rel err {err:.3e}")
    assert err <= TOL_Y


@pytest.mark.parametrize("T,Is", [(20, 96), (200, 96), (300, 256)])
def test_mid_shared_expert_prefill(T, Is):
    """Routed layer plus a bf16 shared expert: T <= 64 on the per-wave kernels,
    larger T on the LDS-tiled GEMMs, with shared rows (Is = 96) and tokens
    that do not fill the last tile."""
    q = _q()
    wl = synth.Workload("mid_sh", 0, T=T, H=512, E=8, I=256, k=2, Is=Is, x_dtype="bf16", router_dtype="bf16",
                        router_sigma=0.05, layer_id=0)
    L = synth.make_layer(wl)
    dl = q.from_layer_inputs(L)
    bufs = dl.routing_buffers(T)
    y = dl.forward(dl.x_tensor(L.x), q.MODE_PREFILL, routing=bufs)
    torch.cuda.synchronize()
    check_routing(bufs, L, label=f"mid shared T={T}")
    ref, _, _ = oracle.layer_inputs(L)
    err = per_token_err(y.cpu().numpy(), ref)
    print(f"mid shared T={T} Is={Is}: per-token rel err {err:.3e}")
    assert err <= TOL_Y


@pytest.mark.parametrize("T,I", [(1, 256), (3, 256), (8, 256), (16, 256), (5, 128)])
def test_mid_shared_expert_decode(T, I):
    """Decode with a bf16 shared expert: its output is added by the T <= 4
    down kernel, by the reduce kernel of the two-half down path (5..16
    tokens) and by the padded down kernel (I below 256)."""
    q = _q()
    wl = synth.Workload("mid_sh_dec", 0, T=T, H=512, E=16, I=I, k=4, Is=96, x_dtype="bf16", router_dtype="bf16",
                        router_sigma=0.05, layer_id=0)
    L = synth.make_layer(wl)
    dl = q.from_layer_inputs(L)
    bufs = dl.routing_buffers(T)
    y = dl.forward(dl.x_tensor(L.x), q.MODE_DECODE, routing=bufs)
    torch.cuda.synchronize()
    check_routing(bufs, L, label=f"shared decode T={T}")
    ref, _, _ = oracle.layer_inputs(L)
    err = per_token_err(y.cpu().numpy(), ref)
    print(f"shared decode T={T} I={I}: per-token rel err {err:.3e}")
    assert err <= TOL_Y


@pytest.mark.parametrize("T,I,bits", [(1, 512, 2), (1, 1024, 2), (1, 512, 4), (3, 512, 2), (4, 1024, 4)])
def test_mid_decode_split_down(T, I, bits):
    """Batches of up to four tokens with I a multiple of 512: the down kernel
    splits each tile's reduction over two waves (one and two super-blocks per
    wave)."""
    q = _q()
    wl = synth.Workload("mid_split", 0, T=T, H=512, E=16, I=I, k=4, x_dtype="f32", router_dtype="f32",
                        router_sigma=0.05, layer_id=0, bits=bits)
    L = synth.make_layer(wl)
    dl = q.from_layer_inputs(L)
    bufs = dl.routing_buffers(T)
    y = dl.forward(dl.x_tensor(L.x), q.MODE_DECODE, routing=bufs)
    torch.cuda.synchronize()
    check_routing(bufs, L, label=f"split down T={T} I={I} bits={bits}")
    ref, _, _ = oracle.layer_inputs(L)
    err = per_token_err(y.cpu().numpy(), ref)
    print(f"split down T={T} I={I} bits={bits}: per-token rel err {err:.3e}")
    assert err <= TOL_Y


def test_mid_wide_tiles_one_expert():
    """Every token's first choice is expert 5: 300 tokens in tiles of 96, 96,
    96 and 12 for that expert, the other experts share the second choices."""
    q = _q()
    T = 300
    L = synth.make_layer(_mid_workload(T))
    bias = np.zeros(L.wl.E, np.float32)
    bias[5] = 100.0
    L.router_bias = bias
    dl = q.from_layer_inputs(L)
    dl.set_router(L.router_w, bias)
    bufs = dl.routing_buffers(T)
    y = dl.forward(dl.x_tensor(L.x), q.MODE_PREFILL, routing=bufs)
    torch.cuda.synchronize()
    idx = check_routing(bufs, L, label="mid one-expert")
    assert np.all(idx[:, 0] == 5)
    ref, _, _ = oracle.layer_inputs(L)
    assert per_token_err(y.cpu().numpy(), ref) <= TOL_Y


@pytest.mark.parametrize("T,mode", [(1, "decode"), (2, "decode"), (4, "decode"), (5, "decode"), (16, "decode"),
                                    (40, "prefill")])
def test_k16_e256_limits(T, mode):
    """The largest top-k (16) over the largest expert count (256)."""
    q = _q()
    wl = synth.Workload("lim", 0, T=T, H=256, E=256, I=128, k=16, x_dtype="f32", router_dtype="f32",
                        router_sigma=0.05, layer_id=0)
    L = synth.make_layer(wl)
    dl = q.from_layer_inputs(L)
    bufs = dl.routing_buffers(T)
    y = dl.forward(dl.x_tensor(L.x), q.MODE_DECODE if mode == "decode" else q.MODE_PREFILL, routing=bufs)
    torch.cuda.synchronize()
    check_routing(bufs, L, label=f"k16 {mode} T={T}")
    ref, _, _ = oracle.layer_inputs(L)
    assert per_token_err(y.cpu().numpy(), ref) <= TOL_Y


@pytest.mark.parametrize("T", [4096, 4100])
def test_prefill_routing_chunk_sizes(T):
    """Prefill routes in 32-token chunks up to 4096 tokens and 64-token chunks
    above: both sides of the switch, the second with a ragged last chunk."""
    q = _q()
    wl = synth.Workload("chunks", 0, T=T, H=256, E=64, I=128, k=4, x_dtype="f32", router_dtype="f32",
                        router_sigma=0.05, layer_id=0)
    L = synth.make_layer(wl)
    dl = q.from_layer_inputs(L)
    bufs = dl.routing_buffers(T)
    y = dl.forward(dl.x_tensor(L.x), q.MODE_PREFILL, routing=bufs)
    torch.cuda.synchronize()
    idx = check_routing(bufs, L, label=f"chunks T={T}")
    ref, ridx, _ = oracle.layer_inputs(L)
    assert np.array_equal(ridx, idx)
    err = per_token_err(y.cpu().numpy(), ref)
    print(f"chunks T={T}: all tokens checked, per-token rel err {err:.3e}")
    assert err <= TOL_Y


@pytest.mark.parametrize("T,mode", [(3, "decode"), (12, "decode"), (70, "prefill")])
def test_nan_token_keeps_others(T, mode):
    """A NaN in one token's activations (out of contract): its logits are NaN,
    it selects experts 0..k-1 (NaN ranks last, ties to the lower index), the
    routing stays a valid permutation, and every other token is unaffected."""
    q = _q()
    L = synth.make_layer("tiny", T=T)
    bad = T // 2
    L.x = L.x.copy()
    L.x[bad, 5] = np.nan
    dl = q.from_layer_inputs(L)
    bufs = dl.routing_buffers(T)
    y = dl.forward(dl.x_tensor(L.x), q.MODE_DECODE if mode == "decode" else q.MODE_PREFILL, routing=bufs)
    torch.cuda.synchronize()
    k, E = L.wl.k, L.wl.E
    idx = bufs["topk_idx"].cpu().numpy()
    assert np.array_equal(idx[bad], np.arange(k))
    lg = bufs["logits"].cpu().numpy()
    assert np.all(np.isnan(lg[bad]))
    counts, offsets, perm = oracle.permute(idx, E)
    assert np.array_equal(bufs["counts"].cpu().numpy(), counts)
    assert np.array_equal(bufs["perm"].cpu().numpy(), perm)
    good = [t for t in range(T) if t != bad]
    ref, ridx, _ = oracle.layer_inputs(L, tokens=good)
    assert np.array_equal(ridx, idx[good])
    ref_lg = oracle.logits(L.x[good].astype(np.float32), L.router_w, L.router_bias)
    assert np.array_equal(lg[good].view(np.uint32), ref_lg.view(np.uint32))
    assert per_token_err(y.cpu().numpy()[good], ref) <= TOL_Y


def test_nan_single_token_decode():
    """T = 1 (the one-token routing inside the gate/up kernel) with a NaN in
    the activations: logits NaN, experts 0..k-1 in rank order, and counts,
    offsets, permutation and tiles still consistent."""
    q = _q()
    wl = synth.Workload("lim1", 0, T=1, H=256, E=256, I=128, k=16, x_dtype="f32", router_dtype="f32",
                        router_sigma=0.05, layer_id=0)
    L = synth.make_layer(wl)
    L.x = L.x.copy()
    L.x[0, 7] = np.nan
    dl = q.from_layer_inputs(L)
    bufs = dl.routing_buffers(1)
    dl.forward(dl.x_tensor(L.x), q.MODE_DECODE, routing=bufs)
    torch.cuda.synchronize()
    idx = bufs["topk_idx"].cpu().numpy()
    assert np.array_equal(idx[0], np.arange(16))
    assert np.all(np.isnan(bufs["logits"].cpu().numpy()))
    counts, offsets, perm = oracle.permute(idx, 256)
    assert np.array_equal(bufs["counts"].cpu().numpy(), counts)
    assert np.array_equal(bufs["offsets"].cpu().numpy(), offsets)
    assert np.array_equal(bufs["perm"].cpu().numpy(), perm)


@pytest.mark.parametrize("mode,T,Is", [("decode", 1, 0), ("decode", 8, 96), ("prefill", 100, 96), ("prefill", 40, 0)])
def test_forward_timed_same_result_and_slots(mode, T, Is):
    """The timed entry point computes bitwise what the plain one does; the
    slots of kernels it launched are stamped after a marker recorded before
    the call, the others (the cache slots, the shared expert without one)
    keep their earlier stamps."""
    q = _q()
    B = q.binding
    wl = synth.Workload("timed", 0, T=T, H=512, E=16, I=256, k=4, Is=Is, x_dtype="bf16", router_dtype="bf16",
                        router_sigma=0.05, layer_id=0)
    L = synth.make_layer(wl)
    dl = q.from_layer_inputs(L)
    m = q.MODE_DECODE if mode == "decode" else q.MODE_PREFILL
    x = dl.x_tensor(L.x)
    y0 = dl.forward(x, m)
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * B.N_TIMED_KERNELS)]
    for e in ev:
        e.record(stream)
    marker = torch.cuda.Event(enable_timing=True)
    marker.record(stream)
    y = torch.empty(T, wl.H, dtype=torch.float32, device=dl.device)
    ws = dl.workspace(T, m)
    B.ds4moe_forward_timed(m, dl.dims, dl.weights(), x, T, y, None, ws, ws.numel(), ev, stream)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), y0.view(torch.int32))
    launched = {s for j, s in enumerate(B.KERNEL_SLOTS) if marker.elapsed_time(ev[2 * j]) >= 0.0}
    assert {"router", "gateup", "down"} <= launched
    assert not {"cache_plan", "cache_fill"} & launched
    assert ({"shared_gateup", "shared_down"} <= launched) == bool(Is)
    assert not ({"shared_gateup", "shared_down"} & launched) or Is
    # the fp16 copy of the shared weights feeds the dense GEMMs (prefill past 64 tokens)
    assert ("shared_convert" in launched) == (mode == "prefill" and bool(Is) and T > 64)
    if mode == "prefill":
        assert {"route", "permute", "combine"} <= launched
    for j, s in enumerate(B.KERNEL_SLOTS):
        if s in launched:
            assert ev[2 * j].elapsed_time(ev[2 * j + 1]) > 0.0, s


def test_prefill_zero_tokens_is_noop(tiny):
    q = _q()
    L, dl = tiny
    y = torch.full((1, L.wl.H), 7.0, device=dl.device)
    x = dl.x_tensor(L.x[:1])
    ws = dl.workspace(1, q.MODE_PREFILL)
    q.ds4moe_forward_prefill(dl.dims, dl.weights(), x, 0, y, None, ws, ws.numel())
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


# ------------------------------------------------------------------ full size


def _full_case(full, name, mode, sample=None, shared=None):
    q = _q()
    L0, dl = shared if shared is not None else full
    L = synth.derive(L0, name)
    x = dl.x_tensor(L.x)
    bufs = dl.routing_buffers(L.T)
    m = q.MODE_DECODE if mode == "decode" else q.MODE_PREFILL
    y = dl.forward(x, m, routing=bufs)
    torch.cuda.synchronize()
    idx = check_routing(bufs, L, label=name)
    toks = list(range(L.T)) if sample is None else sample(idx)
    ref, ridx, _ = oracle.layer_inputs(L, tokens=toks)
    assert np.array_equal(ridx, idx[toks])
    err = per_token_err(y.cpu().numpy()[toks], ref)
    print(f"{name}: {len(toks)} tokens checked, per-token rel err {err:.3e}")
    assert err <= TOL_Y
    return y, idx


def test_full_decode1(full):
    _full_case(full, "decode1", "decode")


@pytest.mark.parametrize("T", [2, 3, 4, 7])
def test_full_decode_small_batches(full, T):
    """Full-size decode at batch sizes between the two decode workloads."""
    q = _q()
    L0, dl = full
    L = synth.derive(L0, "decode16", T=T)
    bufs = dl.routing_buffers(T)
    y = dl.forward(dl.x_tensor(L.x), q.MODE_DECODE, routing=bufs)
    torch.cuda.synchronize()
    check_routing(bufs, L, label=f"decode T={T}")
    ref, _, _ = oracle.layer_inputs(L)
    err = per_token_err(y.cpu().numpy(), ref)
    print(f"decode T={T}: per-token rel err {err:.3e}")
    assert err <= TOL_Y


def test_full_decode16(full):
    _, idx = _full_case(full, "decode16", "decode")
    d = len(np.unique(idx))
    print(f"decode16: {d} distinct experts")
    assert 40 <= d <= 128


def test_full_prefill_all_tokens(full):
    """The 2048-token prefill chunk, every token against the oracle."""
    _full_case(full, "prefill", "prefill")


def test_full_skewed_all_tokens(full, full_shared):
    """The 8192-token Zipf-skewed prefill with the shared expert, every token
    against the oracle: the hottest expert's ~6000 tokens run through
    dozens of full tiles, the coldest expert's few through one partial tile."""
    y, idx = _full_case(full, "skewed", "prefill", shared=full_shared)
    counts = np.bincount(idx.reshape(-1), minlength=256)
    print(f"skewed loads: min {counts.min()} median {int(np.median(counts))} max {counts.max()}")
    assert counts.max() > 1000 and counts.min() < 64


def test_full_deterministic(full):
    q = _q()
    L0, dl = full
    L = synth.derive(L0, "prefill", T=512)
    x = dl.x_tensor(L.x)
    y1 = dl.forward(x, q.MODE_PREFILL).clone()
    y2 = dl.forward(x, q.MODE_PREFILL).clone()
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))
    L = synth.derive(L0, "decode16")
    x = dl.x_tensor(L.x)
    y1 = dl.forward(x, q.MODE_DECODE).clone()
    y2 = dl.forward(x, q.MODE_DECODE).clone()
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))


def test_full_route_only_matches_forward(full):
    L0, dl = full
    L = synth.derive(L0, "prefill")
    rt = dl.route(dl.x_tensor(L.x))
    torch.cuda.synchronize()
    check_routing(rt, L, label="route-only prefill")


# ------------------------------------------------------------------ graph capture


@pytest.mark.parametrize("name,T", [("decode16", 16), ("decode16", 3), ("decode1", 1), ("prefill", 300)])
def test_graph_replay_matches_eager(full, name, T):
    """A layer call captured in a HIP graph gives the eager result on every
    replay, with other eager layer calls on the same workspace in between."""
    q = _q()
    L0, dl = full
    L = synth.derive(L0, name, T=T)
    L2 = synth.derive(L0, name, T=T, batch=1)
    m = q.MODE_DECODE if name.startswith("decode") else q.MODE_PREFILL
    fwd = q.ds4moe_forward_decode if m == q.MODE_DECODE else q.ds4moe_forward_prefill
    x, x2 = dl.x_tensor(L.x), dl.x_tensor(L2.x)
    ws = torch.empty(q.ds4moe_workspace_bytes(dl.dims, T, m), dtype=torch.uint8, device=dl.device)
    y = torch.empty(T, L.wl.H, dtype=torch.float32, device=dl.device)
    y2 = torch.empty_like(y)
    w = dl.weights()
    fwd(dl.dims, w, x, T, y, None, ws, ws.numel())
    torch.cuda.synchronize()
    ref = y.clone()
    fwd(dl.dims, w, x2, T, y2, None, ws, ws.numel())
    torch.cuda.synchronize()
    ref2 = y2.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream(dl.device)
    s.wait_stream(torch.cuda.current_stream(dl.device))
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fwd(dl.dims, w, x, T, y, None, ws, ws.numel(), s)
    torch.cuda.current_stream(dl.device).wait_stream(s)
    for rep in range(3):
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), ref.view(torch.int32)), f"replay {rep}"
        fwd(dl.dims, w, x2, T, y2, None, ws, ws.numel())
        torch.cuda.synchronize()
        assert torch.equal(y2.view(torch.int32), ref2.view(torch.int32)), f"eager after replay {rep}"
    del g


@pytest.mark.parametrize("bits", [2, 4])
def test_prefill_past_the_wide_tile_window(bits):
    """T * k * I large enough (60000 * 16 * 1024) that the down projection's
    activations no longer fit the 2 GiB window of the wide-tile kernels:
    both projections fall back to the 64-token GEMMs with I a multiple of
    256 (the unpadded down instance).  Every token against the oracle."""
    q = _q()
    T = 60000
    wl = synth.Workload("window", 0, T=T, H=256, E=16, I=1024, k=16, x_dtype="f32", router_dtype="f32",
                        router_sigma=0.05, layer_id=0, bits=bits)
    L = synth.make_layer(wl)
    dl = q.from_layer_inputs(L)
    A = T * wl.k
    assert 2 * A * wl.I + 4 * A * (wl.I // 16) > (1 << 31)     # past the window
    bufs = dl.routing_buffers(T)
    y = dl.forward(dl.x_tensor(L.x), q.MODE_PREFILL, routing=bufs)
    torch.cuda.synchronize()
    idx = check_routing(bufs, L, label=f"window bits={bits}")
    ref, ridx, _ = oracle.layer_inputs(L)
    assert np.array_equal(ridx, idx)
    err = per_token_err(y.cpu().numpy(), ref)
    print(f"window bits={bits}: all {T} tokens, per-token rel err {err:.3e}")
    assert err <= TOL_Y


# Per-token activation scales far outside the fp16 range (x is bf16 on the
# boundary, whose range is that of fp32): each token enters the fp16 operands
# pre-scaled by a power of two, so scales from 1e-15 to 1e12 within one batch
# meet the same bar as unit-scale tokens (y scales as x^2: up to ~1e24).
ACT_SCALES = [1e-15, 1e-8, 3e-3, 1.0, 300.0, 6e4, 2e6, 1e12]


@pytest.mark.parametrize("mode,T", [("decode", 1), ("decode", 3), ("decode", 8), ("decode", 16), ("prefill", 40),
                                    ("prefill", 100)])
def test_activation_range(mode, T):
    """Decode at every batch class and prefill on both shared-expert kernel
    forms (T <= 64 per-wave, T > 64 LDS-tiled), tokens cycling through
    ACT_SCALES (T = 1: the largest)."""
    q = _q()
    wl = synth.Workload("range", 0, T=T, H=512, E=16, I=256, k=4, Is=96, x_dtype="bf16", router_dtype="bf16",
                        router_sigma=0.05, layer_id=0)
    L = synth.make_layer(wl)
    xf = oracle.bf16_to_f32(L.x).astype(np.float64)
    sc = np.array([ACT_SCALES[(t + (len(ACT_SCALES) - 1 if T == 1 else 0)) % len(ACT_SCALES)] for t in range(T)])
    L.x = synth.f32_to_bf16_bits((xf * sc[:, None]).astype(np.float32))
    dl = q.from_layer_inputs(L)
    bufs = dl.routing_buffers(T)
    y = dl.forward(dl.x_tensor(L.x), q.MODE_DECODE if mode == "decode" else q.MODE_PREFILL, routing=bufs)
    torch.cuda.synchronize()
    check_routing(bufs, L, label=f"range {mode} T={T}")
    ref, _, _ = oracle.layer_inputs(L)
    yy = y.cpu().numpy()
    assert np.all(np.isfinite(yy)) and np.all(np.isfinite(ref))
    err = per_token_err(yy, ref)
    print(f"range {mode} T={T}: per-token rel err {err:.3e}, |y| from {np.abs(ref).max(axis=1).min():.2e} "
          f"to {np.abs(ref).max(axis=1).max():.2e}")
    assert err <= TOL_Y
