"""GPU parity with the down matrices in a code width of their own
(ds4moe_dims.down_bits): gate/up 2-bit with down 4-bit and the reverse, on
every decode kernel class and both prefill tile forms, plus the full-size
layer with 2-bit gate/up and 4-bit down.  Bars as in test_gpu_parity."""
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


def _run_check(L, mode, dl=None, tokens=None, label=""):
    q = _q()
    dl = dl if dl is not None else q.from_layer_inputs(L)
    bufs = dl.routing_buffers(L.T)
    y = dl.forward(dl.x_tensor(L.x), q.MODE_DECODE if mode == "decode" else q.MODE_PREFILL, routing=bufs)
    torch.cuda.synchronize()
    idx = check_routing(bufs, L, label=label)
    ref, ridx, _ = oracle.layer_inputs(L, tokens=tokens)
    sel = slice(None) if tokens is None else np.asarray(tokens)
    assert np.array_equal(ridx, idx[sel])
    err = per_token_err(y.cpu().numpy()[sel], ref)
    print(f"{label}: per-token rel err {err:.3e}")
    assert err <= TOL_Y
    return dl


@pytest.mark.parametrize("gu,dn", [(2, 4), (4, 2)])
@pytest.mark.parametrize("mode,T,I", [("decode", 1, 512), ("decode", 1, 256), ("decode", 3, 512), ("decode", 4, 256),
                                      ("decode", 9, 256), ("decode", 16, 512), ("decode", 5, 128),
                                      ("prefill", 40, 256), ("prefill", 300, 256), ("prefill", 70, 128)])
def test_mixed_widths_mid(gu, dn, mode, T, I):
    """I = 512: the split one-token down; I = 128: the padded kernels (64-token
    prefill tiles, the decode down for I below 256)."""
    wl = synth.Workload("mix", 0, T=T, H=512, E=16, I=I, k=4, Is=96 if T % 2 else 0, x_dtype="bf16",
                        router_dtype="bf16", router_sigma=0.05, layer_id=0, bits=gu, bits_down=dn)
    L = synth.make_layer(wl)
    _run_check(L, mode, label=f"mix gu={gu} dn={dn} {mode} T={T} I={I}")


@pytest.fixture(scope="module")
def full_mix():
    q = _q()
    L = synth.make_layer("prefill_mix")
    return L, q.from_layer_inputs(L)


def test_mixed_full_dequant_and_sizes(full_mix):
    q = _q()
    L, dl = full_mix
    assert dl.gu_bytes == 2048 * 4096 // 256 * 84 and dl.d_bytes == 4096 * 2048 // 256 * 148
    for e in (0, 201):
        out = torch.empty(4096, 2048, dtype=torch.float32, device=dl.device)
        q.ds4moe_dequant(out, dl.down[e * dl.d_bytes:(e + 1) * dl.d_bytes], 1, 4096, 2048, 4)
        ref = oracle.dequant_f32(L.down[e], bits=4).reshape(4096, 2048)
        assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("T", [1, 4, 16])
def test_mixed_full_decode(full_mix, T):
    L0, dl = full_mix
    _run_check(synth.derive(L0, "decode1_mix", T=T), "decode", dl, label=f"mix full decode T={T}")


def test_mixed_full_prefill_all_tokens(full_mix):
    L0, dl = full_mix
    _run_check(L0, "prefill", dl, label="mix full prefill")
