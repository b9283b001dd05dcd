"""The streaming-read probe that gives the HBM read ceiling: it must read every
16-byte vector of the buffer exactly once, whatever the workgroup count.  Each
workgroup writes the XOR of the dwords it read, so the XOR of all sink words
equals the XOR of every dword of the buffer (XOR is order-free), and a vector
read twice or skipped changes it."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,n_wg", [(16, 1), (4096, 1), (4096, 300), (1 << 20, 7),
                                         ((1 << 20) + 48, 1024), (37 * (1 << 16) + 16 * 9, 4096)])
def test_read_probe_reads_every_vector_once(nbytes, n_wg):
    from quantized_routed_moe_router_amd import binding as B
    rng = np.random.default_rng(nbytes + n_wg)
    host = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32).copy()).to("cuda:0")
    sink = torch.full((n_wg,), -1, dtype=torch.int32, device="cuda:0")
    B.ds4moe_read_probe(buf, nbytes, n_wg, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)
    # a change in one dword changes the result
    host[len(host) // 2] ^= 0x80000001
    buf.copy_(torch.from_numpy(host.view(np.int32).copy()))
    B.ds4moe_read_probe(buf, nbytes, n_wg, sink)
    torch.cuda.synchronize()
    assert np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)) == np.bitwise_xor.reduce(host)
