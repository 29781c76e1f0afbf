"""The read-bandwidth probe reads every word it is given: the xor of its
per-workgroup results equals the xor of the buffer's 32-bit words."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("words,wg", [(4, 1), (1 << 20, 256), ((1 << 20) + 52, 7)])
def test_read_probe_reads_every_word(words, wg):
    import torch

    import activation_sparse_gated_gate_amd as sf
    a = np.random.default_rng(words).integers(0, 2 ** 32, words, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(a.view(np.int32)).to("cuda:0")
    out = torch.zeros(wg, dtype=torch.int32, device="cuda:0")
    s = torch.cuda.current_stream().cuda_stream
    assert sf._lib.sffn_read_probe(buf.data_ptr(), 4 * words, wg, out.data_ptr(), s) == 0
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(a)


@pytest.mark.parametrize("pat", [0, 1])
@pytest.mark.parametrize("inf", [4, 8, 16])
@pytest.mark.parametrize("ntp", [0, 1])
def test_read_probe_cfg_reads_every_word(pat, inf, ntp):
    import torch

    import activation_sparse_gated_gate_amd as sf
    words = (1 << 20) + 52
    a = np.random.default_rng(words + 7 * pat + inf).integers(0, 2 ** 32, words, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(a.view(np.int32)).to("cuda:0")
    s = torch.cuda.current_stream().cuda_stream
    for wg, nt in ((7, 256), (256, 1024), (300, 512)):
        out = torch.zeros(wg, dtype=torch.int32, device="cuda:0")
        cfg = sf.ProbeCfg(wg, nt, pat, inf, ntp)
        import ctypes
        assert sf._lib.sffn_read_probe_cfg(buf.data_ptr(), 4 * words, ctypes.byref(cfg), out.data_ptr(), s) == 0
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
        assert got == np.bitwise_xor.reduce(a), (wg, nt)


def test_latency_probe_times_every_row():
    import torch

    import activation_sparse_gated_gate_amd as sf
    nbuf = 1 << 24
    buf = torch.ones(nbuf // 4, dtype=torch.float32, device="cuda:0")
    n = 64
    offs = torch.arange(n, dtype=torch.int64, device="cuda:0") * 4096
    offs[-1] = 1 << 40   # past the buffer: reads the last row
    out = torch.zeros(n + 2, dtype=torch.int64, device="cuda:0")
    s = torch.cuda.current_stream().cuda_stream
    assert sf._lib.sffn_read_latency_probe(buf.data_ptr(), nbuf, 1024, offs.data_ptr(), n, out.data_ptr(), s) == 0
    torch.cuda.synchronize()
    v = out.cpu().numpy()
    assert (v[:n] > 0).all() and v[n] >= v[:n].sum() and v[n + 1] > 0
    ghz = v[n] / (v[n + 1] * 10.0)
    assert 0.3 < ghz < 3.5, ghz
