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
