"""sffn_forward_noalloc (the forward on the library's built-in scratch, for
callers that cannot allocate) against sffn_forward on a caller-owned scratch:
identical outputs and lists, bit for bit, on calls in a row where each call has
fewer rows than the one before; a layer whose scratch exceeds the built-in
array is refused before any launch.
"""
import numpy as np
import pytest

import synth

from gpu_util import make_layer, tensor

pytestmark = pytest.mark.gpu


def _sf():
    import activation_sparse_gated_gate_amd as sf
    return sf


def _decode_pair(layer, pol, x):
    """(y, idx, count) from sffn_forward and from sffn_forward_noalloc."""
    import torch
    xt = tensor(np.ascontiguousarray(x, np.float32))
    f = layer.desc.d_ff
    out = []
    for noalloc in (False, True):
        y = torch.full_like(xt, float("nan"))
        idx = torch.full((f,), -1, dtype=torch.int32, device=xt.device)
        cnt = torch.full((1,), -1, dtype=torch.int32, device=xt.device)
        if noalloc:
            layer.forward_noalloc(pol, xt, y, idx_out=idx, count_out=cnt)
        else:
            layer.forward(pol, xt, y, idx_out=idx, count_out=cnt)
        torch.cuda.synchronize()
        n = int(cnt.item())
        out.append((y.cpu().numpy(), idx[:n].cpu().numpy(), n))
    return out


def _same(a, b):
    assert a[2] == b[2] and np.array_equal(a[1], b[1]), "selected lists differ"
    assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32)), "outputs differ"


def test_noalloc_decode_matches_forward_on_shrinking_batches():
    sf = _sf()
    assert sf.sffn_noalloc_scratch_bytes() == 80 << 20
    w = synth._make_weights(synth.WT_BF16, 1024, 2816, synth.ACT_SILU, (1951, 1952, 1953))
    x = synth.round_to_bf16(synth.normal_f32(1954, (16, 1024)))
    layer = make_layer(w, 16, rmsnorm=True, residual=True, layouts=sf.LAYOUT_DECODE | sf.LAYOUT_BATCH)
    pol = sf.make_policy("thresh", theta=synth.gate_threshold_for_active_fraction(0.1), use_union=True)
    for rows in (16, 5, 1):   # MFMA tiles, the device's path choice, the batch-1 kernel
        a, b = _decode_pair(layer, pol, x[:rows])
        _same(a, b)
    layer.close()


def test_noalloc_int4_topk_matches_forward():
    sf = _sf()
    w = synth._make_weights(synth.WT_I4, 2048, 2816, synth.ACT_SILU, (1961, 1962, 1963))
    x = synth.normal_f32(1964, (8, 2048))
    layer = make_layer(w, 8)
    pol = sf.make_policy("topk", topk_k=479, use_union=True)
    for rows in (8, 1):
        a, b = _decode_pair(layer, pol, x[:rows])
        _same(a, b)
    layer.close()


def test_noalloc_prefill_matches_forward():
    import torch
    sf = _sf()
    from gpu_util import weights_on_device
    w = synth._make_weights(synth.WT_BF16, 512, 1024, synth.ACT_SILU, (1971, 1972, 1973))
    Y, A = synth.cfg5_activations(L=1000, d=512)
    layer = sf.Layer(512, 1024, 1000, w.wtype, w.act, weights_on_device(w), layouts=sf.LAYOUT_PREFILL)
    for L in (1000, 300):
        At, Yt = tensor(A[:L]), tensor(Y[:L])
        keep = torch.full((L,), -1, dtype=torch.int32, device="cuda:0")
        cnt = torch.full((1,), -1, dtype=torch.int32, device="cuda:0")
        layer.select(sf.make_policy("tokens", mass_thresh=0.5, recent_n=32, min_keep=1), At, keep, cnt)
        pol = sf.make_policy("tokens")
        X1 = torch.full_like(Yt, 0x7FC0)
        X2 = torch.full_like(Yt, 0x7FC0)
        layer.forward(pol, Yt, X1, idx_in=keep, count_in=cnt)
        layer.forward_noalloc(pol, Yt, X2, idx_in=keep, count_in=cnt)
        torch.cuda.synchronize()
        assert np.array_equal(X1.cpu().numpy(), X2.cpu().numpy())
    layer.close()


def test_noalloc_refuses_a_layer_whose_scratch_exceeds_the_array():
    import torch
    sf = _sf()
    d, f, L = 256, 25600, 16384          # prefill scratch holds H: L x d_ff bf16 = 839 MB
    z = torch.zeros(f * d, dtype=torch.int16, device="cuda:0")
    layer = sf.Layer(d, f, L, sf.W_BF16, sf.ACT_SILU, {"w_gate": z, "w_up": z, "w_down": z},
                     layouts=sf.LAYOUT_PREFILL)
    assert layer.scratch_bytes > sf.sffn_noalloc_scratch_bytes()
    Yt = torch.zeros((8, d), dtype=torch.int16, device="cuda:0")
    keep = torch.arange(8, dtype=torch.int32, device="cuda:0")
    cnt = torch.tensor([8], dtype=torch.int32, device="cuda:0")
    with pytest.raises(sf.SffnError) as e:
        layer.forward_noalloc(sf.make_policy("tokens"), Yt, Yt, idx_in=keep, count_in=cnt)
    assert e.value.status == sf.SFFN_ERR_WORKSPACE
    layer.close()
