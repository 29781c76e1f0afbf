"""GPU parity of neuron reordering by activation frequency (WiSparse notes,
section 5): the activation counts, and layers created with a neuron
permutation on the batch-1, batched and prefill paths.

Bars: counts bit-exact (integers); a permuted layer's g' equal bit for bit to
the oracle's g' of the original layer taken in the new order, its selected
set equal to the oracle's through the permutation, its outputs within the
bf16 tolerance of the oracle on the original weights.
"""
import numpy as np
import pytest

import oracle
import synth

from gpu_util import make_layer, rel_l2, run_decode, scratch_views, tensor, weights_on_device

pytestmark = pytest.mark.gpu


def _sf():
    import activation_sparse_gated_gate_amd as sf
    return sf


def test_neuron_counts_match_bincount():
    import torch
    sf = _sf()
    f = 11008
    rng = np.random.default_rng(11)
    counts = torch.zeros(f, dtype=torch.int32, device="cuda:0")
    ref = np.zeros(f, np.int64)
    for n in (0, 1, 1100, 5000, f):
        lst = np.sort(rng.choice(f, n, replace=False)).astype(np.int32)
        idx = torch.full((f,), -1, dtype=torch.int32, device="cuda:0")
        if n:
            idx[:n] = tensor(lst)
        cnt = tensor(np.array([n], np.int32))
        sf.neuron_counts(idx, cnt, counts)
        ref += np.bincount(lst, minlength=f)
    torch.cuda.synchronize()
    assert np.array_equal(counts.cpu().numpy(), ref.astype(np.int32))


def _counts_from_oracle(w, X, bias):
    c = np.zeros(w.d_ff, np.int32)
    for t in range(X.shape[0]):
        c[oracle.decode(w, X[t:t + 1], mode="exact", bias=bias)["idx"]] += 1
    return c


def _permuted_layer(w, perm, max_rows, layouts=None):
    sf = _sf()
    return sf.Layer(w.d_model, w.d_ff, max_rows, w.wtype, w.act, weights_on_device(w),
                    layouts=layouts or sf.LAYOUT_DECODE, perm=tensor(perm.astype(np.int32)))


@pytest.fixture(scope="module")
def relu_layer():
    w = synth.skewed_weights(synth.WT_BF16, 1024, 2816, synth.ACT_RELU, (961, 962, 963, 964))
    X = synth.round_to_bf16(synth.normal_f32(965, (24, 1024)))
    b = synth.gate_offset_for_active_fraction(0.1)
    return w, X, b


@pytest.mark.parametrize("order", ["balance", "cluster", "random"])
def test_permuted_layer_batch1(relu_layer, order):
    sf = _sf()
    w, X, b = relu_layer
    f = w.d_ff
    if order == "random":
        perm = np.random.default_rng(5).permutation(f).astype(np.int32)
    else:
        counts = _counts_from_oracle(w, X[:16], b)
        perm = oracle.frequency_order(counts, order, sf.decode_block_rows(f))
    layer = _permuted_layer(w, perm, 1)
    pol = sf.make_policy("exact", gate_bias=b)
    for t in range(16, 24):
        x = X[t:t + 1]
        y, idx, n = run_decode(layer, pol, x)
        ref = oracle.decode(w, x, mode="exact", bias=b)
        _, g, _ = scratch_views(layer, 1)
        assert np.array_equal(g.cpu().numpy()[0].view(np.uint32), ref["g"][0][perm].view(np.uint32))
        assert np.array_equal(np.sort(perm[idx]), ref["idx"]), "selected sets differ through the permutation"
        assert np.all(np.diff(idx) > 0)
        assert rel_l2(y, ref["y"]) <= 2e-3
    layer.close()


def test_permuted_layer_batched_tiles_and_gather():
    sf = _sf()
    w = synth.skewed_weights(synth.WT_BF16, 1024, 2816, synth.ACT_SILU, (971, 972, 973, 974))
    X = synth.round_to_bf16(synth.normal_f32(975, (16, 1024)))
    theta = synth.gate_threshold_for_active_fraction(0.05)
    c = np.zeros(w.d_ff, np.int32)
    for t in range(8):
        c[oracle.decode(w, X[t:t + 1], mode="thresh", theta=theta)["idx"]] += 1
    perm = oracle.frequency_order(c, "cluster")
    layer = _permuted_layer(w, perm, 8, layouts=sf.LAYOUT_DECODE | sf.LAYOUT_BATCH)
    x = X[8:16]
    ref = oracle.decode(w, x, mode="thresh", theta=theta, union=True)
    for path in (1, 2):   # MFMA tiles, row gather
        pol = sf.make_policy("thresh", theta=theta, use_union=True, batch_path=path)
        y, idx, n = run_decode(layer, pol, x)
        _, g, _ = scratch_views(layer, 8)
        assert np.array_equal(g.cpu().numpy().view(np.uint32), ref["g"][:, perm].view(np.uint32))
        assert np.array_equal(np.sort(perm[idx]), ref["idx"])
        assert rel_l2(y, ref["y"]) <= 2e-3, path
    layer.close()


def test_permuted_layer_prefill():
    import torch
    sf = _sf()
    w = synth.skewed_weights(synth.WT_BF16, 512, 1024, synth.ACT_SILU, (981, 982, 983, 984))
    Y, A = synth.cfg5_activations(L=600, d=512)
    perm = np.random.default_rng(9).permutation(w.d_ff).astype(np.int32)
    layer = _permuted_layer(w, perm, 600, layouts=sf.LAYOUT_PREFILL)
    keep = torch.full((600,), -1, dtype=torch.int32, device="cuda:0")
    cnt = torch.full((1,), -1, dtype=torch.int32, device="cuda:0")
    layer.select(sf.make_policy("tokens", mass_thresh=0.5, recent_n=128, min_keep=1), tensor(A), keep, cnt)
    Yt = tensor(Y)
    X = torch.full_like(Yt, 0x7FC0)
    layer.forward(sf.make_policy("tokens"), Yt, X, idx_in=keep, count_in=cnt)
    torch.cuda.synchronize()
    n = int(cnt.item())
    kept = keep[:n].cpu().numpy()
    k_ref, _, _ = oracle.token_select(oracle.token_norms(A), 0.5, 128, 1)
    assert np.array_equal(kept, k_ref)
    ref = oracle.prefill(w, Y, kept)
    Xn = X.cpu().numpy().view(np.uint16)
    assert rel_l2(synth.bf16_bits_to_f32(Xn), synth.bf16_bits_to_f32(ref)) <= 2e-3
    layer.close()


def test_permuted_layer_same_output_as_the_plain_layer_up_to_order():
    # the permuted layer and the plain layer select the same neurons and agree
    # within the fp32 summation-order difference of the down projection
    sf = _sf()
    w = synth.skewed_weights(synth.WT_F32, 512, 1408, synth.ACT_RELU, (991, 992, 993, 994))
    x = synth.normal_f32(995, (1, 512))
    b = synth.gate_offset_for_active_fraction(0.2)
    perm = np.random.default_rng(3).permutation(1408).astype(np.int32)
    plain = make_layer(w, 1)
    perml = _permuted_layer(w, perm, 1)
    pol = sf.make_policy("exact", gate_bias=b)
    y0, i0, _ = run_decode(plain, pol, x)
    y1, i1, _ = run_decode(perml, pol, x)
    assert np.array_equal(np.sort(perm[i1]), i0)
    assert rel_l2(y1, y0) <= 2e-6
    plain.close()
    perml.close()
