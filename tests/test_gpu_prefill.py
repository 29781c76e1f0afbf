"""GPU parity of the token-selective prefill path against the CPU oracle.

Bars: token scores and keep lists bit-exact; X_next within relative L2 2e-3
(bf16) overall and on the kept rows; rows that are not kept bitwise equal to Y;
mass >= 1 keeps every row.
"""
import numpy as np
import pytest

import oracle
import synth

from gpu_util import rel_l2, tensor

pytestmark = pytest.mark.gpu


def _sf():
    import activation_sparse_gated_gate_amd as sf
    return sf


def make_prefill_layer(w, L):
    sf = _sf()
    from gpu_util import weights_on_device
    return sf.Layer(w.d_model, w.d_ff, L, w.wtype, w.act, weights_on_device(w), layouts=sf.LAYOUT_PREFILL)


def gpu_select(layer, A, mass, recent, min_keep):
    import torch
    sf = _sf()
    At = tensor(A)
    L = A.shape[0]
    keep = torch.full((L,), -1, dtype=torch.int32, device=At.device)
    cnt = torch.full((1,), -1, dtype=torch.int32, device=At.device)
    pol = sf.make_policy("tokens", mass_thresh=mass, recent_n=recent, min_keep=min_keep)
    layer.select(pol, At, keep, cnt)
    torch.cuda.synchronize()
    n = int(cnt.item())
    scores = layer.scratch[:L * 4].view(torch.float32).cpu().numpy()
    return keep, cnt, keep[:n].cpu().numpy(), scores


def gpu_forward(layer, Y, keep, cnt, inplace=False):
    import torch
    sf = _sf()
    Yt = tensor(Y)
    X = Yt if inplace else torch.full_like(Yt, 0x7FC0)  # NaN pattern: every row must be written
    layer.forward(sf.make_policy("tokens"), Yt, X, idx_in=keep, count_in=cnt)
    torch.cuda.synchronize()
    return X.cpu().numpy().view(np.uint16)


def check_select(layer, A, mass, recent, mk):
    keep_t, cnt_t, keep, scores = gpu_select(layer, A, mass, recent, mk)
    s_ref = oracle.token_norms(A)
    assert np.array_equal(scores.view(np.uint32), s_ref.view(np.uint32)), "token scores differ"
    k_ref, _, _ = oracle.token_select(s_ref, mass, recent, mk)
    assert np.array_equal(keep, k_ref), "keep lists differ (%d vs %d)" % (keep.size, k_ref.size)
    return keep_t, cnt_t, keep


@pytest.fixture(scope="module")
def small():
    w = synth._make_weights(synth.WT_BF16, 512, 1024, synth.ACT_SILU, (701, 702, 703))
    Y, A = synth.cfg5_activations(L=1000, d=512)
    layer = make_prefill_layer(w, 1000)
    yield w, Y, A, layer
    layer.close()


@pytest.mark.parametrize("mass", [0.3, 0.5, 0.7, 1.0])
def test_small_prefill_matches_oracle(small, mass):
    w, Y, A, layer = small
    keep_t, cnt_t, keep = check_select(layer, A, mass, 128, 1)
    X = gpu_forward(layer, Y, keep_t, cnt_t)
    ref = oracle.prefill(w, Y, keep)
    Xf, Rf = synth.bf16_bits_to_f32(X), synth.bf16_bits_to_f32(ref)
    rest = np.setdiff1d(np.arange(Y.shape[0]), keep)
    assert np.array_equal(X[rest], Y[rest]), "un-kept rows must equal Y"
    e_all, e_kept = rel_l2(Xf, Rf), rel_l2(Xf[keep], Rf[keep])
    assert e_all <= 2e-3 and e_kept <= 2e-3, (e_all, e_kept)
    if mass >= 1.0:
        assert keep.size == Y.shape[0]


def test_small_prefill_in_place_and_mass_one_equals_dense(small):
    w, Y, A, layer = small
    keep_t, cnt_t, keep = check_select(layer, A, 0.5, 128, 1)
    Xin = gpu_forward(layer, Y, keep_t, cnt_t, inplace=True)
    Xout = gpu_forward(layer, Y, keep_t, cnt_t)
    assert np.array_equal(Xin, Xout)
    # mass = 1.0 goes through the same kernels as every row kept: bitwise equal
    kt1, ct1, k1 = check_select(layer, A, 1.0, 128, 1)
    import torch
    allk = torch.arange(Y.shape[0], dtype=torch.int32, device=kt1.device)
    allc = torch.tensor([Y.shape[0]], dtype=torch.int32, device=kt1.device)
    assert np.array_equal(gpu_forward(layer, Y, kt1, ct1), gpu_forward(layer, Y, allk, allc))


def test_selection_edge_cases(small):
    w, Y, A, layer = small
    L = A.shape[0]
    zero = np.zeros_like(A)
    assert check_select(layer, zero, 0.3, 0, 1)[2].size == L            # all-zero scores: dense
    assert check_select(layer, A, 0.3, L, 1)[2].size == L               # recent_n >= L
    one = check_select(layer, A, 0.0, 0, 1)[2]                          # only the top token
    assert one.size == 1
    assert check_select(layer, A, 0.0, 0, 37)[2].size == 37             # min_keep
    assert check_select(layer, A, 0.0, 5, 3)[2].size == 5               # recent already >= min_keep
    # ties: identical rows give identical scores; lower index first
    T = np.repeat(A[:1], L, axis=0)
    assert list(check_select(layer, T, 0.0, 0, 4)[2]) == [0, 1, 2, 3]
    assert check_select(layer, T, 0.5, 0, 1)[2].size == L // 2


@pytest.mark.parametrize("L", [1, 7, 129, 300])
def test_ragged_lengths(L):
    w = synth._make_weights(synth.WT_BF16, 256, 512, synth.ACT_SILU, (711, 712, 713))
    Y, A = synth.cfg5_activations(L=L, d=256)
    layer = make_prefill_layer(w, L)
    for mass, recent in ((0.4, 3), (0.9, 0), (1.0, 0)):
        keep_t, cnt_t, keep = check_select(layer, A, mass, recent, 1)
        X = gpu_forward(layer, Y, keep_t, cnt_t)
        ref = oracle.prefill(w, Y, keep)
        assert rel_l2(synth.bf16_bits_to_f32(X), synth.bf16_bits_to_f32(ref)) <= 2e-3
    layer.close()


# ---------------------------------------------------------------------------
# config 5: d_model 5120, d_ff 25600, L = 16384
# ---------------------------------------------------------------------------

@pytest.fixture(scope="module")
def cfg5():
    w = synth.cfg5_weights()
    Y, A = synth.cfg5_activations()
    layer = make_prefill_layer(w, synth.CFG5_L)
    yield w, Y, A, layer
    layer.close()


@pytest.mark.parametrize("mass", synth.CFG5_MASS)
def test_cfg5_selection_and_sampled_rows(cfg5, mass):
    w, Y, A, layer = cfg5
    keep_t, cnt_t, keep = check_select(layer, A, mass, synth.CFG5_RECENT, synth.CFG5_MIN_KEEP)
    X = gpu_forward(layer, Y, keep_t, cnt_t)
    rng = np.random.default_rng(int(mass * 100))
    sample = np.sort(rng.choice(keep, size=min(8, keep.size), replace=False)).astype(np.int32)
    Z = oracle.prefill_rows(w, Y, sample)
    Yk = synth.bf16_bits_to_f32(Y[sample]).astype(np.float64)
    ref = synth.bf16_bits_to_f32(oracle.bf16_rne(Yk + Z))
    assert rel_l2(synth.bf16_bits_to_f32(X[sample]), ref) <= 2e-3
    rest = np.setdiff1d(np.arange(Y.shape[0]), keep)
    assert np.array_equal(X[rest], Y[rest])
    frac = keep.size / Y.shape[0]
    print("mass %.1f kept %d (%.4f)" % (mass, keep.size, frac))


def _guarded_scratch(layer, guard=1 << 20):
    """Replace the layer's scratch by a view with 1 MiB of 0xA5 on each side."""
    import torch
    sb = layer.scratch_bytes
    big = torch.full((sb + 2 * guard,), 0xA5, dtype=torch.uint8, device="cuda:0")
    layer.scratch = big[guard:guard + sb]
    return big, guard, sb


def _guards_intact(big, guard, sb):
    import torch
    torch.cuda.synchronize()
    return bool((big[:guard] == 0xA5).all()) and bool((big[guard + sb:] == 0xA5).all())


@pytest.mark.parametrize("L", [256, 1000])
def test_prefill_writes_stay_inside_the_scratch(L):
    # the token sort once wrote its merged order 16384 keys past its chunks,
    # beyond the scratch of any layer with a smaller max_rows
    w = synth._make_weights(synth.WT_BF16, 512, 1024, synth.ACT_SILU, (721, 722, 723))
    Y, A = synth.cfg5_activations(L=L, d=512)
    layer = make_prefill_layer(w, L)
    big, guard, sb = _guarded_scratch(layer)
    keep_t, cnt_t, keep = check_select(layer, A, 0.5, 64, 1)
    X = gpu_forward(layer, Y, keep_t, cnt_t)
    assert _guards_intact(big, guard, sb), "a kernel wrote outside the scratch"
    ref = oracle.prefill(w, Y, keep)
    assert rel_l2(synth.bf16_bits_to_f32(X), synth.bf16_bits_to_f32(ref)) <= 2e-3
    layer.close()
