"""GPU parity of adaptive expert top-K (RedKnot article, section on adaptive
expert top-K) against the oracle: K, the ranked expert indices and their
probabilities bit-exact, on seeded router probabilities (softmax of scaled
normal logits, a per-token sharpness spread so every bucket occurs).
"""
import numpy as np
import pytest

import oracle
import synth

from gpu_util import tensor

pytestmark = pytest.mark.gpu


def gpu_select(p, tau, kmin, kmax):
    import torch

    import activation_sparse_gated_gate_amd as sf
    T = p.shape[0]
    P = tensor(p)
    # poisoned outputs: every slot must be written
    k = torch.full((T,), -7, dtype=torch.int32, device=P.device)
    idx = torch.full((T, kmax), -7, dtype=torch.int32, device=P.device)
    w = torch.full((T, kmax), float("nan"), dtype=torch.float32, device=P.device)
    sf.expert_select(P, tau, kmin, kmax, k_out=k, idx_out=idx, w_out=w)
    torch.cuda.synchronize()
    return k.cpu().numpy(), idx.cpu().numpy(), w.cpu().numpy()


def check(p, tau, kmin, kmax):
    k, idx, w = gpu_select(p, tau, kmin, kmax)
    rk, ridx, rw = oracle.expert_select(p, tau, kmin, kmax)
    assert np.array_equal(k, rk), "K differs at tokens %s" % np.nonzero(k != rk)[0][:8]
    assert np.array_equal(idx, ridx), "ranked experts differ"
    assert np.array_equal(w.view(np.uint32), rw.view(np.uint32)), "probabilities differ"
    return k


@pytest.mark.parametrize("E", synth.EXPERT_E)
def test_page_policy_small(E):
    p = synth.router_probs(1000, E, seed=611)
    k = check(p, synth.EXPERT_TAU, synth.EXPERT_KMIN, synth.EXPERT_KMAX)
    assert set(np.unique(k)) == {3, 4, 5, 6}      # the recipe reaches every bucket


@pytest.mark.parametrize("layer_from,layer_to,kmax", synth.EXPERT_DEPTH_KMAX)
def test_progressive_depth_caps(layer_from, layer_to, kmax):
    p = synth.router_probs(777, 384, seed=612 + kmax)
    k = check(p, synth.EXPERT_TAU, min(synth.EXPERT_KMIN, kmax), kmax)
    assert k.max() <= kmax


@pytest.mark.parametrize("E", [1, 7, 63, 64, 65, 100, 129, 256, 300, 511, 512, 1000, 1024])
def test_expert_counts_across_lane_widths(E):
    p = synth.router_probs(37, E, seed=620 + E)
    kmax = min(E, 16)
    for kmin in sorted({1, min(3, kmax), kmax}):
        check(p, 0.5, kmin, kmax)


@pytest.mark.parametrize("T", [0, 1, 2, 3, 4, 5, 257])
def test_ragged_token_counts(T):
    p = synth.router_probs(max(T, 1), 384, seed=630)[:T]
    if T == 0:
        k, idx, w = gpu_select(p.reshape(0, 384), 0.5, 3, 6)
        assert k.size == 0
        return
    check(p, 0.5, 3, 6)


@pytest.mark.parametrize("T", [8193, 40001])
def test_large_ragged_token_counts(T):
    p = synth.router_probs(T, 256, seed=635)
    check(p, 0.5, 3, 6)


def test_threshold_limits_and_plain_topk():
    p = synth.router_probs(500, 384, seed=640)
    assert np.all(check(p, 0.0, 3, 6) == 3)         # tau 0: the smallest bucket
    assert np.all(check(p, 2.0, 3, 6) == 6)         # unreachable tau: the largest
    assert np.all(check(p, 0.5, 6, 6) == 6)         # one bucket: plain top-6
    assert np.all(check(p, 0.5, 16, 16) == 16)


def test_ties_rank_the_lower_index_first():
    rng = np.random.default_rng(650)
    # probabilities on a coarse grid: many exact ties, zeros among them
    q = rng.integers(0, 8, size=(300, 384)).astype(np.float64)
    q[5] = 1.0                                      # a token whose experts all tie
    q[6] = 0.0
    q[6, [10, 20, 30]] = 1.0
    p = (q / np.maximum(q.sum(axis=1, keepdims=True), 1.0)).astype(np.float32)
    p[7] = -0.0                                     # signed zeros tie with +0
    p[7, ::2] = 0.0
    k = check(p, 0.5, 3, 6)
    _, idx, _ = gpu_select(p, 0.5, 3, 6)
    assert list(idx[5][:3]) == [0, 1, 2]
    assert list(idx[6][:3]) == [10, 20, 30]


def test_full_batch_16384_tokens():
    # one prefill-sized call at the page's policy, both expert counts
    for E in synth.EXPERT_E:
        p = synth.router_probs(synth.EXPERT_T, E, seed=660 + E)
        k = check(p, synth.EXPERT_TAU, synth.EXPERT_KMIN, synth.EXPERT_KMAX)
        print("E %d: mean K %.3f, bucket counts %s" % (E, k.mean(), np.bincount(k, minlength=7)[3:]))
