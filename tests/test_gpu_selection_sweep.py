"""Seeded randomized parity of the token selection (both of its paths) and of
the block-granular selection against the oracle: lengths from 1 to 16384 (the
16 workgroups of the sorted path included), scores with a lognormal spread,
small integers with ties and zeros, all equal, a range far beyond 2^26, a few
tiny rows among ordinary ones, and zeros among a narrow spread; random mass,
recent_n and min_keep; random varlen splits and block sizes 16 / 48 / 128.
Keep lists bit-exact, nothing written past the count."""
import numpy as np
import pytest

import oracle
import synth

from gpu_util import tensor, weights_on_device

pytestmark = pytest.mark.gpu


def _scores(rng, kind, L):
    if kind == 0:
        return 71.6 * np.exp(rng.standard_normal(L))
    if kind == 1:
        return rng.integers(0, 5, L).astype(np.float64)
    if kind == 2:
        return np.full(L, float(rng.uniform(0.01, 100)))
    if kind == 3:
        return np.exp(rng.uniform(-20, 20, L))
    if kind == 4:
        v = 71.6 * np.exp(rng.standard_normal(L))
        v[rng.integers(0, L, max(1, L // 50))] *= 2.0 ** -30
        return v
    v = np.exp(0.3 * rng.standard_normal(L))
    v[rng.integers(0, L, max(1, L // 10))] = 0.0
    return v


def test_randomized_selection_sweep():
    import torch
    import activation_sparse_gated_gate_amd as sf
    d, Lmax = 256, 16384
    w = synth._make_weights(synth.WT_BF16, d, 512, synth.ACT_SILU, (901, 902, 903))
    layer = sf.Layer(d, 512, Lmax, w.wtype, w.act, weights_on_device(w), layouts=sf.LAYOUT_PREFILL)
    rng = np.random.default_rng(2024)
    keep = torch.full((Lmax,), -1, dtype=torch.int32, device="cuda:0")
    cnt = torch.full((1,), -1, dtype=torch.int32, device="cuda:0")
    paths = {1: 0, 2: 0}
    for trial in range(120):
        L = int(rng.choice([1, 2, 15, 16, 17, 1000, 1023, 1024, 1025, 3000, 8191, 16384,
                            int(rng.integers(1, Lmax + 1))]))
        kind = trial % 6
        A = np.zeros((L, d), np.uint16)
        A[:, 5] = synth.f32_to_bf16_bits(_scores(rng, kind, L).astype(np.float32))   # score = |value| exactly
        mass = float(rng.choice([0.0, 0.05, 0.3, 0.5, 0.77, 0.999, 1.0, float(rng.uniform())]))
        recent = int(rng.choice([0, 1, 7, 128, L + 3]))
        mk = int(rng.choice([0, 1, 2, 40, L]))
        At = tensor(A)
        s_ref = oracle.token_norms(A)
        keep.fill_(-1)
        cnt.fill_(-1)
        layer.select(sf.make_policy("tokens", mass_thresh=mass, recent_n=recent, min_keep=mk), At, keep, cnt)
        torch.cuda.synchronize()
        n = int(cnt.item())
        ref = oracle.token_select(s_ref, mass, recent, mk)[0]
        case = (trial, kind, L, mass, recent, mk)
        assert np.array_equal(keep[:n].cpu().numpy(), ref), ("token", case, n, ref.size)
        assert n == L or bool((keep[n:L] == -1).all()), ("token writes past the count", case)
        paths[layer.token_select_path()] += 1
        if L >= 16:
            ncut = min(int(rng.integers(0, 6)), L - 1)
            cuts = np.sort(rng.choice(np.arange(1, L), size=ncut, replace=False))
            cu = np.concatenate([[0], cuts, [L]]).astype(np.int32)
            blk = int(rng.choice([16, 48, 128]))
            keep.fill_(-1)
            cnt.fill_(-1)
            layer.select_blocks(sf.make_block_policy(mass_thresh=mass, block=blk, recent_n=recent, min_keep=mk),
                                At, torch.from_numpy(cu).to("cuda:0"), keep, cnt)
            torch.cuda.synchronize()
            n = int(cnt.item())
            ref = oracle.block_select(s_ref, cu, block=blk, mass=mass, min_full=0.10, max_full=0.50,
                                      recent_n=recent, min_keep=mk)
            assert np.array_equal(keep[:n].cpu().numpy(), ref), ("block", case, blk, cu.tolist(), n, ref.size)
    assert paths[1] > 20 and paths[2] > 20, paths   # both token-selection paths exercised
    layer.close()
