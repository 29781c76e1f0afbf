"""GPU parity of block-granular token selection over varlen batches (RedKnot
article: min_keep per sequence; min_full_ratio / max_full_ratio bounds and a
fixed-budget top-K over 128-token blocks) against the oracle.

Bars: token scores and keep lists bit-exact, the count on the device equal to
the list length; the prefill FFN over the block keep list within relative L2
2e-3 (bf16) with un-kept rows equal to Y.
"""
import numpy as np
import pytest

import oracle
import synth

from gpu_util import rel_l2, tensor

pytestmark = pytest.mark.gpu

PAGE = dict(block=128, min_full=0.10, max_full=0.50, recent_n=128, min_keep=1)


def _sf():
    import activation_sparse_gated_gate_amd as sf
    return sf


def make_layer(w, L):
    sf = _sf()
    from gpu_util import weights_on_device
    return sf.Layer(w.d_model, w.d_ff, L, w.wtype, w.act, weights_on_device(w), layouts=sf.LAYOUT_PREFILL)


def gpu_blocks(layer, A, cu, mass, block, min_full, max_full, recent_n, min_keep):
    import torch
    sf = _sf()
    At = tensor(A)
    L = A.shape[0]
    cut = torch.from_numpy(np.asarray(cu, dtype=np.int32)).to(At.device)
    keep = torch.full((L,), -1, dtype=torch.int32, device=At.device)
    cnt = torch.full((1,), -1, dtype=torch.int32, device=At.device)
    pol = sf.make_block_policy(mass, min_full, max_full, block, recent_n, min_keep)
    layer.select_blocks(pol, At, cut, keep, cnt)
    torch.cuda.synchronize()
    n = int(cnt.item())
    scores = layer.scratch[:L * 4].view(torch.float32).cpu().numpy()
    return keep, cnt, keep[:n].cpu().numpy(), keep.cpu().numpy(), scores


def check(layer, A, cu, mass, block=128, min_full=0.10, max_full=0.50, recent_n=128, min_keep=1):
    keep_t, cnt_t, keep, full, scores = gpu_blocks(layer, A, cu, mass, block, min_full, max_full, recent_n,
                                                   min_keep)
    s_ref = oracle.token_norms(A)
    assert np.array_equal(scores.view(np.uint32), s_ref.view(np.uint32)), "token scores differ"
    ref = oracle.block_select(s_ref, cu, block=block, mass=mass, min_full=min_full, max_full=max_full,
                              recent_n=recent_n, min_keep=min_keep)
    assert np.array_equal(keep, ref), "keep lists differ (%d vs %d)" % (keep.size, ref.size)
    assert np.all(full[keep.size:] == -1), "writes past the count"
    return keep_t, cnt_t, keep


def cu_of(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


@pytest.fixture(scope="module")
def mid():
    w = synth._make_weights(synth.WT_BF16, 512, 1024, synth.ACT_SILU, (721, 722, 723))
    Y, A = synth.cfg5_activations(L=6000, d=512)
    layer = make_layer(w, 6000)
    yield w, Y, A, layer
    layer.close()


@pytest.mark.parametrize("mass", [0.0, 0.3, 0.5, 0.9, 1.0])
def test_varlen_batch_matches_oracle(mid, mass):
    w, Y, A, layer = mid
    cu = cu_of([2000, 129, 1, 128, 0, 1500, 127, 2115])
    check(layer, A, cu, mass)


def test_single_sequence_ffn_over_block_keep_list(mid):
    w, Y, A, layer = mid
    cu = cu_of([6000])
    keep_t, cnt_t, keep = check(layer, A, cu, 0.5)
    sf = _sf()
    import torch
    Yt = tensor(Y)
    X = torch.full_like(Yt, 0x7FC0)
    layer.forward(sf.make_policy("tokens"), Yt, X, idx_in=keep_t, count_in=cnt_t)
    torch.cuda.synchronize()
    Xb = X.cpu().numpy().view(np.uint16)
    ref = oracle.prefill(w, Y, keep)
    rest = np.setdiff1d(np.arange(Y.shape[0]), keep)
    assert np.array_equal(Xb[rest], Y[rest])
    assert rel_l2(synth.bf16_bits_to_f32(Xb), synth.bf16_bits_to_f32(ref)) <= 2e-3
    # whole blocks: the list is a union of few runs
    runs = 1 + int(np.count_nonzero(np.diff(keep) != 1))
    assert runs <= -(-6000 // 128) // 2 + 1


@pytest.mark.parametrize("block,min_full,max_full,recent_n,min_keep", [
    (16, 0.10, 0.50, 128, 1),      # the most blocks a sequence can have
    (128, 0.25, 0.25, 0, 0),       # a fixed budget
    (128, 0.0, 1.0, 0, 0),         # no bounds
    (4096, 0.10, 0.50, 0, 1),      # one or two blocks per sequence
    (128, 0.10, 0.50, 5000, 1),    # recent tail covering most of a sequence
    (128, 0.0, 0.0, 0, 300),       # min_keep alone
])
def test_policy_variants(mid, block, min_full, max_full, recent_n, min_keep):
    w, Y, A, layer = mid
    for cu in (cu_of([6000]), cu_of([3000, 1, 2999])):
        for mass in (0.2, 0.6):
            check(layer, A, cu, mass, block, min_full, max_full, recent_n, min_keep)


def test_degenerate_rows_ties_and_one_token_sequences(mid):
    w, Y, A, layer = mid
    L = A.shape[0]
    zero = np.zeros_like(A)
    assert check(layer, zero, cu_of([L]), 0.3)[2].size == L                 # all-zero scores: dense
    T = np.repeat(A[:1], L, axis=0)                                         # equal masses: lower blocks
    check(layer, T, cu_of([L]), 0.35, recent_n=0)
    check(layer, A, cu_of([1] * 300 + [L - 300]), 0.5)                      # many tiny sequences
    check(layer, A[:300], cu_of([1] * 300), 0.5)                             # nseq = rows


@pytest.mark.parametrize("kind", ["wide", "small_ints"])
def test_exact_and_ordered_block_masses(mid, kind):
    """Scores whose sums are all exact in fp64 take the integer block masses;
    a range wider than 2^26 between the largest and the smallest nonzero score
    takes the fp64 sums in token and rank order.  Both against the oracle, on
    a varlen batch with a ragged last block per sequence and block sizes of
    16 and 48 (blocks straddling the 64-token runs of a thread)."""
    w, Y, A, layer = mid
    L = A.shape[0]
    rng = np.random.default_rng({"wide": 31, "small_ints": 32}[kind])
    v = np.exp(6.0 * rng.standard_normal(L)) if kind == "wide" else rng.integers(0, 4, L).astype(np.float64)
    B = np.zeros_like(A)
    B[:, 7] = synth.f32_to_bf16_bits(v.astype(np.float32))   # one element per row: score = |v| exactly
    cu = cu_of([2500, 1700, 1, 1799])
    for mass in (0.0, 0.3, 0.7, 1.0):
        for block in (16, 48, 128):
            check(layer, B, cu, mass, block=block, recent_n=5)


def test_bad_offsets_stay_in_bounds(mid):
    # offsets that are not a valid partition are clamped and made ascending:
    # no fault, an ascending list of in-range tokens, the count at most rows
    w, Y, A, layer = mid
    L = A.shape[0]
    for cu in ([0, 4000, 100, 9000, -5, L], [7, 7, 3, L + 50]):
        _, _, keep, full, _ = gpu_blocks(layer, A, np.array(cu, np.int32), 0.5, **PAGE)
        assert keep.size <= L
        assert np.all(np.diff(keep) > 0) and (keep.size == 0 or (keep[0] >= 0 and keep[-1] < L))


@pytest.fixture(scope="module")
def big():
    w = synth._make_weights(synth.WT_BF16, 512, 1024, synth.ACT_SILU, (731, 732, 733))
    Y, A = synth.cfg5_activations(L=synth.CFG5_L, d=512)
    layer = make_layer(w, synth.CFG5_L)
    yield w, Y, A, layer
    layer.close()


@pytest.mark.parametrize("mass", synth.CFG5_MASS)
def test_full_length_page_policy(big, mass):
    # L = 16384 at the pages' parameters, as one sequence and as a varlen batch
    w, Y, A, layer = big
    for cu in (cu_of([synth.CFG5_L]), cu_of([8192, 4096, 2048, 1024, 512, 511, 1])):
        keep = check(layer, A, cu, mass)[2]
        print("mass %.1f, %d sequences: kept %d (%.3f)" % (mass, cu.size - 1, keep.size, keep.size / synth.CFG5_L))


def test_block_select_writes_stay_inside_the_scratch():
    # a small layer (max_rows 300) with many one- and two-token sequences, the
    # most per-sequence bookkeeping per scratch byte; 1 MiB of guard bytes
    # around the scratch must stay untouched
    import torch
    w = synth._make_weights(synth.WT_BF16, 512, 1024, synth.ACT_SILU, (741, 742, 743))
    Y, A = synth.cfg5_activations(L=300, d=512)
    layer = make_layer(w, 300)
    guard, sb = 1 << 20, layer.scratch_bytes
    big = torch.full((sb + 2 * guard,), 0xA5, dtype=torch.uint8, device="cuda:0")
    layer.scratch = big[guard:guard + sb]
    for cu in (cu_of([300]), cu_of([1] * 150 + [2] * 75), cu_of([129, 1, 170])):
        for mass in (0.3, 1.0):
            check(layer, A, cu, mass)
    torch.cuda.synchronize()
    assert bool((big[:guard] == 0xA5).all()) and bool((big[guard + sb:] == 0xA5).all()), \
        "a kernel wrote outside the scratch"
    layer.close()
