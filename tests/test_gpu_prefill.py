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
    """keep / cnt: device tensors, or None for the selection left in the scratch."""
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


def _rows_with_scores(v, d=256):
    """Attention rows whose norm is exactly |v_i| (bf16): one nonzero element
    per row (its square and square root are exact in fp32)."""
    A = np.zeros((v.size, d), np.uint16)
    A[:, 3] = synth.f32_to_bf16_bits(v.astype(np.float32))
    return A


@pytest.fixture(scope="module")
def mid():
    w = synth._make_weights(synth.WT_BF16, 256, 512, synth.ACT_SILU, (721, 722, 723))
    layer = make_prefill_layer(w, 3000)
    yield layer
    layer.close()


@pytest.mark.parametrize("kind", ["lognormal", "small_ints", "equal", "wide"])
def test_exact_mass_and_sorted_paths(mid, kind):
    """Both paths of the selection against the oracle, keep lists bit-exact.
    Scores whose partial sums are all exact in fp64 (range at most 2^29 and
    total at most 2^53 ulps of the smallest nonzero score, with at most 2^26
    between the largest and the smallest nonzero score) take the exact-mass
    radix select, ties at the threshold included; a wider range takes the sort.
    3000 tokens: three rounds of 1024 and a ragged tail."""
    rng = np.random.default_rng({"lognormal": 1, "small_ints": 2, "equal": 3, "wide": 4}[kind])
    L = 3000
    v = {"lognormal": lambda: 71.6 * np.exp(rng.standard_normal(L)),
         "small_ints": lambda: rng.integers(0, 5, L).astype(np.float64),
         "equal": lambda: np.full(L, 3.25),
         "wide": lambda: np.exp(6.0 * rng.standard_normal(L))}[kind]()
    A = _rows_with_scores(v)
    for mass, recent, mk in ((0.3, 0, 1), (0.5, 16, 1), (0.77, 5, 3), (0.999, 0, 1), (1.0, 0, 1),
                             (0.0, 0, 1), (0.05, 0, 200)):
        keep = check_select(mid, A, mass, recent, mk)[2]
        path = mid.token_select_path()
        if mass >= 1.0:
            assert path == 1, (kind, mass)              # every token, whatever the scores
        elif kind == "wide":
            assert path == 2, (kind, mass)              # the range alone rules the exact path out
        elif mass == 0.0:
            assert path == 2, (kind, mass)              # empty prefix, min_keep from the sorted order
        elif mk <= 3:
            assert path == 1, (kind, mass, recent, mk)  # mk = 200 may exceed the prefix: either path


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


# The bar is the relative L2 error over all compared rows (2e-3 for bf16).  A
# single row varies around it: rounding X_next to bf16 alone costs about
# 2^-7 / sqrt(12) * 0.74 = 1.7e-3 relative RMS, and H is stored in bf16.  Each
# row is also held to a looser bound, which a wrong or unwritten tile (an O(1)
# error) cannot meet.
ROW_SANITY = 5e-3


def _one_row_per_block(keep, block, seed):
    """One kept token from every run of `block` consecutive positions of the
    keep list (the GEMMs' M-tiles: 128 rows for the small tiles, 256 for the
    large ones, so every tile of either kind is sampled, the last partial one
    included)."""
    rng = np.random.default_rng(seed)
    return np.array([keep[rng.integers(b, min(b + block, keep.size))] for b in range(0, keep.size, block)],
                    np.int32)


@pytest.mark.parametrize("mass", synth.CFG5_MASS)
def test_cfg5_selection_and_every_tile(cfg5, mass):
    """Full shape: keep list bit-exact; every kept row written and finite (X
    starts NaN-filled); one row of every 128-row block of the keep list
    compared with the oracle; un-kept rows bitwise equal to Y."""
    w, Y, A, layer = cfg5
    keep_t, cnt_t, keep = check_select(layer, A, mass, synth.CFG5_RECENT, synth.CFG5_MIN_KEEP)
    # the workload's scores keep every partial sum exact: no sort
    assert layer.token_select_path() == 1
    X = gpu_forward(layer, Y, keep_t, cnt_t)
    Xk = synth.bf16_bits_to_f32(X[keep])
    assert np.isfinite(Xk).all(), "kept rows not written (NaN fill left) or non-finite"
    sample = _one_row_per_block(keep, 128, int(mass * 100))
    Z = oracle.prefill_rows(w, Y, sample)
    Yk = synth.bf16_bits_to_f32(Y[sample]).astype(np.float64)
    ref = synth.bf16_bits_to_f32(oracle.bf16_rne(Yk + Z))
    got = synth.bf16_bits_to_f32(X[sample])
    errs = [rel_l2(got[i], ref[i]) for i in range(sample.size)]
    assert rel_l2(got, ref) <= 2e-3, rel_l2(got, ref)
    assert max(errs) <= ROW_SANITY, (max(errs), int(sample[int(np.argmax(errs))]))
    rest = np.setdiff1d(np.arange(Y.shape[0]), keep)
    assert np.array_equal(X[rest], Y[rest])
    frac = keep.size / Y.shape[0]
    print("mass %.1f kept %d (%.4f), %d rows compared, worst %.3g" % (mass, keep.size, frac, sample.size,
                                                                     max(errs)))


@pytest.mark.parametrize("mass", [0.3, 0.7])
def test_cfg5_sorted_path_full_length(cfg5, mass):
    """Full length through the sorted path: 100 attention rows scaled by 2^-40
    (exact in bf16) put more than 2^26 between the largest and the smallest
    score, so the exact-mass select gives way to the sort, whose 16 workgroups
    meet at two device-scope arrival counters.  Keep list bit-exact."""
    w, Y, A, layer = cfg5
    A2 = A.copy()
    rows = np.arange(0, A.shape[0], A.shape[0] // 100)[:100]
    A2[rows] = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(A[rows]) * np.float32(2.0 ** -40))
    check_select(layer, A2, mass, synth.CFG5_RECENT, synth.CFG5_MIN_KEEP)
    assert layer.token_select_path() == 2


@pytest.mark.parametrize("M", [2048, 1800, 1000])
def test_large_tile_down_projection_every_row(M):
    """d_model 5120 (20 column tiles of 256): 2048 and 1800 kept rows give 8 row
    tiles of 256, 160 large tiles, at least half of the compute units, which
    opens the 256 x 256 down-projection tiles; 1000 rows (80 large tiles) run
    the 128 x 256 ones.  Every row is compared with the oracle (the keep list
    is given by the caller, a seeded random subset with a ragged last tile)."""
    import torch
    w = synth._make_weights(synth.WT_BF16, 5120, 512, synth.ACT_SILU, (741, 742, 743))
    L = 2048
    Y, _ = synth.cfg5_activations(L=L, d=5120)
    rng = np.random.default_rng(744 + M)
    keep = np.sort(rng.choice(L, size=M, replace=False)).astype(np.int32)
    layer = make_prefill_layer(w, L)
    kt = torch.from_numpy(keep).to("cuda:0")
    ct = torch.tensor([M], dtype=torch.int32, device="cuda:0")
    X = gpu_forward(layer, Y, kt, ct)
    ref = oracle.prefill(w, Y, keep)
    Xf, Rf = synth.bf16_bits_to_f32(X), synth.bf16_bits_to_f32(ref)
    assert np.isfinite(Xf[keep]).all()
    errs = np.array([rel_l2(Xf[i], Rf[i]) for i in keep])
    assert rel_l2(Xf[keep], Rf[keep]) <= 2e-3, rel_l2(Xf[keep], Rf[keep])
    assert errs.max() <= ROW_SANITY, (errs.max(), int(keep[int(np.argmax(errs))]))
    rest = np.setdiff1d(np.arange(L), keep)
    assert np.array_equal(X[rest], Y[rest])
    layer.close()


def _down_split(M, d, f, hrows, units):
    """The k ranges the down projection splits into for M kept rows: 0 for
    256 x 256 tiles, 1 for 128 x 256 tiles, else S (the kernel's rule restated
    so that a test can assert which path it covers)."""
    tiles = -(-M // 256) * (d // 256)
    if tiles >= units // 2:
        return 0
    best, br, bs = 1, 0, 0
    for S in range(2, 9):
        if f % (32 * S) or S * M * d * 4 > (hrows - M) * f * 2:
            continue
        r = -(-tiles * S // units)
        if bs == 0 or r * bs < br * S:
            best, br, bs = S, r, S
    return best


@pytest.mark.parametrize("d,f,L,M", [(256, 4096, 512, 200), (512, 4096, 600, 300), (1024, 2048, 1500, 257)])
def test_split_k_down_projection_every_row(d, f, L, M):
    """Few kept rows with room for the partial sums past them in H: the down
    projection splits its k range over several 256 x 256 workgroups and adds
    the partial sums in a fixed order (a ragged last row tile).  Every row is
    compared with the oracle, and a second run gives the same bits."""
    import torch
    units = torch.cuda.get_device_properties(0).multi_processor_count
    assert _down_split(M, d, f, L, units) >= 2
    w = synth._make_weights(synth.WT_BF16, d, f, synth.ACT_SILU, (761, 762, 763))
    Y, _ = synth.cfg5_activations(L=L, d=d)
    rng = np.random.default_rng(764 + M)
    keep = np.sort(rng.choice(L, size=M, replace=False)).astype(np.int32)
    layer = make_prefill_layer(w, L)
    kt = torch.from_numpy(keep).to("cuda:0")
    ct = torch.tensor([M], dtype=torch.int32, device="cuda:0")
    X = gpu_forward(layer, Y, kt, ct)
    assert np.array_equal(gpu_forward(layer, Y, kt, ct), X)
    ref = oracle.prefill(w, Y, keep)
    Xf, Rf = synth.bf16_bits_to_f32(X), synth.bf16_bits_to_f32(ref)
    assert np.isfinite(Xf[keep]).all()
    errs = np.array([rel_l2(Xf[i], Rf[i]) for i in keep])
    assert rel_l2(Xf[keep], Rf[keep]) <= 2e-3, rel_l2(Xf[keep], Rf[keep])
    assert errs.max() <= ROW_SANITY, (errs.max(), int(keep[int(np.argmax(errs))]))
    rest = np.setdiff1d(np.arange(L), keep)
    assert np.array_equal(X[rest], Y[rest])
    layer.close()


def test_forward_without_a_list_uses_the_last_selection(small):
    """sffn_forward(TOKENS) with no keep list runs on the selection the last
    sffn_select or sffn_select_blocks call left in the same scratch."""
    import torch
    sf = _sf()
    w, Y, A, layer = small
    keep_t, cnt_t, keep = check_select(layer, A, 0.5, 64, 1)
    X1 = gpu_forward(layer, Y, keep_t, cnt_t)
    X0 = gpu_forward(layer, Y, None, None)
    assert np.array_equal(X0, X1)
    # a block selection replaces it
    cu = torch.tensor([0, 600, 1000], dtype=torch.int32, device="cuda:0")
    bk = torch.full((1000,), -1, dtype=torch.int32, device="cuda:0")
    bc = torch.full((1,), -1, dtype=torch.int32, device="cuda:0")
    layer.select_blocks(sf.make_block_policy(mass_thresh=0.3, block=16, recent_n=16), tensor(A), cu, bk, bc)
    Xb = gpu_forward(layer, Y, bk, bc)
    assert np.array_equal(gpu_forward(layer, Y, None, None), Xb)
    # one of the two pointers alone is refused
    with pytest.raises(sf.SffnError):
        gpu_forward(layer, Y, keep_t, None)


@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_non_finite_score_keeps_every_token(bad):
    """A NaN or infinite attention row makes the total mass non-finite: every
    token is kept (the oracle's rule), and no kernel writes outside the
    scratch.  The block selection keeps that sequence whole."""
    import torch
    sf = _sf()
    w = synth._make_weights(synth.WT_BF16, 512, 1024, synth.ACT_SILU, (751, 752, 753))
    L = 1000
    Y, A = synth.cfg5_activations(L=L, d=512)
    A = A.copy()
    bits = np.array([bad], np.float32).view(np.uint32)[0] >> 16
    A[137, 5] = np.uint16(bits)
    layer = make_prefill_layer(w, L)
    big, guard, sb = _guarded_scratch(layer)
    keep_t, cnt_t, keep, scores = gpu_select(layer, A, 0.3, 16, 1)
    s_ref = oracle.token_norms(A)
    fin = np.isfinite(s_ref)
    assert np.array_equal(np.isfinite(scores), fin) and np.array_equal(scores[fin], s_ref[fin])
    assert keep.size == L and oracle.token_select(s_ref, 0.3, 16, 1)[0].size == L
    X = gpu_forward(layer, Y, keep_t, cnt_t)
    assert _guards_intact(big, guard, sb), "a kernel wrote outside the scratch"
    cu = torch.tensor([0, 400, L], dtype=torch.int32, device="cuda:0")
    bk = torch.full((L,), -1, dtype=torch.int32, device="cuda:0")
    bc = torch.full((1,), -1, dtype=torch.int32, device="cuda:0")
    pol = sf.make_block_policy(mass_thresh=0.3, block=16, recent_n=16)
    layer.select_blocks(pol, tensor(A), cu, bk, bc)
    torch.cuda.synchronize()
    got = bk[:int(bc.item())].cpu().numpy()
    ref = oracle.block_select(oracle.token_norms(A), cu.cpu().numpy(), block=16, mass=0.3, min_full=0.1,
                              max_full=0.5, recent_n=16, min_keep=1)
    assert np.array_equal(got, ref) and set(range(400)) <= set(got.tolist())
    assert _guards_intact(big, guard, sb), "a kernel wrote outside the scratch"
    layer.close()


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
