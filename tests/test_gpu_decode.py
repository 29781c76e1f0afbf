"""GPU parity of the decode path against the CPU oracle (through the C ABI).

Bars: selected index sets and the fixed-order gate values bit-exact; outputs
within relative L2 1e-5 (fp32), 2e-3 (bf16), 5e-3 (int4, same dequantised
weights); repeated runs bitwise identical.
"""
import numpy as np
import pytest

import oracle
import synth

from gpu_util import make_layer, rel_l2, run_decode, scratch_views

pytestmark = pytest.mark.gpu

TOL = {synth.WT_F32: 1e-5, synth.WT_BF16: 2e-3, synth.WT_I4: 5e-3}


def _sf():
    import activation_sparse_gated_gate_amd as sf
    return sf


def _check(layer, w, x, mode, tol, **kw):
    """Run one call on the GPU and the oracle; compare everything unique."""
    sf = _sf()
    pol = sf.make_policy(mode, gate_bias=kw.get("bias", 0.0), theta=kw.get("theta", 0.0),
                         topk_k=kw.get("topk_k", 1), use_union=kw.get("union", False),
                         batch_path=kw.get("batch_path", 0))
    y, idx, n = run_decode(layer, pol, x)
    ref = oracle.decode(w, x, mode=mode, bias=kw.get("bias", 0.0), theta=kw.get("theta", 0.0),
                        topk_k=kw.get("topk_k", 1), union=kw.get("union", False),
                        rmsnorm=layer.desc.rmsnorm, residual=layer.desc.residual)
    B = x.shape[0]
    xh, g, u = scratch_views(layer, B)
    assert np.array_equal(g.cpu().numpy().view(np.uint32), ref["g"].view(np.uint32)), "gate values differ"
    if layer.desc.rmsnorm:
        assert np.array_equal(xh.cpu().numpy().view(np.uint32), ref["xhat"].view(np.uint32)), "x_hat differs"
    if mode == "topk":
        assert np.array_equal(u.cpu().numpy().view(np.uint32), ref["u"].view(np.uint32)), "up values differ"
    assert n == ref["idx"].size and np.array_equal(idx, ref["idx"]), "selected sets differ"
    err = rel_l2(y, ref["y"])
    assert err <= tol, "relative L2 %.3g > %.3g" % (err, tol)
    return y, ref, err


# ---------------------------------------------------------------------------
# config 1: fp32, 512 / 1408, exact ReLU gating at a = 0.2, 64 tokens
# ---------------------------------------------------------------------------

def test_cfg1_exact_gating_64_tokens_and_equals_dense():
    sf = _sf()
    w = synth.cfg1_weights()
    x = synth.cfg1_tokens(64)
    b = synth.gate_offset_for_active_fraction(synth.CFG1_ACTIVE)
    layer = make_layer(w, 1)
    worst = 0.0
    active = []
    for t in range(64):
        y, ref, err = _check(layer, w, x[t:t + 1], "exact", 1e-5, bias=b)
        worst = max(worst, err)
        active.append(ref["idx"].size / 1408)
        # the dense FFN (plain GEMV kernels) gives the same y
        yd, _, _ = run_decode(layer, sf.make_policy("dense", gate_bias=b), x[t:t + 1], want_list=False)
        assert rel_l2(yd, ref["y"]) <= 1e-5
        assert rel_l2(y, yd) <= 2e-5
    assert abs(np.mean(active) - 0.2) < 0.02
    print("cfg1 worst relL2 %.3g, mean active %.4f" % (worst, np.mean(active)))


def test_cfg1_repeat_is_bitwise_deterministic():
    sf = _sf()
    w = synth.cfg1_weights()
    x = synth.cfg1_tokens(3)
    b = synth.gate_offset_for_active_fraction(0.2)
    layer = make_layer(w, 1)
    pol = sf.make_policy("exact", gate_bias=b)
    for t in range(3):
        y1, i1, _ = run_decode(layer, pol, x[t:t + 1])
        y2, i2, _ = run_decode(layer, pol, x[t:t + 1])
        assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
        assert np.array_equal(i1, i2)


# ---------------------------------------------------------------------------
# config 2: bf16 Llama-2-7B FFN shape, a in {1.0, 0.6, 0.3, 0.1}
# ---------------------------------------------------------------------------

CFG2_TOKENS = 1024     # the benchmark's 1024 seeded tokens per active fraction
CFG2_Y_SAMPLE = 64     # tokens whose output y is compared as well


@pytest.fixture(scope="module")
def cfg2():
    w = synth.cfg2_weights()
    x = synth.cfg2_tokens(CFG2_TOKENS)
    layer = make_layer(w, 1)
    yield w, x, layer
    layer.close()


def _run_tokens_b1(layer, pol, x, keep_y):
    """One batch-1 forward per token (the benchmark's launch configuration);
    returns g' [T, f] (fp32 bits), the selected lists (count, idx [T, f]) and
    y for the first keep_y tokens.  Everything stays on the device until one
    synchronisation at the end."""
    import torch
    from gpu_util import tensor
    T, f = x.shape[0], layer.desc.d_ff
    xt = tensor(np.ascontiguousarray(x, np.float32))
    yt = torch.empty_like(xt)
    g_all = torch.empty((T, f), dtype=torch.float32, device=xt.device)
    idx = torch.full((T, f), -1, dtype=torch.int32, device=xt.device)
    cnt = torch.full((T,), -1, dtype=torch.int32, device=xt.device)
    _, g, _ = scratch_views(layer, 1)
    for t in range(T):
        layer.forward(pol, xt[t:t + 1], yt[t:t + 1], idx_out=idx[t], count_out=cnt[t:t + 1])
        g_all[t].copy_(g[0])
    torch.cuda.synchronize()
    return (g_all.cpu().numpy(), cnt.cpu().numpy(), idx.cpu().numpy(), yt[:keep_y].cpu().numpy())


@pytest.mark.parametrize("a", [1.0, 0.6, 0.3, 0.1])
def test_cfg2_every_token_gate_and_selection_bitwise(cfg2, a):
    """All 1024 tokens of the benchmark at each active fraction, through the
    batch-1 fused kernel: g' and the selected index sets bit-exact against the
    oracle's fixed-order gate; y within 2e-3 on the first 64 tokens."""
    sf = _sf()
    w, x, layer = cfg2
    mode = "all" if a == 1.0 else "exact"
    b = 0.0 if a == 1.0 else synth.gate_offset_for_active_fraction(a)
    g, cnt, idx, y = _run_tokens_b1(layer, sf.make_policy(mode, gate_bias=b), x, CFG2_Y_SAMPLE)
    sel = oracle.decode(w, x, mode=mode, bias=b, outputs=False)
    assert np.array_equal(g.view(np.uint32), sel["g"].view(np.uint32)), "gate values differ"
    bad = [t for t in range(x.shape[0])
           if not np.array_equal(idx[t, :cnt[t]], np.flatnonzero(sel["sel"][t]))]
    assert not bad, "selected sets differ for tokens %s" % bad[:10]
    fr = sel["sel"].mean()
    assert abs(fr - a) < 0.01, fr
    ref = oracle.decode(w, x[:CFG2_Y_SAMPLE], mode=mode, bias=b)
    errs = [rel_l2(y[t], ref["y"][t]) for t in range(CFG2_Y_SAMPLE)]
    assert max(errs) <= 2e-3, max(errs)


def test_cfg2_dense_mode_matches_oracle(cfg2):
    sf = _sf()
    w, x, layer = cfg2
    y, _, _ = run_decode(layer, sf.make_policy("dense"), x[:1], want_list=False)
    ref = oracle.decode(w, x[:1], mode="all")
    assert rel_l2(y, ref["y"]) <= 2e-3


def test_cfg2_select_entry_matches_forward_list(cfg2):
    import torch
    sf = _sf()
    from gpu_util import tensor
    w, x, layer = cfg2
    b = synth.gate_offset_for_active_fraction(0.3)
    pol = sf.make_policy("exact", gate_bias=b)
    xt = tensor(x[:1])
    idx = torch.full((w.d_ff,), -1, dtype=torch.int32, device=xt.device)
    cnt = torch.zeros(1, dtype=torch.int32, device=xt.device)
    layer.select(pol, xt, idx, cnt)
    torch.cuda.synchronize()
    n = int(cnt.item())
    _, fidx, fn = run_decode(layer, pol, x[:1])
    assert n == fn and np.array_equal(idx[:n].cpu().numpy(), fidx)


# ---------------------------------------------------------------------------
# batches, ragged sizes, modes, edge cases (reduced shapes)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("wt", [synth.WT_F32, synth.WT_BF16])
@pytest.mark.parametrize("B", [1, 2, 3, 5, 8, 11, 16])
def test_batches_thresh_and_exact(wt, B):
    d, f = 768, 1664   # d: 3 chunk-columns for fp32 / 1.5 for bf16 (ragged); f: 104 blocks of 16
    act = synth.ACT_SILU
    w = synth._make_weights(wt, d, f, act, (900 + B, 901 + B, 902 + B))
    x = synth.normal_f32(950 + B, (B, d))
    if wt == synth.WT_BF16:
        x = synth.round_to_bf16(x)
    th = synth.gate_threshold_for_active_fraction(0.13)
    tol = TOL[wt]
    relu = synth._make_weights(wt, d, f, synth.ACT_RELU, (900 + B, 901 + B, 902 + B))
    # bf16 runs twice: the VALU gather path and, with the MFMA tile layout, the batched MFMA path
    for layouts in _layouts(wt):
        layer = make_layer(w, 16, layouts=layouts)
        _check(layer, w, x, "thresh", tol, theta=th, union=True)
        _check(layer, w, x, "thresh", tol, theta=th, union=False)
        _check(layer, w, x, "all", tol)
        layer.close()
        lr = make_layer(relu, 16, layouts=layouts)
        _check(lr, relu, x, "exact", tol, bias=synth.gate_offset_for_active_fraction(0.3), union=False)
        lr.close()


def _layouts(wt):
    sf = _sf()
    if wt == synth.WT_BF16:
        return (sf.LAYOUT_DECODE, sf.LAYOUT_DECODE | sf.LAYOUT_BATCH)
    return (sf.LAYOUT_DECODE,)


@pytest.mark.parametrize("B", [5, 8, 16])
def test_batched_mfma_sparse_blocks(B):
    # very few selected neurons: most gate blocks of 16 are empty and skip their weights
    sf = _sf()
    d, f = 1024, 2048
    w = synth._make_weights(synth.WT_BF16, d, f, synth.ACT_RELU, (1901, 1902, 1903))
    x = synth.round_to_bf16(synth.normal_f32(1904 + B, (B, d)))
    layer = make_layer(w, 16, layouts=sf.LAYOUT_DECODE | sf.LAYOUT_BATCH)
    for a in (0.002, 0.02):
        b = synth.gate_offset_for_active_fraction(a)
        _check(layer, w, x, "exact", 2e-3, bias=b, union=True)
        _check(layer, w, x, "exact", 2e-3, bias=b, union=False)
    y, idx, n = run_decode(layer, sf.make_policy("exact", gate_bias=-40.0), x)
    assert n == 0 and np.all(y == 0.0)
    layer.close()


@pytest.mark.parametrize("B", [9, 16])
def test_batched_gate_up_launch_with_a_half_slice(B):
    # d_model 1280 = 2.5 gate slices of 512: the last slice of the class-split gate
    # is half empty (its x pieces and lanes past the row are skipped), with and
    # without the RMSNorm prologue (which writes the class-major x), and every
    # selection mode of the tile path (9..16 tokens)
    sf = _sf()
    d, f = 1280, 1024
    w = synth._make_weights(synth.WT_BF16, d, f, synth.ACT_SILU, (1931, 1932, 1933))
    x = synth.round_to_bf16(synth.normal_f32(1934 + B, (B, d)))
    for rms in (False, True):
        layer = make_layer(w, 16, rmsnorm=rms, residual=rms, layouts=sf.LAYOUT_DECODE | sf.LAYOUT_BATCH)
        _check(layer, w, x, "all", 2e-3, union=True)
        _check(layer, w, x, "thresh", 2e-3, theta=synth.gate_threshold_for_active_fraction(0.3), union=True)
        _check(layer, w, x, "thresh", 2e-3, theta=synth.gate_threshold_for_active_fraction(0.3), union=False)
        _check(layer, w, x, "exact", 2e-3, bias=synth.gate_offset_for_active_fraction(0.05), union=False)
        layer.close()


@pytest.mark.parametrize("B", [5, 8, 16])
def test_batched_tile_and_gather_paths_match_the_oracle(B):
    # the device picks the tile or the gather path from the union size; both forced
    # paths and the automatic choice must match the oracle, from nearly empty to
    # nearly full unions, with and without the union rule
    sf = _sf()
    d, f = 1024, 2048
    w = synth._make_weights(synth.WT_BF16, d, f, synth.ACT_RELU, (1911, 1912, 1913))
    x = synth.round_to_bf16(synth.normal_f32(1914 + B, (B, d)))
    layer = make_layer(w, 16, layouts=sf.LAYOUT_DECODE | sf.LAYOUT_BATCH)
    for a in (0.002, 0.05, 0.3):
        b = synth.gate_offset_for_active_fraction(a)
        for union in (True, False):
            ys = [_check(layer, w, x, "exact", 2e-3, bias=b, union=union, batch_path=p)[0] for p in (1, 2, 0)]
            assert rel_l2(ys[0], ys[1]) <= 2e-3
    th = synth.gate_threshold_for_active_fraction(0.1)
    wt = synth._make_weights(synth.WT_BF16, d, f, synth.ACT_SILU, (1921, 1922, 1923))
    layer_t = make_layer(wt, 16, rmsnorm=True, residual=True, layouts=sf.LAYOUT_DECODE | sf.LAYOUT_BATCH)
    for p in (1, 2, 0):
        _check(layer_t, wt, x, "thresh", 2e-3, theta=th, union=True, batch_path=p)
    with pytest.raises(sf.SffnError):
        run_decode(layer, sf.make_policy("exact", batch_path=3), x)
    layer.close()
    layer_t.close()


def test_rmsnorm_residual_batch16():
    w = synth._make_weights(synth.WT_BF16, 1024, 2048, synth.ACT_SILU, (961, 962, 963))
    x = synth.normal_f32(964, (16, 1024)) * np.float32(2.5)
    th = synth.gate_threshold_for_active_fraction(0.3)
    for layouts in _layouts(synth.WT_BF16):
        layer = make_layer(w, 16, rmsnorm=True, residual=True, layouts=layouts)
        _check(layer, w, x, "thresh", 2e-3, theta=th, union=True)
        _check(layer, w, x[:7], "all", 2e-3)
        layer.close()


def test_no_active_neuron_gives_zero_output():
    sf = _sf()
    w = synth._make_weights(synth.WT_BF16, 512, 1408, synth.ACT_RELU, (971, 972, 973))
    x = synth.round_to_bf16(synth.normal_f32(974, (2, 512)))
    layer = make_layer(w, 2)
    y, idx, n = run_decode(layer, sf.make_policy("exact", gate_bias=-40.0), x)
    assert n == 0 and np.all(y == 0.0)
    layer_r = make_layer(w, 2, residual=True)
    y, idx, n = run_decode(layer_r, sf.make_policy("exact", gate_bias=-40.0), x)
    assert n == 0 and np.array_equal(y, x)


def test_all_neurons_active_exact_equals_all():
    sf = _sf()
    w = synth._make_weights(synth.WT_BF16, 512, 1408, synth.ACT_RELU, (981, 982, 983))
    x = synth.round_to_bf16(synth.normal_f32(984, (1, 512)))
    layer = make_layer(w, 1)
    y1, i1, n1 = run_decode(layer, sf.make_policy("exact", gate_bias=40.0), x)
    y2, i2, n2 = run_decode(layer, sf.make_policy("all", gate_bias=40.0), x)
    assert n1 == n2 == 1408 and np.array_equal(i1, i2)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


# ---------------------------------------------------------------------------
# config 3: int4 weight-aware top-k, batch 1 and 8 (union)
# ---------------------------------------------------------------------------

CFG3_B1_TOKENS = 32    # batch-1 tokens checked per keep fraction
CFG3_B8_BATCHES = 8    # batches of 8 checked per keep fraction


@pytest.fixture(scope="module")
def cfg3():
    w = synth.cfg3_weights()
    x = synth.cfg3_tokens(8 * CFG3_B8_BATCHES)
    layer = make_layer(w, 8)
    yield w, x, layer
    layer.close()


@pytest.mark.parametrize("pct", synth.CFG3_KEEP_PCT)
def test_cfg3_topk_batch1(cfg3, pct):
    """32 single-token calls per keep fraction: g', u and the top-k sets
    bit-exact, y within 5e-3 of the oracle on the same dequantised weights."""
    sf = _sf()
    w, x, layer = cfg3
    k = synth.topk_count(w.d_ff, pct)
    pol = sf.make_policy("topk", topk_k=k)
    ref = oracle.decode(w, x[:CFG3_B1_TOKENS], mode="topk", topk_k=k)
    for t in range(CFG3_B1_TOKENS):
        y, idx, n = run_decode(layer, pol, x[t:t + 1])
        _, g, u = scratch_views(layer, 1)
        assert np.array_equal(g.cpu().numpy()[0].view(np.uint32), ref["g"][t].view(np.uint32)), t
        assert np.array_equal(u.cpu().numpy()[0].view(np.uint32), ref["u"][t].view(np.uint32)), t
        assert n == k and np.array_equal(idx, np.flatnonzero(ref["sel"][t])), t
        assert rel_l2(y[0], ref["y"][t]) <= 5e-3, t


@pytest.mark.parametrize("pct", synth.CFG3_KEEP_PCT)
def test_cfg3_topk_batch8_union(cfg3, pct):
    w, x, layer = cfg3
    k = synth.topk_count(w.d_ff, pct)
    for q in range(CFG3_B8_BATCHES):
        y, ref, err = _check(layer, w, x[8 * q:8 * q + 8], "topk", 5e-3, topk_k=k, union=True)
        dens = ref["idx"].size / w.d_ff
        assert dens > oracle.group_active_probability(pct / 100, 8) - 0.15


@pytest.mark.parametrize("B", [1, 8])
def test_cfg3_int4_dense_mode_matches_all(cfg3, B):
    """The int4 dense baseline (plain fixed-order GEMVs over W_gate, W_up and the
    natural W_down with its [d_model][d_ff / 128] scales) against the oracle's
    every-neuron FFN."""
    sf = _sf()
    w, x, layer = cfg3
    y, _, _ = run_decode(layer, sf.make_policy("dense"), x[:B], want_list=False)
    ref = oracle.decode(w, x[:B], mode="all")
    assert rel_l2(y, ref["y"]) <= 5e-3


@pytest.mark.parametrize("wt,B", [(synth.WT_F32, 4), (synth.WT_BF16, 8), (synth.WT_BF16, 16), (synth.WT_I4, 5),
                                  (synth.WT_I4, 8)])
def test_dense_mode_batches(wt, B):
    sf = _sf()
    w = synth._make_weights(wt, 1024, 2816, synth.ACT_SILU, (1931, 1932, 1933))
    x = synth.normal_f32(1934, (B, 1024))
    if wt == synth.WT_BF16:
        x = synth.round_to_bf16(x)
    layer = make_layer(w, B)
    y, _, _ = run_decode(layer, sf.make_policy("dense", gate_bias=0.25), x, want_list=False)
    ref = oracle.decode(w, x, mode="all", bias=0.25)
    assert rel_l2(y, ref["y"]) <= TOL[wt]
    layer.close()


@pytest.mark.parametrize("d,f,rms", [(4096, 1408, True), (2048, 896, False), (1024, 1408, False)])
def test_int4_dense_one_token(d, f, rms):
    """The int4 dense layer at one token: d_model a multiple of 2048 runs the
    streaming gate + up kernel (writing h) and the row-streaming down GEMV
    (4096: two chunks per lane; RMSNorm and residual), other widths the plain
    fixed-order GEMVs; both against the oracle's every-neuron FFN."""
    sf = _sf()
    w = synth._make_weights(synth.WT_I4, d, f, synth.ACT_SILU, (1941 + d, 1942, 1943))
    x = synth.normal_f32(1944, (1, d))
    layer = make_layer(w, 1, rmsnorm=rms, residual=rms)
    y, _, _ = run_decode(layer, sf.make_policy("dense", gate_bias=0.125), x, want_list=False)
    ref = oracle.decode(w, x, mode="all", bias=0.125, rmsnorm=rms, residual=rms)
    assert rel_l2(y, ref["y"]) <= TOL[synth.WT_I4]
    layer.close()


def test_thresh_theta_must_express_a_threshold_on_the_activation():
    """THRESH is |act(g')| > tau taken as g' > theta: for SiLU that needs theta
    above 0.45511541... (SiLU(theta) beyond SiLU's minimum depth), for ReLU
    theta >= 0; other values are refused before any launch."""
    sf = _sf()
    w = synth._make_weights(synth.WT_BF16, 512, 1408, synth.ACT_SILU, (1941, 1942, 1943))
    x = synth.round_to_bf16(synth.normal_f32(1944, (1, 512)))
    layer = make_layer(w, 1)
    bound = np.float32(0.4551154)   # the largest float below the bound
    for th in (0.0, 0.3, float(bound)):
        with pytest.raises(sf.SffnError) as e:
            run_decode(layer, sf.make_policy("thresh", theta=th), x)
        assert e.value.status == sf.SFFN_ERR_UNSUPPORTED
    with pytest.raises(sf.SffnError) as e:
        run_decode(layer, sf.make_policy("thresh", theta=float("nan")), x)
    assert e.value.status == sf.SFFN_ERR_INVALID_ARG
    _check(layer, w, x, "thresh", 2e-3, theta=float(np.nextafter(bound, np.float32(1))))
    layer.close()
    wr = synth._make_weights(synth.WT_BF16, 512, 1408, synth.ACT_RELU, (1945, 1946, 1947))
    lr = make_layer(wr, 1)
    with pytest.raises(sf.SffnError) as e:
        run_decode(lr, sf.make_policy("thresh", theta=-0.1), x)
    assert e.value.status == sf.SFFN_ERR_UNSUPPORTED
    # theta = 0 on ReLU is exact gating
    _, i0, _ = run_decode(lr, sf.make_policy("thresh", theta=0.0), x)
    _, i1, _ = run_decode(lr, sf.make_policy("exact"), x)
    assert np.array_equal(i0, i1)
    lr.close()


def test_topk_k_equals_f_and_k_one(cfg3):
    w, x, layer = cfg3
    _check(layer, w, x[:2], "topk", 5e-3, topk_k=w.d_ff, union=True)
    _check(layer, w, x[:3], "topk", 5e-3, topk_k=1, union=False)


def test_int4_batch1_topk_edge_cases(cfg3):
    """Batch-1 int4 top-k (the streaming gate + up kernel, then the select):
    k = 1, k = f (every neuron), and a zero token, whose scores all tie at 0
    (the lowest k indices win: the select's equal-key path)."""
    w, x, layer = cfg3
    f = w.d_ff
    _check(layer, w, x[:1], "topk", 5e-3, topk_k=1)
    _check(layer, w, x[1:2], "topk", 5e-3, topk_k=f)
    z = np.zeros((1, w.d_model), np.float32)
    sf = _sf()
    for k in (1, 300, 4000):
        y, idx, n = run_decode(layer, sf.make_policy("topk", topk_k=k), z)
        assert n == k and np.array_equal(idx, np.arange(k)), k
        assert np.all(y == 0.0)


@pytest.mark.parametrize("B", [1, 8])
def test_topk_run_merging_reads_gaps_without_changing_the_result(cfg3, B):
    """merge_gap > 0 also reads the unselected rows of short gaps with h = 0:
    the selected set and y are the same values as without merging."""
    sf = _sf()
    w, x, layer = cfg3
    k = synth.topk_count(w.d_ff, 17)
    base = run_decode(layer, sf.make_policy("topk", topk_k=k, use_union=B > 1), x[:B])
    for gap in (1, 4, 64):
        y, idx, n = run_decode(layer, sf.make_policy("topk", topk_k=k, use_union=B > 1, merge_gap=gap), x[:B])
        assert n == base[2] and np.array_equal(idx, base[1])
        assert np.array_equal(y, base[0]), gap
    with pytest.raises(sf.SffnError):
        run_decode(layer, sf.make_policy("topk", topk_k=k, merge_gap=65), x[:1])


def test_topk_ties_lower_index_first():
    # duplicated neurons give bit-identical scores; k cuts through the tie
    w = synth._make_weights(synth.WT_BF16, 512, 256, synth.ACT_SILU, (991, 992, 993))
    for m in (w.w_gate, w.w_up):
        m[200] = m[17]
        m[90] = m[17]
    w.w_down[:, 200] = w.w_down[:, 17]
    w.w_down[:, 90] = w.w_down[:, 17]
    x = synth.round_to_bf16(synth.normal_f32(994, (1, 512)))
    full = oracle.decode(w, x, mode="topk", topk_k=256)
    s = np.array([oracle.score(full["g"][0, j], full["u"][0, j], full["wdn"][j]) for j in range(256)])
    ahead = int((s > s[17]).sum())
    layer = make_layer(w, 1)
    _, ref, _ = _check(layer, w, x, "topk", 2e-3, topk_k=ahead + 2)
    assert 17 in ref["idx"] and 90 in ref["idx"] and 200 not in ref["idx"]


def test_int4_sparse_union_scales_of_a_third_group():
    """int4 gather with a union so sparse (about 1.5 % of d_ff = 65536) that a
    batch of 16 consecutive rows of one workgroup's share spans three or more
    128-neuron scale groups; the rows past the batch's first and last group
    load their scales on their own."""
    w = synth._make_weights(synth.WT_I4, 256, 65536, synth.ACT_RELU, (981, 982, 983))
    x = synth.normal_f32(985, (2, 256))
    b = synth.gate_offset_for_active_fraction(0.015)
    layer = make_layer(w, 1)
    for t in range(2):
        _, ref, _ = _check(layer, w, x[t:t + 1], "exact", 5e-3, bias=b)
        # the batched gather splits the list into 256 equal shares, rows in
        # batches of 16: the case must occur
        idx, n, P = ref["idx"], ref["idx"].size, 256
        spans = []
        for q in range(P):
            lo, hi = q * n // P, (q + 1) * n // P
            for b0 in range(lo, hi, 16):
                rows = idx[b0:min(hi, b0 + 16)]
                spans.append(len(set((rows >> 7).tolist())))
        assert max(spans) >= 3, "no batch reaches a third scale group"
    layer.close()


@pytest.mark.parametrize("case", ["bf16_b1_exact", "int4_b8_topk", "int4_b1_topk", "bf16_b16_tiles",
                                  "bf16_b16_gather"])
def test_decode_writes_stay_inside_the_scratch(case):
    import torch
    sf = _sf()
    if case == "int4_b8_topk":
        w = synth._make_weights(synth.WT_I4, 512, 1408, synth.ACT_SILU, (731, 732, 733))
        B, layouts, kw = 8, None, dict(mode="topk", topk_k=300, union=True)
    elif case == "int4_b1_topk":
        w = synth._make_weights(synth.WT_I4, 2048, 1408, synth.ACT_SILU, (741, 742, 743))
        B, layouts, kw = 1, None, dict(mode="topk", topk_k=300)
    elif case == "bf16_b1_exact":
        w = synth._make_weights(synth.WT_BF16, 1024, 2816, synth.ACT_RELU, (734, 735, 736))
        B, layouts, kw = 1, None, dict(mode="exact", bias=synth.gate_offset_for_active_fraction(0.1))
    else:
        w = synth._make_weights(synth.WT_BF16, 1024, 2816, synth.ACT_SILU, (737, 738, 739))
        B, layouts = 16, sf.LAYOUT_DECODE | sf.LAYOUT_BATCH
        kw = dict(mode="thresh", theta=synth.gate_threshold_for_active_fraction(0.1), union=True,
                  batch_path=1 if case.endswith("tiles") else 2)
    x = synth.round_to_bf16(synth.normal_f32(740, (B, w.d_model)))
    layer = make_layer(w, B, layouts=layouts)
    guard = 1 << 20
    sb = layer.scratch_bytes
    big = torch.full((sb + 2 * guard,), 0xA5, dtype=torch.uint8, device="cuda:0")
    layer.scratch = big[guard:guard + sb]
    mode = kw.pop("mode")
    _check(layer, w, x, mode, TOL[w.wtype], **kw)
    torch.cuda.synchronize()
    assert bool((big[:guard] == 0xA5).all()) and bool((big[guard + sb:] == 0xA5).all()), \
        "a kernel wrote outside the scratch"
    layer.close()
