"""Pins of the CPU oracle to things other than itself.

Each test checks the oracle against what the pages or the mathematics fix:
values printed in the pages (tests/golden), closed forms, invariants, special
cases with exact answers, independent fp64 numpy / exact-rational computations
and brute force on tiny inputs.  No expected value here comes from the HIP
library.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_values.json")


def tiny_weights(wt, d, f, act, seed=7):
    return synth._make_weights(wt, d, f, act, (seed, seed + 1, seed + 2))


def dense_f64(w: synth.FFNWeights):
    """Weights as fp64 arrays, decoded independently of the oracle (numpy)."""
    if w.wtype == synth.WT_F32:
        return [np.asarray(m, np.float64) for m in (w.w_gate, w.w_up, w.w_down)]
    if w.wtype == synth.WT_BF16:
        return [synth.bf16_bits_to_f32(m).astype(np.float64) for m in (w.w_gate, w.w_up, w.w_down)]
    return [synth.dequantize_int4_g128(m, s).astype(np.float64)
            for m, s in ((w.w_gate, w.s_gate), (w.w_up, w.s_up), (w.w_down, w.s_down))]


def ffn_f64(w, xhat, mask, bias=0.0):
    Wg, Wu, Wd = dense_f64(w)
    g = xhat.astype(np.float64) @ Wg.T + bias
    u = xhat.astype(np.float64) @ Wu.T
    a = np.maximum(g, 0.0) if w.act == synth.ACT_RELU else g / (1.0 + np.exp(-g))
    return (a * u * mask) @ Wd.T


def rel_l2(a, b):
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / max(np.linalg.norm(b), 1e-300))


# ---------------------------------------------------------------------------
# values printed in the pages (cost model)
# ---------------------------------------------------------------------------

def test_cost_model_matches_printed_values():
    g = json.load(open(GOLDEN))
    for e in g["kept_fraction"]:
        assert abs(oracle.kept_fraction(e["a"]) - e["kept"]) <= e["tol"], e["cite"]
    for e in g["ideal_speedup"]:
        assert abs(e["measured"] / oracle.ideal_speedup(e["a"]) - e["fraction_of_ideal"]) <= e["tol"], e["cite"]
    for e in g["group_active_probability"]:
        p = oracle.group_active_probability(e["a"], e["k"])
        if "lower_bound" in e:
            assert p > e["lower_bound"], e["cite"]
        else:
            assert abs(p - e["approx"]) <= e["tol"], e["cite"]


def test_cost_model_limits():
    assert oracle.kept_fraction(1.0) == 1.0
    assert oracle.kept_fraction(0.0) == pytest.approx(1 / 3)
    assert oracle.ideal_speedup(0.1) == pytest.approx(2.5)
    assert oracle.group_active_probability(0.3, 1) == pytest.approx(0.3)


def test_topk_count_rule():
    # k = max(1, int(n * keep_ratio)) (WiSparse notes, section 3.2, select_mask)
    for n in (1, 7, 16, 11008):
        for pct in (0, 1, 17, 30, 50, 100):
            assert synth.topk_count(n, pct) == max(1, int(Fraction(n * pct, 100)))
    assert synth.topk_count(11008, 17) == 1871


# ---------------------------------------------------------------------------
# storage formats
# ---------------------------------------------------------------------------

def test_int4_nibble_order_sign_and_scale():
    # one row of 128 int4 values; bytes hand-packed: low nibble = even column
    packed = np.zeros((1, 64), np.uint8)
    packed[0, 0] = 0x21      # col0 = +1, col1 = +2
    packed[0, 1] = 0xF8      # col2 = -8, col3 = -1
    packed[0, 2] = 0x07      # col4 = +7, col5 = 0
    scales = np.array([[np.float16(0.5).view(np.uint16)]], np.uint16)
    expect = {0: 0.5, 1: 1.0, 2: -4.0, 3: -0.5, 4: 3.5, 5: 0.0}
    for c, v in expect.items():
        x = np.zeros(128, np.float32)
        x[c] = 1.0
        assert oracle.dot_c1(2, packed, scales, 0, x) == np.float32(v)


@pytest.mark.parametrize("bits", [0x0001, 0x03FF, 0x0400, 0x3C00, 0x3555, 0x7BFF, 0x8001, 0xBC00, 0xC8A3])
def test_fp16_scale_decode_matches_ieee(bits):
    packed = np.zeros((1, 64), np.uint8)
    packed[0, 0] = 0x01
    scales = np.array([[bits]], np.uint16)
    x = np.zeros(128, np.float32)
    x[0] = 1.0
    assert oracle.dot_c1(2, packed, scales, 0, x) == np.array([bits], np.uint16).view(np.float16).astype(np.float32)[0]


def test_bf16_rne_against_exact_rationals():
    rng = np.random.default_rng(3)
    vals = list(rng.standard_normal(2000) * 10.0 ** rng.integers(-6, 6, 2000))
    # exact ties between two bf16 neighbours, both parities
    for m in (0x3F80, 0x3F81, 0x4120, 0xC121):
        lo = synth.bf16_bits_to_f32(np.array([m], np.uint16))[0]
        hi = synth.bf16_bits_to_f32(np.array([m + 1], np.uint16))[0]
        vals.append((float(lo) + float(hi)) / 2.0)
    vals = np.array(vals, np.float64)
    got = oracle.bf16_rne(vals)
    for v, b in zip(vals, got):
        fv = Fraction(float(v))
        # candidate neighbours: the bf16 values around v
        f32 = np.float32(v)
        base = int(np.array([f32], np.float32).view(np.uint32)[0]) & 0xFFFF0000
        cands = []
        for off in (-2, -1, 0, 1, 2):
            u = (base + off * 0x10000) & 0xFFFFFFFF
            c = np.array([u], np.uint32).view(np.float32)[0]
            if np.isfinite(c):
                cands.append((abs(Fraction(float(c)) - fv), (u >> 16) & 1, u >> 16))
        cands.sort()
        best = cands[0]
        if len(cands) > 1 and cands[1][0] == best[0]:
            best = min(cands[:2], key=lambda t: t[1])  # tie: even significand
        assert int(b) == best[2], (v, hex(int(b)), hex(best[2]))


# ---------------------------------------------------------------------------
# C1 order: exact special cases that only the fixed order reproduces
# ---------------------------------------------------------------------------

def _row_with_chunks(E, d, entries):
    w = np.zeros((1, d), np.float32)
    for c, v in entries.items():
        w[0, c * E] = v
    return w


def test_c1_chunk_to_accumulator_map_is_c_mod_64():
    # chunks 0 and 64 share accumulator 0; chunk 1 sits in accumulator 1.
    # 2^24 + (-2^24) cancels exactly in acc0 and the 1 in acc1 survives: 1.
    # A blocked map (chunks 0,1 together) or one running sum rounds the 1 away.
    d, E = 512, 4
    w = _row_with_chunks(E, d, {0: 2.0 ** 24, 1: 1.0, 64: -(2.0 ** 24)})
    x = np.ones(d, np.float32)
    assert oracle.dot_c1(0, w, None, 0, x) == np.float32(1.0)
    seq = np.float32(0)
    for v in w[0]:
        seq = np.float32(seq + v)
    assert seq == np.float32(0.0)  # the naive order loses it


def test_c1_final_tree_halves_by_offset():
    # acc0 = 2^24, acc1 = 1, acc32 = -2^24: the offset-halving tree adds
    # acc32 into acc0 first (exact 0) and keeps the 1; a left-to-right sum of
    # the 64 accumulators or an adjacent-pair tree gives 0.
    d, E = 256, 4
    w = _row_with_chunks(E, d, {0: 2.0 ** 24, 1: 1.0, 32: -(2.0 ** 24)})
    assert oracle.dot_c1(0, w, None, 0, np.ones(d, np.float32)) == np.float32(1.0)


def test_c1_elements_in_chunk_are_fused_in_order():
    # one chunk (accumulator 0) holds [1, 2^24, 1, -2^24] times x = 1:
    # fma chain: 1 -> 2^24 + 1 (ties to 2^24) -> 2^24 + 1 (ties to 2^24) -> 0:
    # the in-order chain gives 0 while the exact sum is 2.
    d = 256
    w = np.zeros((1, d), np.float32)
    w[0, :4] = [1.0, 2.0 ** 24, 1.0, -(2.0 ** 24)]
    assert oracle.dot_c1(0, w, None, 0, np.ones(d, np.float32)) == np.float32(0.0)


def test_c1_bf16_and_int4_chunk_sizes():
    # bf16: 8 elements per chunk -> element 8*64 = 512 is chunk 64 (acc 0)
    d = 1024
    wf = np.zeros((1, d), np.float32)
    wf[0, 0] = 2.0 ** 24
    wf[0, 8] = 1.0          # chunk 1 -> acc1
    wf[0, 512] = -(2.0 ** 24)  # chunk 64 -> acc0
    wb = synth.f32_to_bf16_bits(wf)
    assert oracle.dot_c1(1, wb, None, 0, np.ones(d, np.float32)) == np.float32(1.0)
    # int4: 32 elements per chunk, t accumulated per chunk then scaled once
    d = 4096
    q = np.zeros((1, d), np.int8)
    q[0, 0:32] = 7           # chunk 0: t = 7*32 = 224
    s = np.full((1, d // 128), np.float16(1.0).view(np.uint16), np.uint16)
    nib = (q.astype(np.int16) & 0xF).astype(np.uint8)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    x = np.full(d, 0.125, np.float32)
    assert oracle.dot_c1(2, packed, s, 0, x) == np.float32(28.0)


@pytest.mark.parametrize("wt", [0, 1, 2])
def test_c1_close_to_fp64_but_not_the_naive_bits(wt):
    d, f = 1024, 128
    w = tiny_weights(wt, d, f, synth.ACT_RELU, seed=11)
    Wg = dense_f64(w)[0]
    x = synth.normal_f32(12, (d,))
    ex = Wg @ x.astype(np.float64)
    got = np.array([oracle.dot_c1(wt, w.w_gate, w.s_gate, r, x) for r in range(f)], np.float64)
    scale = np.abs(Wg) @ np.abs(x.astype(np.float64))
    assert np.all(np.abs(got - ex) <= 4e-7 * scale)
    wf = Wg.astype(np.float32)
    naive = np.empty(f, np.float32)
    for r in range(f):
        acc = np.float32(0)
        for k in range(d):
            acc = np.float32(acc + wf[r, k] * x[k])
        naive[r] = acc
    assert np.any(naive != got.astype(np.float32))


def test_rms_scale_close_to_fp64():
    x = synth.normal_f32(5, (3584,))
    ex = 1.0 / math.sqrt(float(np.mean(x.astype(np.float64) ** 2)) + 1e-6)
    assert abs(float(oracle.rms_scale(x)) - ex) <= 2e-6 * ex


# ---------------------------------------------------------------------------
# fp64 exp / silu / score
# ---------------------------------------------------------------------------

def test_exp64_within_one_ulp_of_libm():
    assert oracle.exp64(0.0) == 1.0
    zs = np.concatenate([np.linspace(-40, 40, 4001), np.random.default_rng(1).standard_normal(3000) * 8])
    for z in zs:
        e = oracle.exp64(float(z))
        ref = math.exp(float(z))
        assert abs(e - ref) <= math.ulp(ref), z


def test_silu64_and_threshold_equivalence():
    assert oracle.silu64(0.0) == 0.0
    assert oracle.silu64(-1.278464542761074) == pytest.approx(-0.2784645427610738, rel=1e-12)
    # |SiLU(g)| > tau  <=>  g > theta for tau above SiLU's minimum depth
    for a in (0.3, 0.13):
        theta = synth.gate_threshold_for_active_fraction(a)
        tau = oracle.silu64(theta)
        assert tau > 0.2785
        gs = np.random.default_rng(2).standard_normal(20000) * 3
        gs = gs[np.abs(gs - theta) > 1e-9]
        lhs = np.array([abs(oracle.silu64(g)) > tau for g in gs])
        assert np.array_equal(lhs, gs > theta)


def test_score_formula():
    g, u, n = np.float32(0.75), np.float32(-1.5), 2.0
    silu = 0.75 / (1.0 + math.exp(-0.75))
    assert oracle.score(g, u, n) == pytest.approx(abs(silu * -1.5) * 2.0, rel=1e-15)


def test_down_col_norms_are_column_norms_and_exact_for_int4():
    w = tiny_weights(2, 256, 384, synth.ACT_SILU, seed=21)
    n = oracle.down_col_norms(w)
    Wd = dense_f64(w)[2]             # [d, f]; column j = neuron j
    assert np.array_equal(n, np.sqrt(np.sum(Wd[::-1] ** 2, axis=0)))  # any order: exact
    assert not np.allclose(n[:256], np.sqrt(np.sum(Wd ** 2, axis=1)))  # not the rows


# ---------------------------------------------------------------------------
# decode layer: against fp64 numpy, invariants, brute force
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("wt,act", [(0, 0), (1, 0), (2, 1), (1, 1)])
def test_dense_layer_matches_fp64_numpy(wt, act):
    d, f = 256, 384
    w = tiny_weights(wt, d, f, act, seed=31)
    x = synth.normal_f32(32, (3, d))
    r = oracle.decode(w, x, mode="all", bias=-0.25)
    ref = ffn_f64(w, x, np.ones(f), bias=np.float64(np.float32(-0.25)))
    assert rel_l2(r["y"], ref) < 1e-12
    assert r["sel"].all() and r["used"].all()


def test_exact_gating_selects_positive_offset_gate_and_equals_dense():
    w = tiny_weights(0, 512, 1408, synth.ACT_RELU, seed=41)
    x = synth.normal_f32(42, (8, 512))
    b = synth.gate_offset_for_active_fraction(0.2)
    ex = oracle.decode(w, x, mode="exact", bias=b)
    dn = oracle.decode(w, x, mode="all", bias=b)
    # same output: skipped neurons have ReLU(g + b) = 0
    assert rel_l2(ex["y"], dn["y"]) < 1e-13
    Wg = dense_f64(w)[0]
    g64 = x.astype(np.float64) @ Wg.T + b
    far = np.abs(g64) > 1e-4
    assert np.array_equal(ex["sel"][far], (g64 > 0)[far])
    # the offset sets the active fraction (a = 0.2, not 0.8)
    assert abs(ex["sel"].mean() - 0.2) < 0.03
    # the mask applied equals the selection without union
    assert np.array_equal(ex["used"], ex["sel"])


def test_thresh_mode_selects_gate_above_theta():
    w = tiny_weights(1, 512, 2048, synth.ACT_SILU, seed=51)
    x = synth.round_to_bf16(synth.normal_f32(52, (4, 512)))
    th = synth.gate_threshold_for_active_fraction(0.3)
    r = oracle.decode(w, x, mode="thresh", theta=th)
    g64 = x.astype(np.float64) @ dense_f64(w)[0].T
    far = np.abs(g64 - th) > 1e-4
    assert np.array_equal(r["sel"][far], (g64 > th)[far])
    assert abs(r["sel"].mean() - 0.3) < 0.03
    ref = ffn_f64(w, x, r["sel"].astype(np.float64))
    assert rel_l2(r["y"], ref) < 1e-12


def _brute_topk(scores, k):
    n = len(scores)
    sel = np.zeros(n, bool)
    for j in range(n):
        ahead = sum(1 for i in range(n) if scores[i] > scores[j] or (scores[i] == scores[j] and i < j))
        sel[j] = ahead < k
    return sel


@pytest.mark.parametrize("wt,f", [(1, 16), (2, 128)])
def test_topk_matches_brute_force(wt, f):
    d = 128
    w = tiny_weights(wt, d, f, synth.ACT_SILU, seed=61)
    x = synth.normal_f32(62, (5, d))
    Wg, Wu, Wd = dense_f64(w)
    nrm = np.sqrt((Wd ** 2).sum(axis=0))
    for k in (1, 3, 8, f - 1, f):
        r = oracle.decode(w, x, mode="topk", topk_k=k)
        for t in range(x.shape[0]):
            g = x[t].astype(np.float64) @ Wg.T
            u = x[t].astype(np.float64) @ Wu.T
            s = np.abs(g / (1.0 + np.exp(-g)) * u) * nrm
            assert np.array_equal(r["sel"][t], _brute_topk(list(s), k)), (k, t)
            assert r["sel"][t].sum() == k


def test_topk_ties_go_to_lower_index_and_k_equal_f_is_dense():
    d, f = 128, 16
    w = tiny_weights(1, d, f, synth.ACT_SILU, seed=71)
    # neurons 3, 9 and 12 are identical: equal scores, bit for bit
    for m in (w.w_gate, w.w_up):
        m[9] = m[3]
        m[12] = m[3]
    w.w_down[:, 9] = w.w_down[:, 3]
    w.w_down[:, 12] = w.w_down[:, 3]
    x = synth.normal_f32(72, (1, d))
    full = oracle.decode(w, x, mode="topk", topk_k=f)
    s = np.array([oracle.score(full["g"][0, j], full["u"][0, j], full["wdn"][j]) for j in range(f)])
    assert s[3] == s[9] == s[12]
    rank3 = int((s > s[3]).sum())   # neurons strictly ahead of the tied trio
    r = oracle.decode(w, x, mode="topk", topk_k=rank3 + 2)
    assert r["sel"][0, 3] and r["sel"][0, 9] and not r["sel"][0, 12]
    dn = oracle.decode(w, x, mode="all")
    assert rel_l2(full["y"], dn["y"]) < 1e-14


def test_union_batch_of_identical_tokens_equals_single_token():
    d, f = 256, 512
    w = tiny_weights(2, d, f, synth.ACT_SILU, seed=81)
    x1 = synth.normal_f32(82, (1, d))
    x8 = np.repeat(x1, 8, axis=0)
    one = oracle.decode(w, x1, mode="topk", topk_k=87)
    eight = oracle.decode(w, x8, mode="topk", topk_k=87, union=True)
    assert np.array_equal(eight["y"], np.repeat(one["y"], 8, axis=0))
    assert np.array_equal(eight["idx"], one["idx"])


def test_union_applies_the_union_mask_to_every_token():
    d, f = 256, 512
    w = tiny_weights(1, d, f, synth.ACT_SILU, seed=91)
    x = synth.round_to_bf16(synth.normal_f32(92, (4, d)))
    th = synth.gate_threshold_for_active_fraction(0.13)
    r = oracle.decode(w, x, mode="thresh", theta=th, union=True)
    U = r["sel"].any(axis=0)
    assert np.array_equal(r["used"], np.repeat(U[None], 4, axis=0))
    assert rel_l2(r["y"], ffn_f64(w, x, U.astype(np.float64))) < 1e-12
    # the expected union density is the group law 1 - (1 - a)^B
    assert abs(U.mean() - oracle.group_active_probability(r["sel"].mean(), 4)) < 0.06


def test_rmsnorm_prologue_and_residual():
    d, f = 512, 768
    w = tiny_weights(1, d, f, synth.ACT_SILU, seed=101)
    x = synth.normal_f32(102, (3, d)) * np.float32(3.0)
    r = oracle.decode(w, x, mode="all", rmsnorm=True, residual=True)
    x64 = x.astype(np.float64)
    xhat = x64 / np.sqrt(np.mean(x64 ** 2, axis=1, keepdims=True) + 1e-6)
    assert np.allclose(r["xhat"], xhat, rtol=2e-6, atol=0)
    ref = x64 + ffn_f64(w, r["xhat"], np.ones(f))
    assert rel_l2(r["y"], ref) < 1e-12


# ---------------------------------------------------------------------------
# token-selective prefill
# ---------------------------------------------------------------------------

def test_token_norms_close_to_fp64():
    Y, A = synth.cfg5_activations(L=64, d=256)
    s = oracle.token_norms(A)
    ref = np.linalg.norm(synth.bf16_bits_to_f32(A).astype(np.float64), axis=1)
    assert np.all(np.abs(s - ref) <= 1e-6 * ref)


def _brute_token_select(s, mass, recent_n, min_keep):
    L = len(s)
    order = sorted(range(L), key=lambda i: (-Fraction(float(s[i])), i))
    total = sum(Fraction(float(v)) for v in s)
    if mass >= 1 or total == 0:
        return list(range(L))
    chosen = set()
    if mass > 0:
        thr = Fraction(mass) * total
        run = Fraction(0)
        for k, i in enumerate(order):
            run += Fraction(float(s[i]))
            chosen.add(i)
            if run >= thr:
                break
    chosen |= set(range(max(0, L - recent_n), L))
    for i in order:
        if len(chosen) >= min_keep:
            break
        chosen.add(i)
    return sorted(chosen)


def test_token_select_matches_brute_force_on_exact_scores():
    rng = np.random.default_rng(5)
    for trial in range(60):
        L = int(rng.integers(1, 64))
        # small integers and halves: every fp64 partial sum is exact
        s = (rng.integers(0, 40, L) / 2.0).astype(np.float32)
        mass = float(rng.choice([0.0, 0.1, 0.3, 0.5, 0.7, 0.95, 1.0, 1.5]))
        recent = int(rng.integers(0, 5))
        mk = int(rng.integers(0, 4))
        keep, order, cum = oracle.token_select(s, mass, recent, mk)
        assert list(keep) == _brute_token_select(s, mass, recent, mk), (trial, L, mass, recent, mk)


def test_token_select_minimal_prefix_on_random_scores():
    s = np.exp(synth.normal_f32(9, (5000,))).astype(np.float32)
    for mass in (0.3, 0.5, 0.7):
        keep, order, cum = oracle.token_select(s, mass, 0, 0)
        total = math.fsum(float(v) for v in s)
        P = set(keep.tolist())
        m = len(P)
        assert P == set(order[:m].tolist())
        top = sorted(s.astype(np.float64), reverse=True)
        assert math.fsum(top[:m]) >= mass * total * (1 - 1e-12)
        assert math.fsum(top[:m - 1]) < mass * total * (1 + 1e-12)


def _ulp_units(s):
    """Each fp32 score >= 0 as an exact integer in units of the ulp of the
    smallest nonzero score (Python ints), and that ulp's exponent."""
    b = [int(x) for x in s.view(np.uint32)]
    nz = [max(x >> 23, 1) for x in b if x]
    emin = min(nz)
    q = [(((x & 0x7FFFFF) | (0x800000 if x >= 0x800000 else 0)) << (max(x >> 23, 1) - emin)) if x else 0 for x in b]
    return q, emin - 150


def test_exact_mass_condition_makes_the_blocked_prefix_order_free():
    """The shortcut the kernels take (an exactness theorem, not a reading of the
    pages): when the total is at most 2^53 ulps of the smallest nonzero score,
    every partial sum is an fp64 number, so the oracle's blocked fp64 prefix
    equals the exact prefix at every rank, whatever the order of the additions.
    Outside the condition the blocked prefix rounds, which is why the kernels
    then sort and add in order."""
    for seed, L in ((31, 1000), (32, 5000), (33, 16384)):
        s = (71.6 * np.exp(synth.normal_f32(seed, (L,)).astype(np.float64))).astype(np.float32)
        q, e = _ulp_units(s)
        assert sum(q) <= 2 ** 53
        _, order, cum = oracle.token_select(s, 0.5, 0, 1)
        run = 0
        for r, i in enumerate(order):
            run += q[i]
            assert cum[r] == math.ldexp(float(run), e), (seed, r)   # float(run) exact: run <= 2^53
    # 2^60 and then ones: past 2^53 ulps the blocked prefix rounds, the exact one does not
    s = np.array([2.0 ** 60] + [1.0] * 300, np.float32)
    q, e = _ulp_units(s)
    assert sum(q) > 2 ** 53
    _, order, cum = oracle.token_select(s, 0.5, 0, 1)
    assert Fraction(float(cum[-1])) != Fraction(2 ** 60 + 300)   # the blocked prefix rounds
    assert 300.0 + 2.0 ** 60 != cum[-1]                            # another order, other bits


def test_token_select_guards_and_degenerate_rows():
    s = np.exp(synth.normal_f32(10, (300,))).astype(np.float32)
    L = s.size
    assert list(oracle.token_select(s, 1.0, 0, 0)[0]) == list(range(L))     # mass >= 1: dense
    assert list(oracle.token_select(s, 0.2, L, 0)[0]) == list(range(L))     # recent_n >= L
    z = np.zeros(L, np.float32)
    assert list(oracle.token_select(z, 0.5, 0, 1)[0]) == list(range(L))     # all-zero: dense
    one = oracle.token_select(s, 0.0, 0, 1)[0]
    assert list(one) == [int(np.argmax(s))]                                 # just the top token
    five = oracle.token_select(s, 0.0, 0, 5)[0]
    assert sorted(five) == sorted(np.argsort(-s, kind="stable")[:5].tolist())
    keep = oracle.token_select(s, 0.3, 128, 1)[0]
    assert set(range(L - 128, L)) <= set(keep.tolist())                     # recent always kept
    tie = np.ones(10, np.float32)
    assert list(oracle.token_select(tie, 0.0, 0, 3)[0]) == [0, 1, 2]        # ties: lower index


@pytest.mark.parametrize("bad", [np.nan, np.inf])
def test_token_select_non_finite_total_keeps_every_token(bad):
    # a NaN or infinite score makes the total mass non-finite; the selection
    # then keeps every token, like the all-zero row (the pages define the mass
    # only for finite scores)
    s = np.exp(synth.normal_f32(11, (300,))).astype(np.float32)
    for pos in (0, 137, 299):
        t = s.copy()
        t[pos] = bad
        for mass, recent, mk in ((0.3, 0, 1), (0.0, 5, 3), (0.7, 128, 1)):
            assert list(oracle.token_select(t, mass, recent, mk)[0]) == list(range(300))
    # one sequence with a NaN keeps all of its tokens; the other one is unaffected
    t = s.copy()
    t[10] = bad
    cu = np.array([0, 150, 300], np.int32)
    keep = oracle.block_select(t, cu, block=16, mass=0.3, min_full=0.1, max_full=0.5, recent_n=0, min_keep=1)
    other = oracle.block_select(s[150:], np.array([0, 150], np.int32), block=16, mass=0.3, min_full=0.1,
                                max_full=0.5, recent_n=0, min_keep=1)
    assert list(keep) == list(range(150)) + [150 + int(i) for i in other]


def test_selection_only_decode_equals_the_full_call():
    w = tiny_weights(2, 256, 512, synth.ACT_SILU, seed=61)
    x = synth.normal_f32(62, (3, 256))
    for kw in (dict(mode="topk", topk_k=77, union=True), dict(mode="thresh", theta=0.52)):
        full = oracle.decode(w, x, **kw)
        sel = oracle.decode(w, x, outputs=False, **kw)
        assert sel["y"] is None
        for k in ("g", "u", "sel", "used", "idx"):
            assert np.array_equal(sel[k], full[k]), k


def test_token_select_blocked_cum_equals_exact_prefix_for_integer_scores():
    s = np.arange(1, 1001, dtype=np.float32)[::-1].copy()
    keep, order, cum = oracle.token_select(s, 0.5, 0, 0)
    exact = np.cumsum(np.sort(s.astype(np.float64))[::-1])
    assert np.array_equal(cum, exact)


def test_prefill_rows_match_fp64_numpy_and_unkept_rows_pass_through():
    d, f, L = 128, 256, 40
    w = tiny_weights(1, d, f, synth.ACT_SILU, seed=111)
    Y, A = synth.cfg5_activations(L=L, d=d)
    keep = np.array([0, 5, 6, 39], np.int32)
    X = oracle.prefill(w, Y, keep)
    Yf = synth.bf16_bits_to_f32(Y).astype(np.float64)
    Z = ffn_f64(w, Yf[keep], np.ones(f))
    assert rel_l2(oracle.prefill_rows(w, Y, keep), Z) < 1e-12
    rest = np.setdiff1d(np.arange(L), keep)
    assert np.array_equal(X[rest], Y[rest])
    Xk = synth.bf16_bits_to_f32(X[keep]).astype(np.float64)
    assert np.max(np.abs(Xk - (Yf[keep] + Z)) / np.maximum(np.abs(Yf[keep] + Z), 1e-30)) <= 2.0 ** -8
    full = oracle.prefill(w, Y, np.arange(L, dtype=np.int32))
    ref = oracle.bf16_rne(Yf + ffn_f64(w, Yf, np.ones(f)))
    assert np.array_equal(full, ref)


# ---------------------------------------------------------------------------
# adaptive expert top-K (RedKnot article, section on adaptive expert top-K)
# ---------------------------------------------------------------------------

def test_expert_page_parameters():
    g = json.load(open(GOLDEN))
    e = g["adaptive_expert_topk"]
    assert e["threshold"] == 0.5 and e["buckets"] == [3, 4, 5, 6] and e["native_experts_per_token"] == 6
    sched = g["progressive_topk_schedule"]["layers"]
    assert [k for _, _, k in sched] == [6, 5, 4]
    assert max(k for _, _, k in sched) == e["buckets"][-1]


def test_expert_select_hand_worked_cases():
    # confident token: 0.40 + 0.20 + 0.15 = 0.75 >= 0.5 at the smallest bucket
    p = np.array([[0.05, 0.40, 0.20, 0.15, 0.10, 0.05, 0.03, 0.02]], np.float32)
    k, idx, w = oracle.expert_select(p)
    assert k[0] == 3 and list(idx[0]) == [1, 2, 3, -1, -1, -1]
    assert list(w[0][:3]) == [np.float32(0.40), np.float32(0.20), np.float32(0.15)] and np.all(w[0][3:] == 0)
    # diffuse token: six of sixteen equal experts carry 6/16 < 0.5 -> the largest bucket, ties by index
    k, idx, _ = oracle.expert_select(np.full((1, 16), 1 / 16, np.float32))
    assert k[0] == 6 and list(idx[0]) == [0, 1, 2, 3, 4, 5]
    # eight experts of 1/8: the mass after four is exactly 0.5, which reaches the threshold
    k, idx, _ = oracle.expert_select(np.full((1, 8), 0.125, np.float32))
    assert k[0] == 4 and list(idx[0]) == [0, 1, 2, 3, -1, -1]
    # mass crosses between the third and the fourth expert: 0.2 + 3 x 0.1
    p = np.array([[0.2] + [0.1] * 8], np.float32)
    k, idx, _ = oracle.expert_select(p)
    assert k[0] == 4 and list(idx[0][:4]) == [0, 1, 2, 3]


def test_expert_select_threshold_limits_and_plain_topk():
    rng = np.random.default_rng(17)
    p = rng.dirichlet(np.ones(384), size=64).astype(np.float32)
    k0, _, _ = oracle.expert_select(p, tau=0.0)
    assert np.all(k0 == 3)
    k2, _, _ = oracle.expert_select(p, tau=2.0)
    assert np.all(k2 == 6)
    # kmin = kmax: plain top-k, equal to a stable sort of -p
    for kk in (1, 6, 16):
        k, idx, w = oracle.expert_select(p, kmin=kk, kmax=kk)
        assert np.all(k == kk)
        ref = np.argsort(-p, axis=1, kind="stable")[:, :kk]
        assert np.array_equal(idx, ref)
        assert np.array_equal(w, np.take_along_axis(p, ref, axis=1))


def test_expert_select_matches_exhaustive_subsets():
    # K = the smallest bucket b whose best b-subset of experts reaches tau; checked by
    # enumerating every subset in exact rational arithmetic (cases near a tie skipped)
    from fractions import Fraction
    from itertools import combinations
    rng = np.random.default_rng(23)
    checked = 0
    for _ in range(60):
        E = int(rng.integers(6, 10))
        p = rng.dirichlet(np.ones(E) * float(rng.choice([0.3, 1.0, 3.0]))).astype(np.float32)[None, :]
        tau = float(rng.choice([0.3, 0.5, 0.7]))
        best = {b: max(sum(Fraction(float(p[0, j])) for j in c) for c in combinations(range(E), b))
                for b in range(3, 7)}
        if any(abs(float(best[b]) - tau) < 1e-5 for b in best):
            continue
        want = next((b for b in range(3, 7) if best[b] >= Fraction(tau)), 6)
        k, idx, w = oracle.expert_select(p, tau=tau)
        assert k[0] == want
        # the chosen experts carry the best mass for that count
        assert sum(Fraction(float(v)) for v in w[0][:want]) == best[want]
        checked += 1
    assert checked >= 40


def test_expert_select_kept_experts_dominate_and_counts_follow_mass():
    rng = np.random.default_rng(29)
    logits = rng.standard_normal((200, 256)) * rng.uniform(0.5, 6.0, (200, 1))
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p = (p / p.sum(axis=1, keepdims=True)).astype(np.float32)
    k, idx, w = oracle.expert_select(p)
    assert set(np.unique(k)) <= {3, 4, 5, 6} and len(np.unique(k)) >= 3
    for t in range(p.shape[0]):
        sel = idx[t][: k[t]]
        rest = np.setdiff1d(np.arange(256), sel)
        assert p[t, sel].min() >= p[t, rest].max()
        # sharper routing (more mass in the top experts) never asks for more experts
    top3 = np.sort(p, axis=1)[:, ::-1][:, :3].sum(axis=1)
    assert k[top3 >= 0.5].max() == 3


# ---------------------------------------------------------------------------
# block-granular token selection and the layer schedule
# ---------------------------------------------------------------------------

def test_block_select_page_parameters():
    g = json.load(open(GOLDEN))["token_block_selection"]
    assert (g["block_tokens"], g["min_full_ratio"], g["max_full_ratio"]) == (128, 0.10, 0.50)
    assert g["min_keep_per_sequence"] >= 1


def test_block_select_hand_worked():
    s = np.arange(1, 9, dtype=np.float32)          # blocks of 2: masses 3, 7, 11, 15; total 36
    kw = dict(block=2, min_full=0.0, max_full=1.0, recent_n=0, min_keep=0)
    assert list(oracle.block_select(s, [0, 8], mass=0.5, **kw)) == [4, 5, 6, 7]        # 15 + 11 >= 18
    assert list(oracle.block_select(s, [0, 8], mass=0.4, **kw)) == [6, 7]              # 15 >= 14.4
    assert list(oracle.block_select(s, [0, 8], mass=0.42, **kw)) == [4, 5, 6, 7]       # 15 < 15.12
    assert oracle.block_select(s, [0, 8], mass=0.0, **kw).size == 0
    kw_recent = dict(kw, recent_n=1)                                                   # last token's block
    assert list(oracle.block_select(s, [0, 8], mass=0.0, **kw_recent)) == [6, 7]
    assert list(oracle.block_select(s, [0, 8], mass=0.0, **dict(kw, min_keep=3))) == [4, 5, 6, 7]
    # ragged last block: [1,2,3] [4,5,6] [7] -> masses 6, 15, 7
    s7 = np.arange(1, 8, dtype=np.float32)
    assert list(oracle.block_select(s7, [0, 7], block=3, mass=0.6, min_full=0.0, max_full=1.0,
                                    recent_n=0, min_keep=0)) == [3, 4, 5, 6]           # 15 + 7 >= 16.8


def test_block_select_bounds_and_their_fp32_rounding():
    L, B = 1280, 128                                # nb = 10
    s = np.ones(L, dtype=np.float32)
    kw = dict(block=B, recent_n=0, min_keep=0)
    # mass 0: the lower bound alone, ceilf(10 * 0.1f) = 1 (an fp64 product would give 2)
    assert oracle.block_select(s, [0, L], mass=0.0, min_full=0.1, max_full=0.5, **kw).size == B
    # equal masses: K = ceil(10 * mass) blocks, ties to the lower block index
    k = oracle.block_select(s, [0, L], mass=0.35, min_full=0.1, max_full=0.5, **kw)
    assert list(k) == list(range(4 * B))
    # the upper bound: 0.99 would need 10 blocks, capped at floor(10 * 0.5) = 5
    assert oracle.block_select(s, [0, L], mass=0.99, min_full=0.1, max_full=0.5, **kw).size == 5 * B
    # bounds that cross after rounding: nb = 3, ceilf(1.2) = 2 > floorf(1.5) = 1, the lower one wins
    s3 = np.ones(3 * B, dtype=np.float32)
    assert oracle.block_select(s3, [0, 3 * B], mass=0.0, min_full=0.4, max_full=0.5, **kw).size == 2 * B
    # mass >= 1 and all-zero scores are dense, whatever the upper bound
    assert oracle.block_select(s, [0, L], mass=1.0, min_full=0.1, max_full=0.5, **kw).size == L
    assert oracle.block_select(np.zeros(L, np.float32), [0, L], mass=0.3, min_full=0.1, max_full=0.5,
                               **kw).size == L
    with pytest.raises(ValueError):
        oracle.block_select(s, [0, L], min_full=0.6, max_full=0.5)
    with pytest.raises(ValueError):
        oracle.block_select(s, [0, L - 1])


@pytest.mark.parametrize("seed", range(6))
def test_block_select_with_one_token_blocks_is_token_select(seed):
    # block = 1, no bounds: block masses are the token scores and the cumulative
    # mass is sequential; for L <= 256 the token path's blocked sum is that same
    # sequence, so both selections must agree exactly
    rng = np.random.default_rng(900 + seed)
    L = int(rng.integers(1, 257))
    s = rng.integers(0, 6, size=L).astype(np.float32) * np.float32(0.25) if seed % 2 else \
        rng.random(L).astype(np.float32)
    for mass in (0.0, 0.3, 0.7, 1.0):
        for recent, mk in ((0, 0), (5, 1), (0, 40)):
            a = oracle.block_select(s, [0, L], block=1, mass=mass, min_full=0.0, max_full=1.0,
                                    recent_n=recent, min_keep=mk)
            b, _, _ = oracle.token_select(s, mass, recent, mk)
            assert np.array_equal(a, b), (L, mass, recent, mk)


def test_block_select_sequences_are_independent_and_runs_are_few():
    rng = np.random.default_rng(950)
    lens = [0, 1, 127, 128, 129, 700, 5000, 3]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    s = (np.exp(rng.standard_normal(cu[-1])) * rng.random(cu[-1])).astype(np.float32)
    kw = dict(block=128, mass=0.5, min_full=0.1, max_full=0.5, recent_n=128, min_keep=1)
    whole = oracle.block_select(s, cu, **kw)
    parts = [oracle.block_select(s[cu[q]:cu[q + 1]], [0, lens[q]], **kw) + cu[q] for q in range(len(lens))]
    assert np.array_equal(whole, np.concatenate(parts))
    for q, Lq in enumerate(lens):
        mine = whole[(whole >= cu[q]) & (whole < cu[q + 1])] - cu[q]
        if Lq:
            assert mine.size >= 1                                  # min_keep per sequence
            assert Lq - 1 in mine                                   # the recent tail
        nb = -(-Lq // 128)
        blocks = np.unique(mine // 128)
        assert all(np.array_equal(mine[mine // 128 == b], np.arange(b * 128, min(b * 128 + 128, Lq)))
                   for b in blocks)                                 # whole blocks only
        if nb >= 10:
            assert blocks.size <= math.floor(nb * 0.5) + 2          # budget + recent blocks


def test_layer_schedule_tiers_and_presets():
    g = json.load(open(GOLDEN))["ffn_layer_schedule"]
    du, mt, rn = g["presets"]["balanced"]
    assert (du, mt, rn) == (20, 0.5, 128)
    assert [oracle.schedule_mass(l, du, 40, mt, 0.2) for l in (0, 19, 20, 39, 40, 63)] == \
        [1.0, 1.0, 0.5, 0.5, 0.2, 0.2]
    # the dense preset keeps every layer of an 80-layer model dense
    du, mt, _ = g["presets"]["dense"]
    assert all(oracle.schedule_mass(l, du, du, mt, mt) == 1.0 for l in range(80))


# ---------------------------------------------------------------------------
# neuron order by activation frequency (WiSparse notes, section 5)
# ---------------------------------------------------------------------------

def test_frequency_order_hand_worked():
    # counts 5 1 4 2 3 0: ranks 0, 2, 4, 3, 1, 5.  Balance over 3 blocks of 2:
    # snake 0 1 2 2 1 0 -> {0, 5}, {2, 1}, {4, 3}, each block ascending.
    c = np.array([5, 1, 4, 2, 3, 0], np.int32)
    assert oracle.frequency_order(c, "cluster").tolist() == [0, 2, 4, 3, 1, 5]
    assert oracle.frequency_order(c, "balance", 2).tolist() == [0, 5, 1, 2, 3, 4]


@pytest.mark.parametrize("f,seed", [(97, 1), (1408, 2), (4096, 3)])
def test_frequency_order_cluster_is_the_ranking(f, seed):
    c = np.random.default_rng(seed).integers(0, 9, f).astype(np.int32)
    p = oracle.frequency_order(c, "cluster")
    assert sorted(p.tolist()) == list(range(f))
    cc = c[p]
    assert np.all(cc[:-1] >= cc[1:])                      # counts never increase
    tie = cc[:-1] == cc[1:]
    assert np.all(p[:-1][tie] < p[1:][tie])               # ties: lower index first


@pytest.mark.parametrize("f,block,seed", [(1408, 11, 1), (11008, 43, 2), (960, 48, 3)])
def test_frequency_order_balance_spreads_the_counts(f, block, seed):
    c = (np.random.default_rng(seed).pareto(1.2, f) * 10).astype(np.int32)   # a few very hot neurons
    p = oracle.frequency_order(c, "balance", block)
    assert sorted(p.tolist()) == list(range(f))
    blocks = p.reshape(-1, block)
    assert np.all(np.diff(blocks, axis=1) > 0)            # each block ascending
    sums = c[blocks].sum(axis=1)
    # a snake over a non-increasing sequence keeps any two blocks within one count of each other
    assert sums.max() - sums.min() <= c.max()
    # contiguous blocks of the original order are far less even
    orig = c.reshape(-1, block).sum(axis=1)
    assert sums.max() - sums.min() < orig.max() - orig.min()


def test_frequency_order_balance_special_cases():
    c = np.random.default_rng(7).integers(0, 5, 300).astype(np.int32)
    # one block: every neuron in it, ascending -> the identity
    assert np.array_equal(oracle.frequency_order(c, "balance", 300), np.arange(300))
    # blocks of one: the first pass of the snake hands out the ranking in order
    assert np.array_equal(oracle.frequency_order(c, "balance", 1), oracle.frequency_order(c, "cluster"))
