"""HIP graph capture of every entry point's launches: each graph is replayed
several times on new inputs copied into its captured buffers, with eager work
of the same layer in between, and every replay must equal the eager call on
the same inputs bit for bit (all kernels are deterministic).  This covers the
device-side decisions inside a graph: the batched path switch, the device
counts that size the prefill GEMMs and the block selection."""
import numpy as np
import pytest

import synth

from gpu_util import make_layer, tensor

pytestmark = pytest.mark.gpu


def _sf():
    import activation_sparse_gated_gate_amd as sf
    return sf


def capture(fn):
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        fn()                                  # warm-up outside the capture
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return g


def replay_and_compare(g, inputs, bufs, outs, eager):
    """For each input set: copy into the captured buffers, replay, then run the
    eager call on the same inputs into fresh outputs and compare bitwise."""
    import torch
    for vals in inputs:
        for b, v in zip(bufs, vals):
            b.copy_(v)
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        ref = eager(vals)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), "graph replay differs from the eager call"


def test_decode_batch1_graph():
    import torch
    sf = _sf()
    w = synth._make_weights(synth.WT_BF16, 1024, 2816, synth.ACT_RELU, (1931, 1932, 1933))
    layer = make_layer(w, 1)
    pol = sf.make_policy("exact", gate_bias=synth.gate_offset_for_active_fraction(0.1))
    xs = [tensor(synth.round_to_bf16(synth.normal_f32(1934 + i, (1, 1024)))) for i in range(4)]
    xb, yb = xs[0].clone(), torch.empty_like(xs[0])
    g = capture(lambda: layer.forward(pol, xb, yb))

    def eager(vals):
        y = torch.empty_like(vals[0])
        layer.forward(pol, vals[0], y)
        return [y]
    replay_and_compare(g, [[x] for x in xs[1:]] + [[xs[0]]], [xb], [yb], eager)
    layer.close()


def test_decode_batched_graph_switches_paths_inside_the_graph():
    import torch
    sf = _sf()
    d, f = 1024, 2048
    w = synth._make_weights(synth.WT_BF16, d, f, synth.ACT_RELU, (1941, 1942, 1943))
    layer = make_layer(w, 16, layouts=sf.LAYOUT_DECODE | sf.LAYOUT_BATCH)
    pol = sf.make_policy("exact", gate_bias=synth.gate_offset_for_active_fraction(0.01), use_union=True)
    x = tensor(synth.round_to_bf16(synth.normal_f32(1944, (5, d))))
    # scaled inputs move the union across the breakeven: small scale -> few active
    scales = [1.0, 40.0, 0.5, 25.0]
    idx = torch.empty(f, dtype=torch.int32, device=x.device)
    cnt = torch.empty(1, dtype=torch.int32, device=x.device)
    union = []
    for s in scales:
        layer.select(pol, x * s, idx, cnt)
        torch.cuda.synchronize()
        union.append(int(cnt.item()) / f)
    assert min(union) < 0.2 and max(union) > 0.5, union   # both sides of the 5-token breakeven (0.25)
    xb, yb = x.clone(), torch.empty_like(x)
    g = capture(lambda: layer.forward(pol, xb, yb))

    def eager(vals):
        y = torch.empty_like(vals[0])
        layer.forward(pol, vals[0], y)
        return [y]
    replay_and_compare(g, [[x * s] for s in scales], [xb], [yb], eager)
    layer.close()


def test_prefill_select_and_forward_graph():
    import torch
    sf = _sf()
    w = synth._make_weights(synth.WT_BF16, 512, 1024, synth.ACT_SILU, (1951, 1952, 1953))
    L = 1000
    layer = sf.Layer(512, 1024, L, sf.W_BF16, sf.ACT_SILU,
                     {k: tensor(getattr(w, k)) for k in ("w_gate", "w_up", "w_down")}, layouts=sf.LAYOUT_PREFILL)
    sets = []
    for i in range(3):
        Y, A = synth.cfg5_activations(L=L, d=512) if i == 0 else (
            synth.f32_to_bf16_bits(synth.normal_f32(1960 + i, (L, 512))),
            synth.f32_to_bf16_bits(synth.normal_f32(1970 + i, (L, 512)) * np.float32(1 + i)))
        sets.append([tensor(Y), tensor(A)])
    Yb, Ab = sets[0][0].clone(), sets[0][1].clone()
    keep = torch.empty(L, dtype=torch.int32, device=Yb.device)
    cnt = torch.empty(1, dtype=torch.int32, device=Yb.device)
    X = torch.empty_like(Yb)
    psel = sf.make_policy("tokens", mass_thresh=0.5, recent_n=64, min_keep=1)
    pfwd = sf.make_policy("tokens")

    def run(Yt, At, keep_t, cnt_t, Xt):
        layer.select(psel, At, keep_t, cnt_t)
        layer.forward(pfwd, Yt, Xt, idx_in=keep_t, count_in=cnt_t)
    g = capture(lambda: run(Yb, Ab, keep, cnt, X))

    def eager(vals):
        k2 = torch.full_like(keep, -1)
        c2 = torch.empty_like(cnt)
        x2 = torch.empty_like(X)
        run(vals[0], vals[1], k2, c2, x2)
        n = int(c2.item())
        k2[n:] = keep[n:]   # entries past the count are not part of the result
        return [x2, c2, k2]
    replay_and_compare(g, sets[1:] + sets[:1], [Yb, Ab], [X, cnt, keep], eager)
    layer.close()


def test_block_selection_and_expert_select_graph():
    import torch
    sf = _sf()
    w = synth._make_weights(synth.WT_BF16, 512, 1024, synth.ACT_SILU, (1981, 1982, 1983))
    L = 3000
    layer = sf.Layer(512, 1024, L, sf.W_BF16, sf.ACT_SILU,
                     {k: tensor(getattr(w, k)) for k in ("w_gate", "w_up", "w_down")}, layouts=sf.LAYOUT_PREFILL)
    cu = torch.tensor([0, 1000, 1001, 2500, 3000], dtype=torch.int32, device="cuda:0")
    As = [tensor(synth.f32_to_bf16_bits(synth.normal_f32(1990 + i, (L, 512))
                                         * np.exp(synth.normal_f32(1995 + i, (L, 1))))) for i in range(3)]
    P = [tensor(synth.router_probs(777, 384, seed=2000 + i)) for i in range(3)]
    Ab, Pb = As[0].clone(), P[0].clone()
    keep = torch.empty(L, dtype=torch.int32, device=Ab.device)
    cnt = torch.empty(1, dtype=torch.int32, device=Ab.device)
    k = torch.empty(777, dtype=torch.int32, device=Ab.device)
    idx = torch.empty((777, 6), dtype=torch.int32, device=Ab.device)
    wv = torch.empty((777, 6), dtype=torch.float32, device=Ab.device)
    bpol = sf.make_block_policy(0.5, 0.1, 0.5, 128, 128, 1)

    def run(At, Pt, keep_t, cnt_t, k_t, idx_t, w_t):
        layer.select_blocks(bpol, At, cu, keep_t, cnt_t)
        sf.expert_select(Pt, 0.5, 3, 6, k_out=k_t, idx_out=idx_t, w_out=w_t)
    g = capture(lambda: run(Ab, Pb, keep, cnt, k, idx, wv))

    def eager(vals):
        outs = [torch.full_like(keep, -1), torch.empty_like(cnt), torch.empty_like(k), torch.empty_like(idx),
                torch.empty_like(wv)]
        run(vals[0], vals[1], *outs)
        n = int(outs[1].item())
        outs[0][n:] = keep[n:]
        return [outs[1], outs[0], outs[2], outs[3], outs[4]]
    replay_and_compare(g, [[As[i], P[i]] for i in (1, 2, 0)], [Ab, Pb], [cnt, keep, k, idx, wv], eager)
    layer.close()
