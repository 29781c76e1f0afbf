"""Helpers for the GPU parity tests: upload seeded inputs, run the C ABI,
compare with the oracle.  Nothing here computes the FFN."""
from __future__ import annotations

import numpy as np


def dev():
    import torch
    return torch.device("cuda:0")


def tensor(a: np.ndarray):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(dev())


def weights_on_device(w):
    out = {"w_gate": tensor(w.w_gate), "w_up": tensor(w.w_up), "w_down": tensor(w.w_down)}
    if w.s_gate is not None:
        out.update(s_gate=tensor(w.s_gate), s_up=tensor(w.s_up), s_down=tensor(w.s_down))
    return out


def make_layer(w, max_rows, rmsnorm=False, residual=False, layouts=None):
    import activation_sparse_gated_gate_amd as sf
    return sf.Layer(w.d_model, w.d_ff, max_rows, w.wtype, w.act, weights_on_device(w), rmsnorm=rmsnorm,
                    residual=residual, layouts=layouts or sf.LAYOUT_DECODE)


def align256(v):
    return (v + 255) & ~255


def scratch_views(layer, B):
    """Views of the decode scratch: x_hat [B, d] and g' [B, f] (fp32).  Offsets
    follow the library's scratch layout for a decode layer: x_hat first, then
    g' (both sized by max_rows)."""
    import torch
    d, f, mr = layer.desc.d_model, layer.desc.d_ff, layer.desc.max_rows
    s = layer.scratch
    xh = s[:mr * d * 4].view(torch.float32)[:B * d].view(B, d)
    o = align256(mr * d * 4)
    g = s[o:o + mr * f * 4].view(torch.float32)[:B * f].view(B, f)
    o2 = align256(o + mr * f * 4)
    u = s[o2:o2 + mr * f * 4].view(torch.float32)[:B * f].view(B, f)
    return xh, g, u


def run_decode(layer, policy, x: np.ndarray, want_list=True):
    """Returns (y float32 [B, d], idx int32 ascending, count)."""
    import torch
    xt = tensor(np.ascontiguousarray(x, np.float32))
    y = torch.empty_like(xt)
    f = layer.desc.d_ff
    idx = torch.full((f,), -1, dtype=torch.int32, device=dev()) if want_list else None
    cnt = torch.full((1,), -1, dtype=torch.int32, device=dev()) if want_list else None
    layer.forward(policy, xt, y, idx_out=idx, count_out=cnt)
    torch.cuda.synchronize()
    if not want_list:
        return y.cpu().numpy(), None, None
    n = int(cnt.item())
    return y.cpu().numpy(), idx[:n].cpu().numpy(), n


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a))
