"""CPU oracle for the activation-sparse gated FFN (ctypes wrapper of oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  The HIP library never imports, links or calls it and
shares no code with it; the two meet only in the seeded inputs of ``synth``.

Every function forwards to the plain C implementation in ``oracle.c``; the
definitions, the passages they follow and the fixed fp32 / fp64 orders used
for selection decisions are documented there.  ``build()`` compiles the
library with gcc if it is missing (or always, when asked).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ALL, EXACT, THRESH, TOPK = 0, 1, 2, 3
MODES = {"all": ALL, "exact": EXACT, "thresh": THRESH, "topk": TOPK}

_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so (gcc, -O2 -ffp-contract=off, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-D_DEFAULT_SOURCE", "-ffp-contract=off", "-fno-fast-math",
               "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build()
    lib = C.CDLL(_LIB)
    P = C.c_void_p
    I = C.c_int
    F = C.c_float
    D = C.c_double
    lib.ora_dot_c1.argtypes = [I, I, I, P, P, I, P]
    lib.ora_dot_c1.restype = F
    lib.ora_rms_scale.argtypes = [P, I, F]
    lib.ora_rms_scale.restype = F
    lib.ora_exp64.argtypes = [D]
    lib.ora_exp64.restype = D
    lib.ora_silu64.argtypes = [D]
    lib.ora_silu64.restype = D
    lib.ora_score.argtypes = [F, F, D]
    lib.ora_score.restype = D
    lib.ora_down_col_norms.argtypes = [I, I, I, P, P, P]
    lib.ora_down_col_norms.restype = None
    lib.ora_decode.argtypes = [I, I, I, I, P, P, P, P, P, P, I, F, I, I, F, F, I, I, I, P,
                               P, P, P, P, P, P, P, I]
    lib.ora_decode.restype = I
    lib.ora_token_norms.argtypes = [P, I, I, P, I]
    lib.ora_token_norms.restype = None
    lib.ora_token_select.argtypes = [P, I, D, I, I, P, P, P]
    lib.ora_token_select.restype = I
    lib.ora_prefill_rows.argtypes = [I, I, P, P, P, P, P, I, P, I]
    lib.ora_block_select.argtypes = [P, I, P, I, I, D, F, F, I, I, P]
    lib.ora_block_select.restype = I
    lib.ora_schedule_mass.argtypes = [I, I, I, D, D]
    lib.ora_schedule_mass.restype = D
    lib.ora_expert_select.argtypes = [P, I, I, F, I, I, P, P, P]
    lib.ora_frequency_order.restype = C.c_int
    lib.ora_frequency_order.argtypes = [P, I, I, I, P]
    lib.ora_expert_select.restype = I
    lib.ora_prefill_rows.restype = None
    lib.ora_bf16_rne.argtypes = [D]
    lib.ora_bf16_rne.restype = C.c_uint16
    lib.ora_bf16_rne_array.argtypes = [P, C.c_size_t, P]
    lib.ora_bf16_rne_array.restype = None
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dt):
    return None if a is None else np.ascontiguousarray(a, dtype=dt)


def _wdtype(wt):
    return {0: np.float32, 1: np.uint16, 2: np.uint8}[wt]


def default_threads() -> int:
    return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

def dot_c1(wt, w, scales, r, x) -> np.float32:
    """Row r of W (natural layout) dotted with x in the fixed fp32 order."""
    lib = _load()
    w = _c(w, _wdtype(wt))
    rows = w.shape[0]
    cols = w.shape[1] * (2 if wt == 2 else 1)
    x = _c(x, np.float32)
    s = _c(scales, np.uint16)
    return np.float32(lib.ora_dot_c1(wt, rows, cols, _p(w), _p(s), int(r), _p(x)))


def rms_scale(x, eps=1e-6) -> np.float32:
    x = _c(x, np.float32)
    return np.float32(_load().ora_rms_scale(_p(x), x.size, eps))


def exp64(z: float) -> float:
    return _load().ora_exp64(float(z))


def silu64(g: float) -> float:
    return _load().ora_silu64(float(g))


def score(g: float, u: float, n: float) -> float:
    return _load().ora_score(float(np.float32(g)), float(np.float32(u)), float(n))


def down_col_norms(weights) -> np.ndarray:
    w = weights
    out = np.empty(w.d_ff, dtype=np.float64)
    wd = _c(w.w_down, _wdtype(w.wtype))
    sd = _c(w.s_down, np.uint16)
    _load().ora_down_col_norms(w.wtype, w.d_model, w.d_ff, _p(wd), _p(sd), _p(out))
    return out


def decode(weights, x, mode="all", bias=0.0, theta=0.0, topk_k=1, union=False,
           rmsnorm=False, eps=1e-6, residual=False, threads=None, outputs=True):
    """One gated-FFN layer over the rows of x (fp32 [B, d]).

    Returns a dict: y (fp64 [B, d]; x + y when residual), xhat, g (gate
    pre-activation + bias in the fixed fp32 order), u (TOPK only), sel (each
    token's own selection, bool [B, f]), used (the mask its output sums over),
    idx (ascending indices of the union of the used masks), wdn (TOPK column
    norms).  outputs=False computes the selection only (y is None).
    """
    w = weights
    lib = _load()
    x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.float32)
    B, d = x.shape
    f = w.d_ff
    assert d == w.d_model
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    dt = _wdtype(w.wtype)
    wg, wu, wd = _c(w.w_gate, dt), _c(w.w_up, dt), _c(w.w_down, dt)
    sg, su, sd = _c(w.s_gate, np.uint16), _c(w.s_up, np.uint16), _c(w.s_down, np.uint16)
    xhat = np.empty((B, d), np.float32)
    g = np.empty((B, f), np.float32)
    u = np.zeros((B, f), np.float32)
    sel = np.empty((B, f), np.uint8)
    used = np.empty((B, f), np.uint8)
    y = np.empty((B, d), np.float64) if outputs else None
    wdn = np.zeros(f, np.float64)
    rc = lib.ora_decode(w.wtype, d, f, w.act, _p(wg), _p(sg), _p(wu), _p(su), _p(wd), _p(sd),
                        int(rmsnorm), float(eps), int(residual), m, float(bias), float(theta),
                        int(topk_k), int(union), B, _p(x), _p(xhat), _p(g), _p(u), _p(sel),
                        _p(used), _p(y), _p(wdn), int(threads or default_threads()))
    if rc != 0:
        raise ValueError("oracle decode rejected its arguments")
    idx = np.flatnonzero(used.any(axis=0)).astype(np.int32)
    return dict(y=y, xhat=xhat, g=g, u=u, sel=sel.astype(bool), used=used.astype(bool),
                idx=idx, wdn=wdn)


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------

def token_norms(A_bf16, threads=None) -> np.ndarray:
    A = _c(A_bf16, np.uint16)
    L, d = A.shape
    s = np.empty(L, np.float32)
    _load().ora_token_norms(_p(A), L, d, _p(s), int(threads or default_threads()))
    return s


def token_select(s, mass, recent_n=128, min_keep=1):
    """Returns (keep ascending int32, order int32, cum fp64)."""
    s = _c(s, np.float32)
    L = s.size
    keep = np.empty(max(L, 1), np.int32)
    order = np.empty(max(L, 1), np.int32)
    cum = np.empty(max(L, 1), np.float64)
    n = _load().ora_token_select(_p(s), L, float(mass), int(recent_n), int(min_keep), _p(keep),
                                 _p(order), _p(cum))
    if n < 0:
        raise ValueError("oracle token_select rejected its arguments")
    return keep[:n].copy(), order[:L].copy(), cum[:L].copy()


def block_select(s, cu_seqlens, block=128, mass=0.5, min_full=0.10, max_full=0.50, recent_n=128, min_keep=1):
    """Block-granular token selection over sequences [cu[q], cu[q+1]): the kept
    token indices in ascending order (see ora_block_select)."""
    s = _c(s, np.float32)
    cu = _c(cu_seqlens, np.int32)
    rows = s.size
    keep = np.empty(max(rows, 1), dtype=np.int32)
    n = _load().ora_block_select(_p(s), rows, _p(cu), cu.size - 1, int(block), float(mass),
                                 float(min_full), float(max_full), int(recent_n), int(min_keep), _p(keep))
    if n < 0:
        raise ValueError("oracle block_select rejected its arguments")
    return keep[:n].copy()


def schedule_mass(layer, dense_until, deep_layer_start, mass_thresh, mass_thresh_deep) -> float:
    return float(_load().ora_schedule_mass(int(layer), int(dense_until), int(deep_layer_start),
                                           float(mass_thresh), float(mass_thresh_deep)))


def expert_select(probs, tau=0.5, kmin=3, kmax=6):
    """Adaptive expert top-K: returns (K int32 [T], idx int32 [T, kmax], w fp32 [T, kmax])."""
    p = _c(probs, np.float32)
    T, E = p.shape
    k = np.empty(max(T, 1), np.int32)
    idx = np.empty((max(T, 1), kmax), np.int32)
    w = np.empty((max(T, 1), kmax), np.float32)
    if _load().ora_expert_select(_p(p), T, E, float(tau), int(kmin), int(kmax), _p(k), _p(idx), _p(w)) != 0:
        raise ValueError("oracle expert_select rejected its arguments")
    return k[:T].copy(), idx[:T].copy(), w[:T].copy()


def frequency_order(counts, mode="cluster", block=1) -> np.ndarray:
    """Neuron order by activation count: perm[j] = the neuron at position j
    (mode 'cluster' or 'balance' over blocks of `block` positions)."""
    c = _c(counts, np.int32)
    perm = np.empty(max(c.size, 1), np.int32)
    m = {"cluster": 0, "balance": 1}[mode]
    if _load().ora_frequency_order(_p(c), int(c.size), m, int(block), _p(perm)) != 0:
        raise ValueError("oracle frequency_order rejected its arguments")
    return perm[:c.size].copy()


def prefill_rows(weights, Y_bf16, rows, threads=None) -> np.ndarray:
    """Z (fp64 [n, d]) of the listed rows of Y through the SwiGLU FFN."""
    w = weights
    assert w.wtype == 1
    Y = _c(Y_bf16, np.uint16)
    rows = _c(rows, np.int32)
    Z = np.empty((rows.size, w.d_model), np.float64)
    _load().ora_prefill_rows(w.d_model, w.d_ff, _p(_c(w.w_gate, np.uint16)),
                             _p(_c(w.w_up, np.uint16)), _p(_c(w.w_down, np.uint16)), _p(Y),
                             _p(rows), rows.size, _p(Z), int(threads or default_threads()))
    return Z


def bf16_rne(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint16)
    _load().ora_bf16_rne_array(_p(v), v.size, _p(out))
    return out


def prefill(weights, Y_bf16, keep, threads=None) -> np.ndarray:
    """X_next (bf16 bits [L, d]): Y + FFN(Y) on the kept rows, Y elsewhere."""
    Y = _c(Y_bf16, np.uint16)
    X = Y.copy()
    if len(keep):
        Z = prefill_rows(weights, Y, keep, threads)
        yk = (Y[keep].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        X[keep] = bf16_rne(yk + Z)
    return X


# ---------------------------------------------------------------------------
# closed forms of the cost model
# ---------------------------------------------------------------------------

def kept_fraction(a: float) -> float:
    """Fraction of FFN bytes / work kept under exact gating: the gate is read
    in full and W_up / W_down only for the active fraction a, (1 + 2a) / 3
    (denseflux, section 3, cost metric; section 5.3)."""
    return (1.0 + 2.0 * a) / 3.0


def ideal_speedup(a: float) -> float:
    """The speed-up ceiling implied by the kept bytes, 3 / (1 + 2a)."""
    return 1.0 / kept_fraction(a)


def group_active_probability(a: float, k: int) -> float:
    """Probability that a group of k independent neurons, each active with
    probability a, has at least one active member, 1 - (1 - a)^k (denseflux,
    section 4.2).  The same law gives the expected union density of a batch."""
    return 1.0 - (1.0 - a) ** k
