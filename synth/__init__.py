"""Seeded synthetic inputs for the activation-sparse gated FFN.

This module holds only input preparation: seeded normal draws, the fp32 ->
bf16 storage rounding, the symmetric int4 group quantiser that produces the
stored weight format, and the workload parameters (gate offsets and
thresholds) that turn an active fraction into a number.  None of the FFN's
own arithmetic lives here.  Both the CPU oracle and the HIP path receive the
exact same bytes from these generators.

Recipes (one seed per tensor, numpy PCG64, float64 draws scaled then cast to
fp32 with round-to-nearest-even):

* config 1: fp32 weights, d_model 512, d_ff 1408, N(0, 1/512); 64 tokens N(0,1).
* config 2: bf16 weights at the Llama-2-7B FFN shape (4096 / 11008), N(0, 1/d_in);
  tokens N(0,1) rounded to bf16-representable fp32.
* config 3: Qwen2.5-3B FFN shape (2048 / 11008), weights N(0, 1/d_in) quantised to
  int4 in groups of 128 along the input dimension with fp16 scales.
* config 4: 28 layers at 3584 / 18944, bf16, N(0, 1/d_in); input [16 x 3584] N(0,1).
* config 5: d_model 5120, d_ff 25600, L = 16384; Y ~ N(0,1) bf16; the attention
  output A has rows r_i * eps_i with r_i = exp(N(0,1)) (log-normal row scales)
  and eps_i ~ N(0, I); weights N(0, 1/d_in) bf16.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# ---------------------------------------------------------------------------
# primitive draws and storage formats
# ---------------------------------------------------------------------------

_CHUNK_ELEMS = 1 << 24  # draw at most 16M float64 values at a time


def normal_f32(seed: int, shape, sigma: float = 1.0) -> np.ndarray:
    """N(0, sigma^2) drawn in float64 from PCG64(seed), scaled, then cast to fp32.

    Large tensors are drawn in row chunks from the one generator, which yields
    the same stream as a single call.
    """
    shape = tuple(int(s) for s in shape)
    g = np.random.Generator(np.random.PCG64(seed))
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(-1)
    n = flat.size
    pos = 0
    while pos < n:
        m = min(_CHUNK_ELEMS, n - pos)
        flat[pos:pos + m] = (g.standard_normal(m, dtype=np.float64) * sigma).astype(np.float32)
        pos += m
    return out


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 values that are exactly representable in bf16 (RNE)."""
    return bf16_bits_to_f32(f32_to_bf16_bits(a))


QGROUP = 128


def quantize_int4_g128(w: np.ndarray):
    """Symmetric int4 quantiser producing the stored weight format.

    w: fp32 [rows, cols] with groups of 128 consecutive columns (the input
    dimension).  Per group s = fp16(max|w| / 7) (s = 0 gives q = 0) and
    q = clamp(rne(w / s), -8, 7).  Nibbles are two's complement, the even
    column in the low nibble.

    Returns (packed uint8 [rows, cols/2], scales as fp16 bit patterns uint16
    [rows, cols/128]).
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    assert cols % QGROUP == 0
    g = w.reshape(rows, cols // QGROUP, QGROUP)
    amax = np.abs(g).max(axis=2)
    s16 = (amax / np.float32(7.0)).astype(np.float16)
    s32 = s16.astype(np.float32)
    safe = np.where(s32 > 0, s32, np.float32(1.0))
    q = np.rint(g / safe[:, :, None])
    q = np.where(s32[:, :, None] > 0, q, 0.0)
    q = np.clip(q, -8, 7).astype(np.int8).reshape(rows, cols)
    nib = (q.astype(np.int16) & 0xF).astype(np.uint8)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return np.ascontiguousarray(packed), np.ascontiguousarray(s16.view(np.uint16))


def dequantize_int4_g128(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Inverse of the storage format (for building test inputs, not for checking)."""
    rows = packed.shape[0]
    lo = (packed & 0xF).astype(np.int16)
    hi = (packed >> 4).astype(np.int16)
    q = np.empty((rows, packed.shape[1] * 2), dtype=np.int16)
    q[:, 0::2] = lo
    q[:, 1::2] = hi
    q = np.where(q >= 8, q - 16, q).astype(np.float32)
    s = scales.view(np.float16).astype(np.float32)
    return q * np.repeat(s, QGROUP, axis=1)


# ---------------------------------------------------------------------------
# workload parameters
# ---------------------------------------------------------------------------

def gate_offset_for_active_fraction(a: float) -> float:
    """Offset b = -Phi^-1(1 - a) for the gate pre-activation so that a fraction
    a of N(0,1) gate values is positive after the offset (fp64, then fp32)."""
    from scipy.special import ndtri
    return float(np.float32(-ndtri(1.0 - a)))


def gate_threshold_for_active_fraction(a: float) -> float:
    """theta = Phi^-1(1 - a): the gate-domain threshold that keeps a fraction a
    of N(0,1) gate values (fp64, then fp32)."""
    from scipy.special import ndtri
    return float(np.float32(ndtri(1.0 - a)))


def topk_count(n: int, pct: int) -> int:
    """k = max(1, floor(n * pct / 100)) in integer arithmetic."""
    return max(1, (n * pct) // 100)


# ---------------------------------------------------------------------------
# weights container
# ---------------------------------------------------------------------------

WT_F32, WT_BF16, WT_I4 = 0, 1, 2
ACT_RELU, ACT_SILU = 0, 1


@dataclass
class FFNWeights:
    """One gated-FFN layer in its natural storage layout.

    w_gate, w_up: [d_ff, d_model] row-major (row j = neuron j).
    w_down: [d_model, d_ff] row-major (column j = neuron j).
    fp32 -> float32 arrays; bf16 -> uint16 bit patterns; int4 -> packed uint8
    [rows, cols/2] plus fp16-bit scales [rows, cols/128] in s_*.
    """
    wtype: int
    d_model: int
    d_ff: int
    act: int
    w_gate: np.ndarray
    w_up: np.ndarray
    w_down: np.ndarray
    s_gate: np.ndarray | None = None
    s_up: np.ndarray | None = None
    s_down: np.ndarray | None = None
    meta: dict = field(default_factory=dict)


def _make_weights(wtype, d, f, act, seeds, sigma_in=None, rows_sub=None):
    sg = math.sqrt(1.0 / d)
    sd = math.sqrt(1.0 / f)
    wg = normal_f32(seeds[0], (f, d), sg)
    wu = normal_f32(seeds[1], (f, d), sg)
    wd = normal_f32(seeds[2], (d, f), sd)
    if wtype == WT_F32:
        return FFNWeights(wtype, d, f, act, wg, wu, wd)
    if wtype == WT_BF16:
        return FFNWeights(wtype, d, f, act, f32_to_bf16_bits(wg), f32_to_bf16_bits(wu), f32_to_bf16_bits(wd))
    pg, qg = quantize_int4_g128(wg)
    pu, qu = quantize_int4_g128(wu)
    pd, qd = quantize_int4_g128(wd)
    return FFNWeights(wtype, d, f, act, pg, pu, pd, qg, qu, qd)


def skewed_weights(wtype, d, f, act, seeds, sigma_row=0.6):
    """As _make_weights (fp32 / bf16), with row j of W_gate scaled by
    exp(sigma_row * z_j), z ~ N(0, 1) from seeds[3]: neurons then differ in how
    often they pass the gate, the skew that neuron reordering by activation
    frequency works on (real models have hot and cold neurons; the plain
    workloads' neurons are all alike)."""
    sg = math.sqrt(1.0 / d)
    sd = math.sqrt(1.0 / f)
    scale = np.exp(sigma_row * np.random.Generator(np.random.PCG64(seeds[3])).standard_normal(f))
    wg = (normal_f32(seeds[0], (f, d), sg).astype(np.float64) * scale[:, None]).astype(np.float32)
    wu = normal_f32(seeds[1], (f, d), sg)
    wd = normal_f32(seeds[2], (d, f), sd)
    if wtype == WT_F32:
        return FFNWeights(wtype, d, f, act, wg, wu, wd)
    assert wtype == WT_BF16
    return FFNWeights(wtype, d, f, act, f32_to_bf16_bits(wg), f32_to_bf16_bits(wu), f32_to_bf16_bits(wd))


def permuted_weights(w, perm):
    """The same layer with its neurons stored in the order perm (new j = old perm[j])."""
    return FFNWeights(w.wtype, w.d_model, w.d_ff, w.act, np.ascontiguousarray(w.w_gate[perm]),
                      np.ascontiguousarray(w.w_up[perm]), np.ascontiguousarray(w.w_down[:, perm]))


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

def cfg1_weights():
    return _make_weights(WT_F32, 512, 1408, ACT_RELU, (101, 102, 103))


def cfg1_tokens(n=64):
    return normal_f32(150, (n, 512))


CFG1_ACTIVE = 0.2


def cfg2_weights(d=4096, f=11008):
    return _make_weights(WT_BF16, d, f, ACT_RELU, (201, 202, 203))


def cfg2_tokens(n=1024, d=4096):
    return round_to_bf16(normal_f32(250, (n, d)))


CFG2_ACTIVE = (1.0, 0.6, 0.3, 0.1)


def cfg3_weights(d=2048, f=11008):
    return _make_weights(WT_I4, d, f, ACT_SILU, (301, 302, 303))


def cfg3_tokens(n=1024, d=2048):
    return normal_f32(350, (n, d))


CFG3_KEEP_PCT = (17, 30, 50)


CFG4_LAYERS = 28
CFG4_D, CFG4_F, CFG4_B = 3584, 18944, 16


def cfg4_layer_weights(layer, d=CFG4_D, f=CFG4_F):
    base = 4000 + 10 * layer
    return _make_weights(WT_BF16, d, f, ACT_SILU, (base + 1, base + 2, base + 3))


def cfg4_input(b=CFG4_B, d=CFG4_D):
    return normal_f32(4050, (b, d))


def cfg4_schedule(layer):
    """(mode, active fraction) for layer `layer` of the 28-layer stack:
    layers 0-7 dense, 8-19 a ~ 0.3, 20-27 a ~ 0.13."""
    if layer < 8:
        return ("all", 1.0)
    if layer < 20:
        return ("thresh", 0.3)
    return ("thresh", 0.13)


CFG5_D, CFG5_F, CFG5_L = 5120, 25600, 16384
CFG5_MASS = (0.3, 0.5, 0.7, 1.0)
CFG5_RECENT, CFG5_MIN_KEEP = 128, 1


def cfg5_weights(d=CFG5_D, f=CFG5_F):
    return _make_weights(WT_BF16, d, f, ACT_SILU, (501, 502, 503))


def cfg5_activations(L=CFG5_L, d=CFG5_D):
    """(Y, A) as bf16 bit patterns [L, d]: Y ~ N(0,1); A_i = r_i * eps_i with
    r_i = exp(N(0,1)) and eps_i ~ N(0, I)."""
    y = f32_to_bf16_bits(normal_f32(551, (L, d)))
    eps = normal_f32(552, (L, d))
    r = np.exp(normal_f32(553, (L,)).astype(np.float64)).astype(np.float32)
    a = f32_to_bf16_bits(eps * r[:, None])
    return y, a


# ---------------------------------------------------------------------------
# adaptive expert top-K: router probabilities
# ---------------------------------------------------------------------------

EXPERT_E = (384, 256)             # routed experts (Pro / Flash models of the RedKnot article)
EXPERT_T = 16384                  # tokens per call: one prefill-sized batch
EXPERT_TAU, EXPERT_KMIN, EXPERT_KMAX = 0.5, 3, 6
EXPERT_DEPTH_KMAX = ((0, 15, 6), (16, 39, 5), (40, 60, 4))   # progressive per-depth cap


def router_probs(T=EXPERT_T, E=EXPERT_E[0], seed=601):
    """Router probabilities [T, E] fp32: per token a softmax over E of s_t * z_tj
    with z ~ N(0, 1) and a sharpness s_t log-uniform on [2, 4], so that some
    tokens put most of their mass on a few experts and others spread it (the
    mass-0.5 rule then picks every bucket 3..6).  Softmax in float64, stored
    fp32 with round-to-nearest-even."""
    rng = np.random.default_rng(seed)
    s = np.exp(rng.uniform(math.log(2.0), math.log(4.0), T))
    out = np.empty((T, E), dtype=np.float32)
    step = max(1, _CHUNK_ELEMS // max(E, 1))
    for t0 in range(0, T, step):
        t1 = min(T, t0 + step)
        z = rng.standard_normal((t1 - t0, E)) * s[t0:t1, None]
        z -= z.max(axis=1, keepdims=True)
        e = np.exp(z)
        out[t0:t1] = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    return out
