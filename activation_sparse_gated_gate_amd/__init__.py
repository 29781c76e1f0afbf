"""Python binding of libsffn, the gfx950 activation-sparse gated FFN library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/sffn.h``.  PyTorch supplies
device memory (``tensor.data_ptr()``) and streams
(``torch.cuda.current_stream().cuda_stream``).  Importing this package loads
``libsffn.so`` from this directory and raises if it has not been built: there
is no fallback path.

The functions ``sffn_workspace_size``, ``sffn_create``, ``sffn_select``,
``sffn_forward``, ``sffn_destroy`` and ``sffn_status_string`` mirror the C
entry points; ``Layer`` wraps them with workspace allocation.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsffn.so")

SFFN_OK, SFFN_ERR_INVALID_ARG, SFFN_ERR_UNSUPPORTED, SFFN_ERR_WORKSPACE, SFFN_ERR_HIP = 0, 1, 2, 3, 4
W_F32, W_BF16, W_INT4_G128 = 0, 1, 2
ACT_RELU, ACT_SILU = 0, 1
MODE_ALL, MODE_EXACT, MODE_THRESH, MODE_TOPK, MODE_TOKENS, MODE_DENSE = 0, 1, 2, 3, 4, 5
LAYOUT_DECODE, LAYOUT_PREFILL, LAYOUT_BATCH = 1, 2, 4
MODES = {"all": MODE_ALL, "exact": MODE_EXACT, "thresh": MODE_THRESH, "topk": MODE_TOPK,
         "tokens": MODE_TOKENS, "dense": MODE_DENSE}

EXPORTS = ("sffn_workspace_size", "sffn_create", "sffn_select", "sffn_forward", "sffn_destroy",
           "sffn_status_string", "sffn_last_hip_error", "sffn_set_kernel_timer", "sffn_expert_select",
           "sffn_select_blocks", "sffn_schedule_mass", "sffn_neuron_counts", "sffn_frequency_order",
           "sffn_decode_block_rows", "sffn_create_permuted", "sffn_read_probe", "sffn_forward_noalloc",
           "sffn_noalloc_scratch_bytes", "sffn_read_probe_cfg", "sffn_read_latency_probe",
           "sffn_token_select_path")


class LayerDesc(C.Structure):
    _fields_ = [("d_model", C.c_int32), ("d_ff", C.c_int32), ("max_rows", C.c_int32),
                ("wtype", C.c_int32), ("act", C.c_int32), ("rmsnorm", C.c_int32),
                ("residual", C.c_int32), ("eps", C.c_float), ("layouts", C.c_int32)]


class Policy(C.Structure):
    _fields_ = [("mode", C.c_int32), ("gate_bias", C.c_float), ("theta", C.c_float),
                ("topk_k", C.c_int32), ("use_union", C.c_int32), ("recent_n", C.c_int32),
                ("min_keep", C.c_int32), ("batch_path", C.c_int32), ("merge_gap", C.c_int32),
                ("reserved", C.c_int32), ("mass_thresh", C.c_double)]


class ExpertPolicy(C.Structure):
    _fields_ = [("tau", C.c_float), ("kmin", C.c_int32), ("kmax", C.c_int32), ("reserved", C.c_int32)]


class BlockPolicy(C.Structure):
    _fields_ = [("mass_thresh", C.c_double), ("min_full_ratio", C.c_float), ("max_full_ratio", C.c_float),
                ("block", C.c_int32), ("recent_n", C.c_int32), ("min_keep", C.c_int32), ("reserved", C.c_int32)]


class ProbeCfg(C.Structure):
    _fields_ = [("workgroups", C.c_int32), ("threads", C.c_int32), ("pattern", C.c_int32),
                ("in_flight", C.c_int32), ("nontemporal", C.c_int32)]


class SffnError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = "%s: %s" % (what, sffn_status_string(status))
        if status == SFFN_ERR_HIP:
            msg += " (%s)" % _lib.sffn_last_hip_error().decode()
        super().__init__(msg)
        self.status = status


def _load():
    # torch first: libsffn then binds to the HIP runtime torch already loaded
    # (same soname), so both share one runtime, one device context and streams.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError("libsffn.so is not built (%s); run __graft_entry__.build() or "
                          "python activation_sparse_gated_gate_amd/build.py" % LIB_PATH)
    lib = C.CDLL(LIB_PATH)
    P, I, Z = C.c_void_p, C.c_int32, C.c_size_t
    lib.sffn_workspace_size.argtypes = [C.POINTER(LayerDesc), C.POINTER(Z), C.POINTER(Z)]
    lib.sffn_workspace_size.restype = I
    lib.sffn_create.argtypes = [C.POINTER(LayerDesc), P, P, P, P, P, P, P, Z, P, C.POINTER(P)]
    lib.sffn_create.restype = I
    lib.sffn_select.argtypes = [P, C.POINTER(Policy), P, I, P, P, P, Z, P]
    lib.sffn_select.restype = I
    lib.sffn_forward.argtypes = [P, C.POINTER(Policy), P, I, P, P, P, P, P, P, Z, P]
    lib.sffn_forward.restype = I
    lib.sffn_forward_noalloc.argtypes = [P, C.POINTER(Policy), P, I, P, P, P, P, P, P]
    lib.sffn_forward_noalloc.restype = I
    lib.sffn_noalloc_scratch_bytes.argtypes = []
    lib.sffn_noalloc_scratch_bytes.restype = Z
    lib.sffn_destroy.argtypes = [P]
    lib.sffn_destroy.restype = None
    lib.sffn_status_string.argtypes = [I]
    lib.sffn_status_string.restype = C.c_char_p
    lib.sffn_last_hip_error.argtypes = []
    lib.sffn_last_hip_error.restype = C.c_char_p
    lib.sffn_set_kernel_timer.argtypes = [P, P, P, I]
    lib.sffn_select_blocks.restype = I
    lib.sffn_select_blocks.argtypes = [P, C.POINTER(BlockPolicy), P, I, P, I, P, P, P, Z, P]
    lib.sffn_schedule_mass.restype = C.c_double
    lib.sffn_schedule_mass.argtypes = [I, I, I, C.c_double, C.c_double]
    lib.sffn_expert_select.restype = I
    lib.sffn_expert_select.argtypes = [P, I, I, C.POINTER(ExpertPolicy), P, P, P, P]
    lib.sffn_set_kernel_timer.restype = I
    lib.sffn_neuron_counts.restype = I
    lib.sffn_neuron_counts.argtypes = [P, P, I, P, P]
    lib.sffn_frequency_order.restype = I
    lib.sffn_frequency_order.argtypes = [P, I, I, I, P]
    lib.sffn_decode_block_rows.restype = I
    lib.sffn_decode_block_rows.argtypes = [I]
    lib.sffn_read_probe.restype = I
    lib.sffn_read_probe.argtypes = [P, Z, I, P, P]
    lib.sffn_read_probe_cfg.restype = I
    lib.sffn_read_probe_cfg.argtypes = [P, Z, C.POINTER(ProbeCfg), P, P]
    lib.sffn_read_latency_probe.restype = I
    lib.sffn_read_latency_probe.argtypes = [P, Z, I, P, I, P, P]
    lib.sffn_token_select_path.restype = I
    lib.sffn_token_select_path.argtypes = [P, P, Z, P, P]
    lib.sffn_create_permuted.restype = I
    lib.sffn_create_permuted.argtypes = [C.POINTER(LayerDesc), P, P, P, P, P, Z, P, C.POINTER(P)]
    return lib


_lib = _load()


# ---------------------------------------------------------------------------
# the C entry points, one to one
# ---------------------------------------------------------------------------

def sffn_status_string(status: int) -> str:
    return _lib.sffn_status_string(int(status)).decode()


def sffn_workspace_size(desc: LayerDesc):
    """Returns (status, persistent_bytes, scratch_bytes)."""
    p, s = C.c_size_t(0), C.c_size_t(0)
    st = _lib.sffn_workspace_size(C.byref(desc), C.byref(p), C.byref(s))
    return st, p.value, s.value


def sffn_create(desc, w_gate, w_up, w_down, s_gate, s_up, s_down, persistent, persistent_bytes, stream):
    """Pointers are ints (device addresses) or None.  Returns (status, handle)."""
    h = C.c_void_p(0)
    st = _lib.sffn_create(C.byref(desc), w_gate, w_up, w_down, s_gate, s_up, s_down, persistent,
                          persistent_bytes, stream, C.byref(h))
    return st, h.value


def sffn_select(handle, policy, inp, rows, idx_out, count_out, scratch, scratch_bytes, stream) -> int:
    return _lib.sffn_select(handle, C.byref(policy), inp, int(rows), idx_out, count_out, scratch,
                            scratch_bytes, stream)


def sffn_forward(handle, policy, inp, rows, out, idx_in, count_in, idx_out, count_out, scratch,
                 scratch_bytes, stream) -> int:
    return _lib.sffn_forward(handle, C.byref(policy), inp, int(rows), out, idx_in, count_in, idx_out,
                             count_out, scratch, scratch_bytes, stream)


def sffn_forward_noalloc(handle, policy, inp, rows, out, idx_in, count_in, idx_out, count_out, stream) -> int:
    return _lib.sffn_forward_noalloc(handle, C.byref(policy), inp, int(rows), out, idx_in, count_in, idx_out,
                                     count_out, stream)


def sffn_noalloc_scratch_bytes() -> int:
    return int(_lib.sffn_noalloc_scratch_bytes())


def sffn_destroy(handle) -> None:
    _lib.sffn_destroy(handle)


def sffn_select_blocks(handle, policy, A, rows, cu_seqlens, nseq, idx_out, count_out, scratch, scratch_bytes,
                       stream) -> int:
    return _lib.sffn_select_blocks(handle, C.byref(policy), A, int(rows), cu_seqlens, int(nseq), idx_out,
                                   count_out, scratch, scratch_bytes, stream)


def sffn_schedule_mass(layer, dense_until, deep_layer_start, mass_thresh, mass_thresh_deep) -> float:
    return float(_lib.sffn_schedule_mass(int(layer), int(dense_until), int(deep_layer_start), float(mass_thresh),
                                         float(mass_thresh_deep)))


def make_block_policy(mass_thresh=0.5, min_full_ratio=0.10, max_full_ratio=0.50, block=128, recent_n=128,
                      min_keep=1) -> BlockPolicy:
    return BlockPolicy(float(mass_thresh), float(min_full_ratio), float(max_full_ratio), int(block), int(recent_n),
                       int(min_keep), 0)


def sffn_expert_select(probs, tokens, experts, policy, k_out, idx_out, w_out, stream) -> int:
    return _lib.sffn_expert_select(probs, int(tokens), int(experts), C.byref(policy), k_out, idx_out, w_out,
                                   stream)


def expert_select(probs, tau=0.5, kmin=3, kmax=6, k_out=None, idx_out=None, w_out=None, stream=None):
    """Adaptive expert top-K on device probabilities [T, E] (fp32): returns (K [T] int32,
    experts [T, kmax] int32, probabilities [T, kmax] fp32), all device tensors."""
    import torch
    T, E = probs.shape
    dev = probs.device
    k_out = k_out if k_out is not None else torch.empty(T, dtype=torch.int32, device=dev)
    idx_out = idx_out if idx_out is not None else torch.empty((T, kmax), dtype=torch.int32, device=dev)
    w_out = w_out if w_out is not None else torch.empty((T, kmax), dtype=torch.float32, device=dev)
    st = (stream if stream is not None else torch.cuda.current_stream()).cuda_stream
    pol = ExpertPolicy(float(tau), int(kmin), int(kmax), 0)
    status = sffn_expert_select(probs.data_ptr(), T, E, pol, k_out.data_ptr(), idx_out.data_ptr(),
                                w_out.data_ptr(), st)
    if status != SFFN_OK:
        raise SffnError(status, "sffn_expert_select")
    return k_out, idx_out, w_out


def sffn_set_kernel_timer(handle, begin_events, end_events, n) -> int:
    """begin_events / end_events: ctypes arrays of hipEvent_t handles (or None when n = 0)."""
    return _lib.sffn_set_kernel_timer(handle, begin_events, end_events, int(n))


# ---------------------------------------------------------------------------
# convenience wrapper over torch-owned memory
# ---------------------------------------------------------------------------

BATCH_PATH_AUTO, BATCH_PATH_TILED, BATCH_PATH_GATHER = 0, 1, 2


def make_policy(mode="all", gate_bias=0.0, theta=0.0, topk_k=1, use_union=False, mass_thresh=1.0,
                recent_n=0, min_keep=1, batch_path=BATCH_PATH_AUTO, merge_gap=0) -> Policy:
    m = MODES[mode] if isinstance(mode, str) else int(mode)
    return Policy(m, float(gate_bias), float(theta), int(topk_k), int(bool(use_union)), int(recent_n),
                  int(min_keep), int(batch_path), int(merge_gap), 0, float(mass_thresh))


def _ptr(t):
    return None if t is None else t.data_ptr()


ORDER_CLUSTER, ORDER_BALANCE = 0, 1


def neuron_counts(idx, count, counts, stream=None):
    """counts[idx[q]] += 1 for q < count (device int32 tensors; sffn_neuron_counts)."""
    import torch
    s = (stream if stream is not None else torch.cuda.current_stream()).cuda_stream
    st = _lib.sffn_neuron_counts(idx.data_ptr(), count.data_ptr(), int(counts.numel()), counts.data_ptr(), s)
    if st != SFFN_OK:
        raise SffnError(st, "sffn_neuron_counts")


def frequency_order(counts, mode=ORDER_CLUSTER, block=1):
    """Host int32 counts [d_ff] -> perm [d_ff] (sffn_frequency_order)."""
    import numpy as np
    c = np.ascontiguousarray(counts, dtype=np.int32)
    perm = np.empty(c.size, np.int32)
    st = _lib.sffn_frequency_order(c.ctypes.data, int(c.size), int(mode), int(block), perm.ctypes.data)
    if st != SFFN_OK:
        raise SffnError(st, "sffn_frequency_order")
    return perm


def decode_block_rows(d_ff: int) -> int:
    """Consecutive neurons per workgroup of the batch-1 kernel (sffn_decode_block_rows)."""
    return int(_lib.sffn_decode_block_rows(int(d_ff)))


class Layer:
    """One FFN layer on the current CUDA (HIP) device.

    weights: dict with device tensors 'w_gate', 'w_up', 'w_down' and, for int4,
    's_gate', 's_up', 's_down' (uint8 packed / int16-viewed fp16 bits, natural
    layout as documented in sffn.h).  The persistent and scratch workspaces are
    torch uint8 tensors owned by this object.
    """

    def __init__(self, d_model, d_ff, max_rows, wtype, act, weights, rmsnorm=False, residual=False,
                 eps=1e-6, layouts=LAYOUT_DECODE, stream=None, perm=None):
        import torch
        self.desc = LayerDesc(int(d_model), int(d_ff), int(max_rows), int(wtype), int(act),
                              int(bool(rmsnorm)), int(bool(residual)), float(eps), int(layouts))
        st, pb, sb = sffn_workspace_size(self.desc)
        if st != SFFN_OK:
            raise SffnError(st, "sffn_workspace_size")
        dev = weights["w_gate"].device
        self.persistent = torch.empty(pb, dtype=torch.uint8, device=dev)
        self.scratch = torch.empty(sb, dtype=torch.uint8, device=dev)
        self.persistent_bytes, self.scratch_bytes = pb, sb
        s = self._stream(stream)
        if perm is None:
            st, h = sffn_create(self.desc, _ptr(weights["w_gate"]), _ptr(weights["w_up"]),
                                _ptr(weights["w_down"]), _ptr(weights.get("s_gate")),
                                _ptr(weights.get("s_up")), _ptr(weights.get("s_down")),
                                self.persistent.data_ptr(), pb, s)
        else:
            # perm: device int32 [d_ff], new neuron j = original neuron perm[j]
            hh = C.c_void_p()
            st = _lib.sffn_create_permuted(C.byref(self.desc), _ptr(weights["w_gate"]), _ptr(weights["w_up"]),
                                           _ptr(weights["w_down"]), perm.data_ptr(), self.persistent.data_ptr(),
                                           pb, s, C.byref(hh))
            h = hh.value
        if st != SFFN_OK:
            raise SffnError(st, "sffn_create")
        self.handle = h

    @staticmethod
    def _stream(stream):
        import torch
        return (stream if stream is not None else torch.cuda.current_stream()).cuda_stream

    def select(self, policy: Policy, inp, idx_out, count_out, stream=None):
        st = sffn_select(self.handle, policy, inp.data_ptr(), inp.shape[0], idx_out.data_ptr(),
                         count_out.data_ptr(), self.scratch.data_ptr(), self.scratch_bytes,
                         self._stream(stream))
        if st != SFFN_OK:
            raise SffnError(st, "sffn_select")

    def token_select_path(self, stream=None) -> int:
        """Which path made the last token selection on this layer's scratch:
        1 the exact-mass radix select, 2 the sort (sffn_token_select_path)."""
        import torch
        out = torch.full((1,), -1, dtype=torch.int32, device=self.scratch.device)
        st = _lib.sffn_token_select_path(self.handle, self.scratch.data_ptr(), self.scratch_bytes,
                                         out.data_ptr(), self._stream(stream))
        if st != SFFN_OK:
            raise SffnError(st, "sffn_token_select_path")
        return int(out.item())

    def select_blocks(self, policy: BlockPolicy, A, cu_seqlens, idx_out, count_out, stream=None):
        st = sffn_select_blocks(self.handle, policy, A.data_ptr(), A.shape[0], cu_seqlens.data_ptr(),
                                cu_seqlens.shape[0] - 1, idx_out.data_ptr(), count_out.data_ptr(),
                                self.scratch.data_ptr(), self.scratch_bytes, self._stream(stream))
        if st != SFFN_OK:
            raise SffnError(st, "sffn_select_blocks")

    def forward(self, policy: Policy, inp, out, idx_in=None, count_in=None, idx_out=None,
                count_out=None, stream=None):
        st = sffn_forward(self.handle, policy, inp.data_ptr(), inp.shape[0], out.data_ptr(),
                          _ptr(idx_in), _ptr(count_in), _ptr(idx_out), _ptr(count_out),
                          self.scratch.data_ptr(), self.scratch_bytes, self._stream(stream))
        if st != SFFN_OK:
            raise SffnError(st, "sffn_forward")

    def forward_noalloc(self, policy: Policy, inp, out, idx_in=None, count_in=None, idx_out=None,
                        count_out=None, stream=None):
        """sffn_forward_noalloc: as forward, on the library's built-in scratch."""
        st = sffn_forward_noalloc(self.handle, policy, inp.data_ptr(), inp.shape[0], out.data_ptr(),
                                  _ptr(idx_in), _ptr(count_in), _ptr(idx_out), _ptr(count_out),
                                  self._stream(stream))
        if st != SFFN_OK:
            raise SffnError(st, "sffn_forward_noalloc")

    def close(self):
        if getattr(self, "handle", None):
            sffn_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
