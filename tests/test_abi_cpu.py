"""Host-side checks of the C-ABI library (no GPU needed).

The library loads, exports every symbol include/sffn.h declares, and rejects
bad descriptors / arguments before it would touch the GPU.
"""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


def _declared():
    src = "".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"\b(sffn_[a-z_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("sffn_workspace_size", "sffn_create", "sffn_select", "sffn_forward", "sffn_destroy",
              "sffn_status_string"):
        assert n in names


def test_library_exports_every_declared_symbol():
    import activation_sparse_gated_gate_amd as sf
    lib = C.CDLL(sf.LIB_PATH)
    for n in _declared():
        assert hasattr(lib, n), n
    assert set(sf.EXPORTS) >= set(_declared())


def _desc(**kw):
    import activation_sparse_gated_gate_amd as sf
    base = dict(d_model=4096, d_ff=11008, max_rows=1, wtype=sf.W_BF16, act=sf.ACT_RELU, rmsnorm=0,
                residual=0, eps=1e-6, layouts=sf.LAYOUT_DECODE)
    base.update(kw)
    return sf.LayerDesc(*[base[k] for k, _ in sf.LayerDesc._fields_])


def test_workspace_sizes_cover_the_layouts():
    import activation_sparse_gated_gate_amd as sf
    st, pb, sb = sf.sffn_workspace_size(_desc())
    assert st == sf.SFFN_OK
    mat = 4096 * 11008 * 2
    assert pb >= 4 * mat + 11008 * 8        # W_gate, W_up, W_down^T, W_down, norms
    assert sb >= 256 * 4096 * 4             # partial sums
    st, pb5, sb5 = sf.sffn_workspace_size(_desc(d_model=5120, d_ff=25600, max_rows=16384,
                                                act=sf.ACT_SILU, layouts=sf.LAYOUT_PREFILL))
    assert st == sf.SFFN_OK
    assert pb5 >= 3 * 5120 * 25600 * 2
    assert sb5 >= 16384 * 25600 * 2
    # the MFMA tile copies of W_up and W_down for batched decode
    st, pbb, sbb = sf.sffn_workspace_size(_desc(layouts=sf.LAYOUT_DECODE | sf.LAYOUT_BATCH, max_rows=16))
    assert st == sf.SFFN_OK and pbb >= pb + 2 * mat


@pytest.mark.parametrize("kw,status", [
    (dict(d_model=4000), 1), (dict(d_ff=1000), 1), (dict(max_rows=0), 1), (dict(max_rows=17), 1),
    (dict(wtype=3), 1), (dict(act=2), 1), (dict(layouts=0), 1), (dict(layouts=4), 1),
    (dict(wtype=2, max_rows=16), 2), (dict(layouts=2, wtype=0, act=1), 2),
    (dict(layouts=2, act=0), 2), (dict(layouts=2, max_rows=16385, act=1), 1),
    (dict(layouts=8), 1), (dict(layouts=5, wtype=0), 2), (dict(layouts=5, wtype=2, act=1), 2),
    (dict(layouts=6, act=1), 2),
])
def test_descriptor_validation(kw, status):
    import activation_sparse_gated_gate_amd as sf
    st, _, _ = sf.sffn_workspace_size(_desc(**kw))
    assert st == status


def test_create_rejects_bad_arguments_before_any_launch():
    import activation_sparse_gated_gate_amd as sf
    d = _desc()
    st, pb, _ = sf.sffn_workspace_size(d)
    fake = 1 << 20  # never dereferenced: validation fails first
    assert sf.sffn_create(d, None, fake, fake, None, None, None, fake, pb, None)[0] == sf.SFFN_ERR_INVALID_ARG
    assert sf.sffn_create(d, fake, fake, fake, fake, None, None, fake, pb, None)[0] == sf.SFFN_ERR_INVALID_ARG
    assert sf.sffn_create(d, fake, fake, fake, None, None, None, fake + 16, pb, None)[0] == sf.SFFN_ERR_INVALID_ARG
    assert sf.sffn_create(d, fake, fake, fake, None, None, None, fake, pb - 1, None)[0] == sf.SFFN_ERR_WORKSPACE
    d4 = _desc(wtype=sf.W_INT4_G128, act=sf.ACT_SILU, d_model=2048)
    st, pb4, _ = sf.sffn_workspace_size(d4)
    assert sf.sffn_create(d4, fake, fake, fake, None, None, None, fake, pb4, None)[0] == sf.SFFN_ERR_INVALID_ARG


def test_select_forward_reject_null_handle():
    import activation_sparse_gated_gate_amd as sf
    p = sf.make_policy("exact")
    assert sf.sffn_forward(None, p, 1 << 20, 1, 1 << 21, None, None, None, None, 1 << 22, 1, None) == 1
    assert sf.sffn_select(None, p, 1 << 20, 1, 1 << 21, 1 << 21, 1 << 22, 1, None) == 1


def test_status_strings():
    import activation_sparse_gated_gate_amd as sf
    assert sf.sffn_status_string(0) == "ok"
    assert sf.sffn_status_string(3) == "workspace too small"
    assert sf.sffn_status_string(99) == "unknown status"


@pytest.mark.parametrize("T,E,tau,kmin,kmax,ptrs,status", [
    (0, 384, 0.5, 3, 6, False, 0),            # no tokens: nothing to do, no pointer needed
    (4, 384, 0.5, 3, 6, False, 1),            # tokens without buffers
    (-1, 384, 0.5, 3, 6, True, 1),
    (4, 0, 0.5, 1, 1, True, 1),
    (4, 1025, 0.5, 3, 6, True, 1),            # more experts than one wave holds
    (4, 384, 0.5, 0, 6, True, 1),             # kmin < 1
    (4, 384, 0.5, 4, 3, True, 1),             # kmin > kmax
    (4, 5, 0.5, 3, 6, True, 1),               # kmax > experts
    (4, 384, 0.5, 3, 17, True, 1),            # kmax above the per-token limit
    (4, 384, float("nan"), 3, 6, True, 1),
])
def test_expert_select_validation(T, E, tau, kmin, kmax, ptrs, status):
    import activation_sparse_gated_gate_amd as sf
    fake = (1 << 20) if ptrs else None   # never dereferenced: validation fails first
    pol = sf.ExpertPolicy(tau, kmin, kmax, 0)
    if status == 0:
        assert sf.sffn_expert_select(fake, T, E, pol, fake, fake, fake, None) == 0
    else:
        assert sf.sffn_expert_select(fake, T, E, pol, fake, fake, fake, None) == sf.SFFN_ERR_INVALID_ARG


def test_expert_select_rejects_null_policy():
    import activation_sparse_gated_gate_amd as sf
    lib = C.CDLL(sf.LIB_PATH)
    lib.sffn_expert_select.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p,
                                       C.c_void_p, C.c_void_p]
    assert lib.sffn_expert_select(None, 0, 384, None, None, None, None, None) == sf.SFFN_ERR_INVALID_ARG


def test_select_blocks_rejects_null_handle_and_policy():
    import activation_sparse_gated_gate_amd as sf
    fake = 1 << 20   # never dereferenced: validation fails first
    pol = sf.make_block_policy()
    assert sf.sffn_select_blocks(None, pol, fake, 16, fake, 1, fake, fake, fake, 1 << 20, None) == \
        sf.SFFN_ERR_INVALID_ARG
    lib = C.CDLL(sf.LIB_PATH)
    lib.sffn_select_blocks.argtypes = [C.c_void_p] * 4 + [C.c_void_p, C.c_int32] + [C.c_void_p] * 3 + \
        [C.c_size_t, C.c_void_p]
    lib.sffn_select_blocks.argtypes[3] = C.c_int32
    assert lib.sffn_select_blocks(fake, None, fake, 16, fake, 1, fake, fake, fake, 1 << 20, None) == \
        sf.SFFN_ERR_INVALID_ARG


def test_schedule_mass_matches_the_oracle():
    import activation_sparse_gated_gate_amd as sf
    import oracle
    for du, deep in ((3, 40), (20, 40), (32, 48), (80, 80), (0, 0)):
        for layer in range(0, 82, 3):
            assert sf.sffn_schedule_mass(layer, du, deep, 0.5, 0.2) == oracle.schedule_mass(layer, du, deep, 0.5, 0.2)


# ---------------------------------------------------------------------------
# neuron reordering: host logic (no GPU)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("f,block,seed", [(6, 2, 1), (1408, 6, 2), (11008, 43, 3), (1000, 48, 4), (777, 1, 5),
                                          (512, 512, 6)])
def test_frequency_order_matches_the_oracle(f, block, seed):
    import numpy as np

    import activation_sparse_gated_gate_amd as sf
    import oracle
    rng = np.random.default_rng(seed)
    counts = rng.integers(0, 40, f).astype(np.int32)   # many ties
    for mode, name in ((sf.ORDER_CLUSTER, "cluster"), (sf.ORDER_BALANCE, "balance")):
        got = sf.frequency_order(counts, mode, block)
        ref = oracle.frequency_order(counts, name, block)
        assert np.array_equal(got, ref), name


def test_frequency_order_and_create_permuted_validation():
    import numpy as np

    import activation_sparse_gated_gate_amd as sf
    lib = sf._lib
    c = np.zeros(8, np.int32)
    p = np.zeros(8, np.int32)
    assert lib.sffn_frequency_order(None, 8, 0, 1, p.ctypes.data) == sf.SFFN_ERR_INVALID_ARG
    assert lib.sffn_frequency_order(c.ctypes.data, 8, 2, 1, p.ctypes.data) == sf.SFFN_ERR_INVALID_ARG
    assert lib.sffn_frequency_order(c.ctypes.data, 8, 1, 0, p.ctypes.data) == sf.SFFN_ERR_INVALID_ARG
    assert lib.sffn_frequency_order(c.ctypes.data, 8, 1, 9, p.ctypes.data) == sf.SFFN_ERR_INVALID_ARG
    c[3] = -1
    assert lib.sffn_frequency_order(c.ctypes.data, 8, 0, 1, p.ctypes.data) == sf.SFFN_ERR_INVALID_ARG
    assert lib.sffn_neuron_counts(None, None, 8, None, None) == sf.SFFN_ERR_INVALID_ARG
    assert [sf.decode_block_rows(f) for f in (0, 128, 1408, 11008, 12288, 18944)] == [0, 1, 6, 43, 48, 48]
    h = C.c_void_p()
    d = _desc(wtype=sf.W_INT4_G128)
    assert lib.sffn_create_permuted(C.byref(d), 16, 16, 16, 16, 256, 1 << 40, None, C.byref(h)) == \
        sf.SFFN_ERR_UNSUPPORTED
    d = _desc()
    assert lib.sffn_create_permuted(C.byref(d), 16, 16, 16, None, 256, 1 << 40, None, C.byref(h)) == \
        sf.SFFN_ERR_INVALID_ARG


def test_read_probe_validation():
    import activation_sparse_gated_gate_amd as sf
    lib = sf._lib
    assert lib.sffn_read_probe(None, 1024, 1, 16, None) == sf.SFFN_ERR_INVALID_ARG
    assert lib.sffn_read_probe(256, 1000, 1, 16, None) == sf.SFFN_ERR_INVALID_ARG     # size not a multiple of 16
    assert lib.sffn_read_probe(264, 1024, 1, 16, None) == sf.SFFN_ERR_INVALID_ARG     # misaligned
    assert lib.sffn_read_probe(256, 1024, 0, 16, None) == sf.SFFN_ERR_INVALID_ARG     # no workgroups
    assert lib.sffn_read_probe(256, 1024, 1, None, None) == sf.SFFN_ERR_INVALID_ARG


def test_bench_refuses_more_than_one_gpu():
    # one GPU only: the benchmark exits with a message before it touches a device
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_policy_layout_matches_the_header():
    import ctypes as C

    import activation_sparse_gated_gate_amd as sf
    assert C.sizeof(sf.Policy) == 48
    assert sf.Policy.merge_gap.offset == 32 and sf.Policy.mass_thresh.offset == 40
    assert C.sizeof(sf.ProbeCfg) == 20


def test_probe_cfg_and_latency_probe_validation():
    import ctypes as C

    import activation_sparse_gated_gate_amd as sf
    lib = sf._lib
    ok = sf.ProbeCfg(256, 1024, 0, 8, 1)
    assert lib.sffn_read_probe_cfg(None, 1024, C.byref(ok), 16, None) == sf.SFFN_ERR_INVALID_ARG
    for bad in (sf.ProbeCfg(0, 1024, 0, 8, 1), sf.ProbeCfg(256, 300, 0, 8, 1), sf.ProbeCfg(256, 1024, 2, 8, 1),
                sf.ProbeCfg(256, 1024, 0, 5, 1), sf.ProbeCfg(256, 1024, 0, 8, 2)):
        assert lib.sffn_read_probe_cfg(256, 1024, C.byref(bad), 16, None) == sf.SFFN_ERR_INVALID_ARG
    assert lib.sffn_read_latency_probe(None, 4096, 1024, 16, 4, 16, None) == sf.SFFN_ERR_INVALID_ARG
    assert lib.sffn_read_latency_probe(256, 4096, 1000, 16, 4, 16, None) == sf.SFFN_ERR_INVALID_ARG   # row size
    assert lib.sffn_read_latency_probe(256, 512, 1024, 16, 4, 16, None) == sf.SFFN_ERR_INVALID_ARG    # buffer < row
    assert lib.sffn_read_latency_probe(256, 4096, 1024, 16, 0, 16, None) == sf.SFFN_ERR_INVALID_ARG   # n
