"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects invalid arguments before touching the device."""
import ctypes
import os
import re
import subprocess

import pytest

from dsa_top_sparse_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

OK, NULL, SHAPE, DTYPE, UNSUP, WS, DEV, ALIGN = 0, -1, -2, -3, -4, -5, -6, -7
FAKE = 1 << 20  # an aligned address that is never dereferenced on these paths


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return binding.lib()


def dims(**kw):
    base = dict(n_q=16, offset=100, n_heads=64, d_latent=512, d_rope=64, n_idx_heads=4, d_idx=128,
                top_k=2048, sm_scale=1.0 / 24.0, act_dtype=0, idx_dtype=0)
    base.update(kw)
    return binding.Dims(*[base[f] for f, _ in binding.Dims._fields_])


def test_exports_every_declared_symbol(L):
    decl = declared_functions()
    assert decl == sorted(binding.EXPORTED)
    for name in decl:
        assert hasattr(L, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True,
                        check=True).stdout
    exported = sorted(set(re.findall(r" T (dsa_[a-z0-9_]+)$", nm, flags=re.M)))
    assert exported == decl
    # nothing but the C ABI is exported
    assert not re.search(r" T _Z", nm)


def test_status_strings_and_version(L):
    for s in (OK, NULL, SHAPE, DTYPE, UNSUP, WS, DEV, ALIGN):
        assert binding.status_string(s) and binding.status_string(s) != "unknown status"
    assert binding.status_string(12345) == "unknown status"
    assert binding.version() >= 100


def test_dims_struct_layout_matches_header():
    # 8 int32 + float + 2 int32, no padding
    assert ctypes.sizeof(binding.Dims) == 11 * 4


def _idx(L, d, ld=None, p=(FAKE, FAKE, FAKE, FAKE)):
    ld = d.offset + d.n_q if ld is None else ld
    return L.dsa_indexer_scores(ctypes.byref(d), p[0], p[1], p[2], p[3], ld, None)


def test_indexer_rejects_bad_arguments(L):
    assert L.dsa_indexer_scores(None, FAKE, FAKE, FAKE, FAKE, 200, None) == NULL
    assert _idx(L, dims(n_q=-1)) == SHAPE
    assert _idx(L, dims(offset=-5)) == SHAPE
    assert _idx(L, dims(offset=2**31 - 10, n_q=20), ld=2**31 + 10) == SHAPE
    assert _idx(L, dims(n_idx_heads=0)) == SHAPE
    assert _idx(L, dims(d_idx=-1)) == SHAPE
    assert _idx(L, dims(idx_dtype=7)) == DTYPE
    assert _idx(L, dims(), ld=115) == SHAPE  # ld < offset + n_q
    assert _idx(L, dims(), p=(FAKE, None, FAKE, FAKE)) == NULL
    assert _idx(L, dims(), p=(FAKE, FAKE, FAKE, FAKE + 4)) == ALIGN
    # plain-kernel limit: n_idx_heads * d_idx above the LDS-resident row
    assert _idx(L, dims(n_idx_heads=3, d_idx=4096)) == UNSUP
    # an empty chunk is a no-op, pointers may be NULL
    assert _idx(L, dims(n_q=0), ld=100, p=(None, None, None, None)) == OK


def test_topk_rejects_bad_arguments(L):
    d = dims()
    ld = d.offset + d.n_q
    assert L.dsa_topk_workspace_bytes(ctypes.byref(d)) == 0
    assert L.dsa_topk_select(None, FAKE, ld, FAKE, None, 0, None) == NULL
    assert L.dsa_topk_select(ctypes.byref(dims(top_k=0)), FAKE, ld, FAKE, None, 0, None) == SHAPE
    assert L.dsa_topk_select(ctypes.byref(dims(top_k=(1 << 20) + 1)), FAKE, ld, FAKE, None, 0, None) == SHAPE
    assert L.dsa_topk_select(ctypes.byref(d), FAKE, ld - 1, FAKE, None, 0, None) == SHAPE
    assert L.dsa_topk_select(ctypes.byref(d), None, ld, FAKE, None, 0, None) == NULL
    assert L.dsa_topk_select(ctypes.byref(d), FAKE, ld, FAKE + 8, None, 0, None) == ALIGN
    assert L.dsa_topk_select(ctypes.byref(dims(n_q=0)), None, 100, None, None, 0, None) == OK


def test_attention_rejects_bad_arguments(L):
    def call(d, q=FAKE, kv=FAKE, idx=FAKE, out=FAKE, lse=None):
        return L.dsa_sparse_mla_fwd(ctypes.byref(d), q, kv, idx, out, lse, None)

    assert L.dsa_sparse_mla_fwd(None, FAKE, FAKE, FAKE, FAKE, None, None) == NULL
    assert call(dims(n_heads=0)) == SHAPE
    assert call(dims(d_latent=0)) == SHAPE
    assert call(dims(d_rope=-1)) == SHAPE
    assert call(dims(top_k=0)) == SHAPE
    assert call(dims(sm_scale=float("nan"))) == SHAPE
    assert call(dims(sm_scale=float("inf"))) == SHAPE
    assert call(dims(act_dtype=2)) == DTYPE
    assert call(dims(), kv=None) == NULL
    assert call(dims(), out=None) == NULL
    assert call(dims(), lse=FAKE + 4) == ALIGN
    # plain-kernel limits: wide rows or very large k
    assert call(dims(n_heads=8, d_latent=4000, d_rope=64)) == UNSUP
    assert call(dims(n_heads=8, top_k=5000)) == UNSUP
    assert call(dims(n_q=0), q=None, kv=None, idx=None, out=None) == OK


def test_prefill_chunk_rejects_bad_arguments(L):
    def call(d, ld=None, **kw):
        a = dict(q=FAKE, kv_chunk=FAKE, q_idx=FAKE, w=FAKE, kx_chunk=FAKE, kv_cache=FAKE * 2,
                 kx_cache=FAKE * 4, scores=FAKE, idx=FAKE, out=FAKE, lse=None)
        a.update(kw)
        ld = d.offset + d.n_q if ld is None else ld
        return L.dsa_prefill_chunk(ctypes.byref(d), a["q"], a["kv_chunk"], a["q_idx"], a["w"], a["kx_chunk"],
                                   a["kv_cache"], a["kx_cache"], a["scores"], ld, a["idx"], a["out"], a["lse"],
                                   None, 0, None)

    assert L.dsa_prefill_chunk(None, *([FAKE] * 8), 200, FAKE, FAKE, None, None, 0, None) == NULL
    # each step's checks run before anything is enqueued
    assert call(dims(idx_dtype=9)) == DTYPE
    assert call(dims(), ld=100) == SHAPE
    assert call(dims(top_k=0)) == SHAPE
    assert call(dims(sm_scale=float("nan"))) == SHAPE
    assert call(dims(), kv_chunk=None) == NULL
    assert call(dims(), kx_chunk=FAKE + 4) == ALIGN
    # no score matrix: steps 1-2 run fused and need the fused call's workspace
    assert call(dims(), scores=None) == WS
    # a chunk that partially overlaps its destination rows
    d = dims()
    dst = FAKE * 2 + d.offset * 1152
    assert call(d, kv_chunk=dst + 1152) == SHAPE
    assert call(dims(n_q=0), q=None, kv_chunk=None, q_idx=None, w=None, kx_chunk=None, kv_cache=None,
                kx_cache=None, scores=None, idx=None, out=None) == OK


def test_decode_workspace_and_bad_arguments(L):
    d = dims(n_q=4, offset=40000)
    ws = L.dsa_sparse_mla_decode_workspace_bytes(ctypes.byref(d))
    # 4 queries x 16 splits of 128 slots x 64 heads x (512 + 1) fp32
    assert ws == 16 * 4 * 64 * 513 * 4
    assert L.dsa_sparse_mla_decode_workspace_bytes(ctypes.byref(dims(n_q=8192))) == 0  # enough queries: no split
    assert L.dsa_sparse_mla_decode_workspace_bytes(ctypes.byref(dims(n_q=4, act_dtype=1))) == 0  # plain kernel
    assert L.dsa_sparse_mla_decode_workspace_bytes(ctypes.byref(dims(n_q=-1))) == 0

    def call(dd, ws_ptr=FAKE, ws_bytes=ws, **kw):
        a = dict(q=FAKE, kv=FAKE, idx=FAKE, out=FAKE, lse=None)
        a.update(kw)
        return L.dsa_sparse_mla_decode(ctypes.byref(dd), a["q"], a["kv"], a["idx"], a["out"], a["lse"], ws_ptr,
                                       ws_bytes, None)

    assert call(d, ws_ptr=None) == WS
    assert call(d, ws_bytes=ws - 1) == WS
    assert call(d, ws_ptr=FAKE + 4) == ALIGN
    assert call(dims(n_q=4, top_k=0)) == SHAPE
    assert call(d, out=None) == NULL
    assert call(dims(n_q=0), q=None, kv=None, idx=None, out=None, ws_ptr=None, ws_bytes=0) == OK


def test_decode_noalloc_rejects_before_the_device(L):
    def call(dd, **kw):
        a = dict(q=FAKE, kv=FAKE, idx=FAKE, out=FAKE, lse=None)
        a.update(kw)
        return L.dsa_sparse_mla_decode_noalloc(ctypes.byref(dd), a["q"], a["kv"], a["idx"], a["out"], a["lse"], None)

    # 16 queries x 16 splits of 128 slots: 256 partials of 64 x 513 fp32, past the 32 MiB scratch
    assert L.dsa_sparse_mla_decode_workspace_bytes(ctypes.byref(dims(n_q=16, offset=40000))) > 32 << 20
    assert call(dims(n_q=16, offset=40000)) == WS
    assert call(dims(n_q=4), out=None) == NULL
    assert call(dims(n_q=4), lse=FAKE + 4) == ALIGN
    assert call(dims(n_q=4, top_k=0)) == SHAPE
    assert call(dims(n_q=0), q=None, kv=None, idx=None, out=None) == OK


def test_measurement_library_exports():
    # the benchmark's micro-kernel library (achievable MFMA and copy rates):
    # built beside the product library, its two entry points exported, and its
    # argument checks answer before any launch
    from dsa_top_sparse_amd import build as hip_build
    if not os.path.exists(hip_build.PEAKS_LIB):
        pytest.skip("measurement library not built")
    P = ctypes.CDLL(hip_build.PEAKS_LIB)
    P.dsa_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    P.dsa_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    assert P.dsa_peak_mfma(0, 1, FAKE, None) != 0
    assert P.dsa_peak_mfma(1, 1, None, None) != 0
    assert P.dsa_peak_copy(FAKE, FAKE, 17, None) != 0
    assert P.dsa_peak_copy(None, FAKE, 16, None) != 0


def test_lds_poison_build_exports_the_same_entry_points():
    # the debug build whose kernels poison their LDS first (compared with the
    # product build in tests/test_gpu_lds_poison.py): built beside it by
    # build(), the same C ABI and nothing else
    from dsa_top_sparse_amd import build as hip_build
    assert os.path.exists(hip_build.LDS_POISON_LIB), "run __graft_entry__.build() first"
    nm = subprocess.run(["nm", "-D", "--defined-only", hip_build.LDS_POISON_LIB], capture_output=True, text=True,
                        check=True).stdout
    assert sorted(set(re.findall(r" T (dsa_[a-z0-9_]+)$", nm, flags=re.M))) == declared_functions()
    assert not re.search(r" T _Z", nm)
    with binding.use_library(hip_build.LDS_POISON_LIB) as P:
        assert P._name == hip_build.LDS_POISON_LIB and binding.lib() is P
        assert binding.status_string(SHAPE) != "unknown status"
        d = dims(n_q=4, top_k=0)  # argument checks answer before any launch
        assert P.dsa_sparse_mla_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, None) == SHAPE
    assert binding.lib()._name == binding.LIB_PATH
