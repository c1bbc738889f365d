"""ctypes binding of ``libdsa_amd.so`` (the C ABI in ``include/dsa.h``).

Argument marshalling only: every step of the path runs in the HIP kernels of
the library. PyTorch provides device memory and the stream handle. The module
raises if the library has not been built -- there is no fallback path.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Dict, Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libdsa_amd.so")

DSA_BF16 = 0
DSA_F32 = 1

# Every symbol include/dsa.h declares.
EXPORTED = (
    "dsa_indexer_scores",
    "dsa_topk_workspace_bytes",
    "dsa_topk_select",
    "dsa_indexer_topk_workspace_bytes",
    "dsa_indexer_topk",
    "dsa_sparse_mla_fwd",
    "dsa_prefill_chunk",
    "dsa_sparse_mla_decode_workspace_bytes",
    "dsa_sparse_mla_decode",
    "dsa_sparse_mla_decode_noalloc",
    "dsa_self_test",
    "dsa_status_string",
    "dsa_version",
)

STATUS = {0: "DSA_OK", -1: "DSA_ERR_NULL", -2: "DSA_ERR_SHAPE", -3: "DSA_ERR_DTYPE",
          -4: "DSA_ERR_UNSUPPORTED", -5: "DSA_ERR_WORKSPACE", -6: "DSA_ERR_DEVICE",
          -7: "DSA_ERR_ALIGN"}


class Dims(ctypes.Structure):
    """Mirror of ``dsa_dims``."""

    _fields_ = [
        ("n_q", ctypes.c_int32),
        ("offset", ctypes.c_int32),
        ("n_heads", ctypes.c_int32),
        ("d_latent", ctypes.c_int32),
        ("d_rope", ctypes.c_int32),
        ("n_idx_heads", ctypes.c_int32),
        ("d_idx", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("act_dtype", ctypes.c_int32),
        ("idx_dtype", ctypes.c_int32),
    ]


class DsaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} returned {STATUS.get(status, status)}: {status_string(status)}")


_lib = None


def _load(path: str) -> ctypes.CDLL:
    """Loads one build of the HIP library and declares its entry points."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: run __graft_entry__.build() "
                           "(or python -m dsa_top_sparse_amd.build) first")
    L = ctypes.CDLL(path)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    dp = ctypes.POINTER(Dims)
    L.dsa_indexer_scores.argtypes = [dp, vp, vp, vp, vp, i64, vp]
    L.dsa_topk_workspace_bytes.argtypes = [dp]
    L.dsa_topk_workspace_bytes.restype = sz
    L.dsa_topk_select.argtypes = [dp, vp, i64, vp, vp, sz, vp]
    L.dsa_sparse_mla_fwd.argtypes = [dp, vp, vp, vp, vp, vp, vp]
    L.dsa_indexer_topk_workspace_bytes.argtypes = [dp]
    L.dsa_indexer_topk_workspace_bytes.restype = sz
    L.dsa_indexer_topk.argtypes = [dp, vp, vp, vp, vp, vp, sz, vp]
    L.dsa_prefill_chunk.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, vp, vp, sz, vp]
    L.dsa_sparse_mla_decode_workspace_bytes.argtypes = [dp]
    L.dsa_sparse_mla_decode_workspace_bytes.restype = sz
    L.dsa_sparse_mla_decode.argtypes = [dp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.dsa_sparse_mla_decode_noalloc.argtypes = [dp, vp, vp, vp, vp, vp, vp]
    for f in (L.dsa_indexer_scores, L.dsa_topk_select, L.dsa_indexer_topk, L.dsa_sparse_mla_fwd, L.dsa_prefill_chunk,
              L.dsa_sparse_mla_decode, L.dsa_sparse_mla_decode_noalloc):
        f.restype = ctypes.c_int
    L.dsa_self_test.argtypes = []
    L.dsa_self_test.restype = ctypes.c_int
    L.dsa_status_string.argtypes = [ctypes.c_int]
    L.dsa_status_string.restype = ctypes.c_char_p
    L.dsa_version.restype = ctypes.c_int32
    return L


def lib() -> ctypes.CDLL:
    """Loads the HIP library (raises if it is missing: build it first)."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


@contextlib.contextmanager
def use_library(path: str):
    """Inside the block, every call of this module goes to another build of
    the library at `path` (the tests use the LDS-poisoned debug build)."""
    global _lib
    saved = lib()
    _lib = _load(path)
    try:
        yield _lib
    finally:
        _lib = saved


def status_string(status: int) -> str:
    return lib().dsa_status_string(int(status)).decode()


def version() -> int:
    return int(lib().dsa_version())


def self_test() -> None:
    """Runs the matrix-core layout self-test on the current device (raises on failure)."""
    _check("dsa_self_test", lib().dsa_self_test())


def make_dims(cfg, n_q: Optional[int] = None, offset: Optional[int] = None) -> Dims:
    """dsa_dims for a config (anything with the DsaConfig attributes)."""
    code = {"bf16": DSA_BF16, "f32": DSA_F32}
    return Dims(cfg.n_q if n_q is None else n_q, cfg.offset if offset is None else offset,
                cfg.n_heads, cfg.d_latent, cfg.d_rope, cfg.n_idx_heads, cfg.d_idx, cfg.top_k,
                cfg.sm_scale, code[cfg.act_dtype], code[cfg.idx_dtype])


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise DsaError(fn, status)


def _contig(*ts):
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensors passed to the DSA library must be contiguous")


def _fits(t, elems: int, itemsize: int, name: str) -> None:
    """Raises ValueError unless tensor ``t`` holds ``elems`` elements of ``itemsize`` bytes.

    A host-side guard only: a tensor smaller than what the dims describe would
    make a kernel write or read past its allocation.
    """
    if t is None:
        return
    if t.element_size() != itemsize:
        raise ValueError(f"{name}: element size {t.element_size()} B, the dims need {itemsize} B")
    if t.numel() < elems:
        raise ValueError(f"{name}: {t.numel()} elements, the dims need at least {elems}")


def _act_size(dims: Dims) -> int:
    return 2 if dims.act_dtype == DSA_BF16 else 4


def _idx_size(dims: Dims) -> int:
    return 2 if dims.idx_dtype == DSA_BF16 else 4


def _check_indexer_sizes(dims: Dims, q_idx, w_idx, k_idx, scores, ld: int) -> None:
    if dims.n_q <= 0:
        return
    _fits(q_idx, dims.n_q * dims.n_idx_heads * dims.d_idx, _idx_size(dims), "q_idx")
    _fits(w_idx, dims.n_q * dims.n_idx_heads, 4, "w_idx")
    _fits(k_idx, (dims.offset + dims.n_q) * dims.d_idx, _idx_size(dims), "k_idx_cache")
    _fits(scores, dims.n_q * int(ld), 4, "scores")


def _check_topk_sizes(dims: Dims, scores, ld: int, idx) -> None:
    if dims.n_q <= 0:
        return
    _fits(scores, dims.n_q * int(ld), 4, "scores")
    _fits(idx, dims.n_q * dims.top_k, 4, "idx")


def _check_mla_sizes(dims: Dims, q, kv, idx, out, lse) -> None:
    if dims.n_q <= 0:
        return
    d_qk = dims.d_latent + dims.d_rope
    _fits(q, dims.n_q * dims.n_heads * d_qk, _act_size(dims), "q")
    _fits(kv, (dims.offset + dims.n_q) * d_qk, _act_size(dims), "kv_cache")
    _fits(idx, dims.n_q * dims.top_k, 4, "idx")
    _fits(out, dims.n_q * dims.n_heads * dims.d_latent, 4, "out")
    _fits(lse, dims.n_q * dims.n_heads, 4, "lse")


def indexer_scores(dims: Dims, q_idx, w_idx, k_idx, scores, ld: int, stream=None) -> None:
    _contig(q_idx, w_idx, k_idx, scores)
    _check_indexer_sizes(dims, q_idx, w_idx, k_idx, scores, ld)
    _check("dsa_indexer_scores", lib().dsa_indexer_scores(
        ctypes.byref(dims), _ptr(q_idx), _ptr(w_idx), _ptr(k_idx), _ptr(scores), int(ld),
        _stream(stream)))


def topk_workspace_bytes(dims: Dims) -> int:
    return int(lib().dsa_topk_workspace_bytes(ctypes.byref(dims)))


def topk_select(dims: Dims, scores, ld: int, idx, workspace=None, stream=None) -> None:
    _contig(scores, idx)
    _check_topk_sizes(dims, scores, ld, idx)
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("dsa_topk_select", lib().dsa_topk_select(
        ctypes.byref(dims), _ptr(scores), int(ld), _ptr(idx), _ptr(workspace), ws,
        _stream(stream)))


def indexer_topk_workspace_bytes(dims: Dims) -> int:
    return int(lib().dsa_indexer_topk_workspace_bytes(ctypes.byref(dims)))


def indexer_topk(dims: Dims, q_idx, w_idx, k_idx, idx, workspace, stream=None) -> None:
    """Indexer scores and top-k select in one call, without the score matrix."""
    _contig(q_idx, w_idx, k_idx, idx, workspace)
    if dims.n_q > 0:
        _fits(q_idx, dims.n_q * dims.n_idx_heads * dims.d_idx, _idx_size(dims), "q_idx")
        _fits(w_idx, dims.n_q * dims.n_idx_heads, 4, "w_idx")
        _fits(k_idx, (dims.offset + dims.n_q) * dims.d_idx, _idx_size(dims), "k_idx_cache")
        _fits(idx, dims.n_q * dims.top_k, 4, "idx")
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("dsa_indexer_topk", lib().dsa_indexer_topk(
        ctypes.byref(dims), _ptr(q_idx), _ptr(w_idx), _ptr(k_idx), _ptr(idx), _ptr(workspace), ws,
        _stream(stream)))


def sparse_mla_fwd(dims: Dims, q, kv, idx, out, lse=None, stream=None) -> None:
    _contig(q, kv, idx, out, lse)
    _check_mla_sizes(dims, q, kv, idx, out, lse)
    _check("dsa_sparse_mla_fwd", lib().dsa_sparse_mla_fwd(
        ctypes.byref(dims), _ptr(q), _ptr(kv), _ptr(idx), _ptr(out), _ptr(lse),
        _stream(stream)))


def sparse_mla_decode_workspace_bytes(dims: Dims) -> int:
    return int(lib().dsa_sparse_mla_decode_workspace_bytes(ctypes.byref(dims)))


def sparse_mla_decode(dims: Dims, q, kv, idx, out, lse=None, workspace=None, stream=None) -> None:
    _contig(q, kv, idx, out, lse, workspace)
    _check_mla_sizes(dims, q, kv, idx, out, lse)
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("dsa_sparse_mla_decode", lib().dsa_sparse_mla_decode(
        ctypes.byref(dims), _ptr(q), _ptr(kv), _ptr(idx), _ptr(out), _ptr(lse), _ptr(workspace), ws,
        _stream(stream)))


def sparse_mla_decode_noalloc(dims: Dims, q, kv, idx, out, lse=None, stream=None) -> None:
    _contig(q, kv, idx, out, lse)
    _check_mla_sizes(dims, q, kv, idx, out, lse)
    _check("dsa_sparse_mla_decode_noalloc", lib().dsa_sparse_mla_decode_noalloc(
        ctypes.byref(dims), _ptr(q), _ptr(kv), _ptr(idx), _ptr(out), _ptr(lse), _stream(stream)))


def prefill_chunk(dims: Dims, q, kv_chunk, q_idx, w_idx, k_idx_chunk, kv_cache, k_idx_cache, scores, ld: int,
                  idx, out, lse=None, workspace=None, stream=None) -> None:
    """scores=None runs steps 1-2 fused (dsa_indexer_topk); workspace must then
    hold indexer_topk_workspace_bytes(dims) bytes."""
    _contig(q, kv_chunk, q_idx, w_idx, k_idx_chunk, kv_cache, k_idx_cache, scores, idx, out, lse)
    if scores is None:
        ld = 0
        need = indexer_topk_workspace_bytes(dims)
        if dims.n_q > 0 and (workspace is None or workspace.numel() * workspace.element_size() < need):
            raise ValueError(f"dsa_prefill_chunk without scores needs a workspace of {need} bytes")
    else:
        _check_indexer_sizes(dims, q_idx, w_idx, k_idx_cache, scores, ld)
        _check_topk_sizes(dims, scores, ld, idx)
    _check_mla_sizes(dims, q, kv_cache, idx, out, lse)
    if dims.n_q > 0:
        _fits(kv_chunk, dims.n_q * (dims.d_latent + dims.d_rope), _act_size(dims), "kv_chunk")
        _fits(k_idx_chunk, dims.n_q * dims.d_idx, _idx_size(dims), "k_idx_chunk")
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("dsa_prefill_chunk", lib().dsa_prefill_chunk(
        ctypes.byref(dims), _ptr(q), _ptr(kv_chunk), _ptr(q_idx), _ptr(w_idx), _ptr(k_idx_chunk),
        _ptr(kv_cache), _ptr(k_idx_cache), _ptr(scores), int(ld), _ptr(idx), _ptr(out), _ptr(lse),
        _ptr(workspace), ws, _stream(stream)))


# ---------------------------------------------------------------- plumbing


def to_device(inputs: Dict, device="cuda") -> Dict:
    """Host arrays from the seeded generator -> device tensors (bf16 stays bf16 bits)."""
    import numpy as np
    import torch
    out = {}
    for k, v in inputs.items():
        if not isinstance(v, np.ndarray) or k.startswith("dup_"):
            continue
        if v.dtype == np.uint16:
            t = torch.from_numpy(v.view(np.int16)).to(device).view(torch.bfloat16)
        else:
            t = torch.from_numpy(np.ascontiguousarray(v)).to(device)
        out[k] = t
    return out


def alloc_outputs(cfg, device="cuda", ld: Optional[int] = None, with_lse: bool = True) -> Dict:
    import torch
    ld = cfg.t_ctx if ld is None else ld
    o = {
        "scores": torch.empty((cfg.n_q, ld), dtype=torch.float32, device=device),
        "idx": torch.empty((cfg.n_q, cfg.top_k), dtype=torch.int32, device=device),
        "out": torch.empty((cfg.n_q, cfg.n_heads, cfg.d_latent), dtype=torch.float32, device=device),
        "lse": torch.empty((cfg.n_q, cfg.n_heads), dtype=torch.float32, device=device) if with_lse else None,
        "ld": ld,
    }
    ws = topk_workspace_bytes(make_dims(cfg))
    o["workspace"] = torch.empty(ws, dtype=torch.uint8, device=device) if ws else None
    return o


def run_chunk(cfg, dev: Dict, outs: Dict, stream=None) -> None:
    """The whole hot path for one chunk: indexer -> top-k -> sparse attention."""
    dims = make_dims(cfg)
    indexer_scores(dims, dev["qidx"], dev["w"], dev["kidx"], outs["scores"], outs["ld"], stream)
    topk_select(dims, outs["scores"], outs["ld"], outs["idx"], outs["workspace"], stream)
    sparse_mla_fwd(dims, dev["q"], dev["kv"], outs["idx"], outs["out"], outs["lse"], stream)
