"""CPU oracle for the DSA prefill hot path (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package. It wraps ``dsa_oracle.c`` (plain C, fp64, OpenMP over
queries) through ctypes. It shares no code with the HIP library and never
imports it.

The three steps it computes, with the passages they follow, are described at
the top of ``dsa_oracle.c``:
  * ``indexer_scores`` -- ReLU-weighted indexer scores of every causal key,
  * ``topk_select``    -- per-query top-k, lower key index wins ties,
  * ``sparse_mla``     -- fp64 softmax attention over the selected latent rows.

Parity status: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py`` (library-routine and brute-force special cases,
closed forms, invariants). What the pages leave open is fixed by the readings
listed in the design notes; beyond those readings the semantics of the pages'
own model are unpinned, because the pages print no DSA formula or values.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libdsa_oracle.so")
_lib = None

BF16 = 0
F32 = 1


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O2, OpenMP). Returns the library path."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        i32, i64, vp, dbl = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
        lib.oracle_indexer_scores.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, i64, vp, i32]
        lib.oracle_topk_select.argtypes = [i32, i32, i32, vp, i64, vp, vp, i32]
        lib.oracle_sparse_mla.argtypes = [i32, i32, i32, i32, i32, dbl, i32, vp, vp, vp, i32, vp,
                                          vp, vp, i32]
        for f in (lib.oracle_indexer_scores, lib.oracle_topk_select, lib.oracle_sparse_mla):
            f.restype = i32
        lib.oracle_num_threads.restype = i32
        lib.oracle_set_threads.argtypes = [i32]
        _lib = lib
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_threads(n: int) -> None:
    """Threads of the oracle's parallel loops from now on (results do not depend on it)."""
    _load().oracle_set_threads(int(n))


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    raise TypeError(f"oracle inputs are bf16 bits (uint16) or float32, got {a.dtype}")


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _rows(rows: Optional[Sequence[int]], n_q: int):
    if rows is None:
        return None, n_q
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
    if r.size and (r.min() < 0 or r.max() >= n_q):
        raise ValueError("row index out of range")
    return r, int(r.size)


def indexer_scores(n_q: int, offset: int, qidx: np.ndarray, w: np.ndarray, kidx: np.ndarray,
                   ld: Optional[int] = None, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Scores [len(rows)][ld] fp32 (rows default to all queries)."""
    qidx = np.ascontiguousarray(qidx)
    kidx = np.ascontiguousarray(kidx)
    w = np.ascontiguousarray(w, dtype=np.float32)
    n_idx_heads, d_idx = qidx.shape[1], qidx.shape[2]
    assert qidx.shape[0] == n_q and kidx.shape[0] >= offset + n_q and kidx.shape[1] == d_idx
    assert qidx.dtype == kidx.dtype and w.shape == (n_q, n_idx_heads)
    ld = offset + n_q if ld is None else int(ld)
    r, n_rows = _rows(rows, n_q)
    out = np.empty((n_rows, ld), dtype=np.float32)
    st = _load().oracle_indexer_scores(n_q, offset, n_idx_heads, d_idx, _dtype_code(qidx),
                                       _ptr(qidx), _ptr(w), _ptr(kidx), _ptr(out), ld,
                                       _ptr(r), n_rows)
    if st != 0:
        raise RuntimeError(f"oracle_indexer_scores failed ({st})")
    return out


def topk_select(n_q: int, offset: int, top_k: int, scores: np.ndarray,
                rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Indices [len(rows)][top_k] int32; scores row r belongs to query rows[r]."""
    scores = np.ascontiguousarray(scores, dtype=np.float32)
    r, n_rows = _rows(rows, n_q)
    assert scores.shape[0] == n_rows
    out = np.empty((n_rows, top_k), dtype=np.int32)
    st = _load().oracle_topk_select(n_q, offset, top_k, _ptr(scores), scores.shape[1], _ptr(out),
                                    _ptr(r), n_rows)
    if st != 0:
        raise RuntimeError(f"oracle_topk_select failed ({st})")
    return out


def sparse_mla(n_q: int, offset: int, sm_scale: float, d_v: int, q: np.ndarray, kv: np.ndarray,
               idx: np.ndarray, rows: Optional[Sequence[int]] = None):
    """(out [len(rows)][H][d_v] float64, lse [len(rows)][H] float64)."""
    q = np.ascontiguousarray(q)
    kv = np.ascontiguousarray(kv)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    n_heads, d_qk = q.shape[1], q.shape[2]
    assert q.shape[0] == n_q and kv.shape[1] == d_qk and q.dtype == kv.dtype
    r, n_rows = _rows(rows, n_q)
    assert idx.shape[0] == n_rows
    top_k = idx.shape[1]
    out = np.empty((n_rows, n_heads, d_v), dtype=np.float64)
    lse = np.empty((n_rows, n_heads), dtype=np.float64)
    st = _load().oracle_sparse_mla(n_q, offset, n_heads, d_qk, d_v, float(sm_scale),
                                   _dtype_code(q), _ptr(q), _ptr(kv), _ptr(idx), top_k,
                                   _ptr(out), _ptr(lse), _ptr(r), n_rows)
    if st != 0:
        raise RuntimeError(f"oracle_sparse_mla failed ({st})")
    return out, lse


def full_path(cfg, inputs, rows: Optional[Sequence[int]] = None):
    """All three steps for the listed query rows of one chunk call.

    ``cfg`` needs n_q, offset, top_k, sm_scale and d_latent; ``inputs`` holds
    q, kv, qidx, kidx, w as drawn by the seeded generator.
    """
    s = indexer_scores(cfg.n_q, cfg.offset, inputs["qidx"], inputs["w"], inputs["kidx"],
                       rows=rows)
    idx = topk_select(cfg.n_q, cfg.offset, cfg.top_k, s, rows=rows)
    out, lse = sparse_mla(cfg.n_q, cfg.offset, cfg.sm_scale, cfg.d_latent, inputs["q"],
                          inputs["kv"], idx, rows=rows)
    return {"scores": s, "idx": idx, "out": out, "lse": lse}
