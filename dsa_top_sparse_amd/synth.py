"""Seeded synthetic inputs for the DSA prefill hot path.

This module is shared by the GPU path's tests/bench and by the CPU oracle's
tests. It holds none of the method's arithmetic: it only draws random numbers,
rounds them to the storage dtype and lays them out. Nothing here scores,
selects or attends.

Workload shapes follow the feedman.me page ("GLM-5.3-Flash prefill on M5
Ultra ..."): a prompt processed in 2,048- or 8,192-token chunks (its
per-component profile table, "8,192 tokens in 2,048-token chunks", and the
"Bigger prefill chunks" paragraph) against a cache of earlier tokens with a
latent KV row of 512 values per token ("Why the hand-off is cheap"), and a
top-2,048 selection per query (the paragraph on the work that is not a
matmul). The 17.5k-token prompt of the same page sets the 17,536-token context
of one workload.

Distributions (the pages give none; fixed here so that both sides agree):
  * q and the latent cache kv: fp32 N(0, 1) draws, rounded to bf16
    round-to-nearest-even (the tiny config keeps them in fp32);
  * indexer queries/keys: uniform integers in [-3, 3] (exact in bf16 and fp32),
    so every indexer score is an exact small integer;
  * indexer head weights: uniform in {1.0, 2.0} (fp32);
  * optional duplication: a fraction of cache rows get a copy of the indexer
    key of another (non-duplicated) row, which creates many exactly tied
    scores.
Draw order per config: q, kv, qidx, kidx, w, then the duplication choices.
Generator: NumPy PCG64 seeded with the config's seed.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict

import numpy as np

BF16 = "bf16"
F32 = "f32"


@dataclasses.dataclass(frozen=True)
class DsaConfig:
    """Shape of one prefill chunk call.

    n_q      : chunk length (queries in this call)
    offset   : absolute position of query 0; the cache holds offset + n_q rows
    n_heads  : attention query heads sharing one latent KV row per token
    d_latent : latent (value) width; values are the first d_latent dims of a row
    d_rope   : extra key-only dims appended to each latent row
    n_idx_heads, d_idx : indexer heads and their width (one shared key row per token)
    top_k    : keys kept per query
    """

    name: str
    n_q: int
    offset: int
    n_heads: int
    d_latent: int
    d_rope: int
    n_idx_heads: int
    d_idx: int
    top_k: int
    act_dtype: str = BF16
    idx_dtype: str = BF16
    dup_frac: float = 0.0
    seed: int = 0
    idx_lo: int = -3
    idx_hi: int = 3

    @property
    def t_ctx(self) -> int:
        return self.offset + self.n_q

    @property
    def d_qk(self) -> int:
        return self.d_latent + self.d_rope

    @property
    def sm_scale(self) -> float:
        """Softmax scale 1/sqrt(d_latent + d_rope), rounded to fp32."""
        return float(np.float32(1.0 / math.sqrt(self.d_qk)))

    def replace(self, **kw) -> "DsaConfig":
        return dataclasses.replace(self, **kw)


# The five workloads: a tiny CPU-scale chunk, a 2k chunk at offset 0 (every
# query has <= 2,048 causal keys, so top-k keeps all of them), the last 2k
# chunk of a ~17.5k prompt, an 8k chunk on an 8k cache, and an 8k chunk on a
# ~48k cache with 25 % duplicated indexer-key rows.
CONFIGS: Dict[str, DsaConfig] = {
    "C0": DsaConfig("C0_tiny_256", 256, 0, 4, 64, 16, 2, 32, 64, F32, F32, 0.0, 0),
    "C1": DsaConfig("C1_chunk2k_off0", 2048, 0, 64, 512, 64, 4, 128, 2048, seed=1),
    "C2": DsaConfig("C2_chunk2k_off15488", 2048, 15488, 64, 512, 64, 4, 128, 2048, seed=2),
    "C3": DsaConfig("C3_chunk8k_off8192", 8192, 8192, 64, 512, 64, 4, 128, 2048, seed=3),
    "C4": DsaConfig("C4_chunk8k_off40960_dup25", 8192, 40960, 64, 512, 64, 4, 128, 2048,
                    dup_frac=0.25, seed=4),
}


# Whole prompts from empty caches (offset 0, n_q = prompt length), for the
# chunked-prefill driver: the pages' 8,192-token prefill and their
# ~17.5k-token prompt, with the shapes and distributions of C1.
PROMPTS: Dict[str, DsaConfig] = {
    "P8K": DsaConfig("P8K_prompt8192", 8192, 0, 64, 512, 64, 4, 128, 2048, seed=5),
    "P17K": DsaConfig("P17K_prompt17536", 17536, 0, 64, 512, 64, 4, 128, 2048, seed=6),
}

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == BF16:
        return f32_to_bf16_bits(x32)
    if dtype == F32:
        return np.ascontiguousarray(x32, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def generate(cfg: DsaConfig) -> Dict[str, np.ndarray]:
    """Draw the inputs of one chunk call.

    Returns host arrays (bf16 as uint16 bit patterns, fp32 as float32):
      q    [n_q][n_heads][d_qk]      act dtype
      kv   [t_ctx][d_qk]             act dtype (first d_latent dims = values)
      qidx [n_q][n_idx_heads][d_idx] idx dtype (integers in [idx_lo, idx_hi])
      kidx [t_ctx][d_idx]            idx dtype
      w    [n_q][n_idx_heads]        fp32 in {1, 2}
      dup_dst, dup_src               int64 row indices of the duplication
    """
    rng = np.random.Generator(np.random.PCG64(cfg.seed))
    q = rng.standard_normal((cfg.n_q, cfg.n_heads, cfg.d_qk), dtype=np.float32)
    q = _store(q, cfg.act_dtype)
    kv = rng.standard_normal((cfg.t_ctx, cfg.d_qk), dtype=np.float32)
    kv = _store(kv, cfg.act_dtype)
    qidx = rng.integers(cfg.idx_lo, cfg.idx_hi + 1, size=(cfg.n_q, cfg.n_idx_heads, cfg.d_idx))
    qidx = _store(qidx.astype(np.float32), cfg.idx_dtype)
    kidx = rng.integers(cfg.idx_lo, cfg.idx_hi + 1, size=(cfg.t_ctx, cfg.d_idx))
    kidx = _store(kidx.astype(np.float32), cfg.idx_dtype)
    w = rng.integers(1, 3, size=(cfg.n_q, cfg.n_idx_heads)).astype(np.float32)
    dup_dst = np.zeros(0, dtype=np.int64)
    dup_src = np.zeros(0, dtype=np.int64)
    n_dup = int(math.floor(cfg.dup_frac * cfg.t_ctx))
    if n_dup > 0:
        dup_dst = np.sort(rng.choice(cfg.t_ctx, size=n_dup, replace=False)).astype(np.int64)
        keep = np.ones(cfg.t_ctx, dtype=bool)
        keep[dup_dst] = False
        sources = np.flatnonzero(keep)
        dup_src = sources[rng.integers(0, sources.size, size=n_dup)].astype(np.int64)
        kidx[dup_dst] = kidx[dup_src]
    return {"q": q, "kv": kv, "qidx": qidx, "kidx": kidx, "w": w,
            "dup_dst": dup_dst, "dup_src": dup_src}


def tiny_config(**kw) -> DsaConfig:
    """A small custom shape for unit tests (defaults mirror the tiny config)."""
    base = CONFIGS["C0"].replace(name="custom")
    return base.replace(**kw)
