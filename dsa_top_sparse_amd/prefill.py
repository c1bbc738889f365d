"""Chunked prefill driver over ``dsa_prefill_chunk``.

A prompt of T tokens starts from empty caches and is processed in successive
chunks (the feedman.me page profiles 8,192 tokens in 2,048-token chunks, and
a 17.5k-token prompt). Each call appends the chunk's latent and indexer-key
rows to the caches and runs the indexer, the top-k select and the sparse
attention for the chunk's queries. This module only slices tensors and loops
over chunks; the work happens in the library.
"""
from __future__ import annotations

from typing import Dict, Optional

from . import binding


def alloc_prompt_outputs(cfg, device: str = "cuda") -> Dict:
    """Whole-prompt outputs plus empty caches for a prompt config (offset 0, n_q = T)."""
    import torch
    T = cfg.n_q
    act = torch.bfloat16 if cfg.act_dtype == "bf16" else torch.float32
    idt = torch.bfloat16 if cfg.idx_dtype == "bf16" else torch.float32
    return {
        "kv_cache": torch.empty((T, cfg.d_latent + cfg.d_rope), dtype=act, device=device),
        "kidx_cache": torch.empty((T, cfg.d_idx), dtype=idt, device=device),
        "idx": torch.empty((T, cfg.top_k), dtype=torch.int32, device=device),
        "out": torch.empty((T, cfg.n_heads, cfg.d_latent), dtype=torch.float32, device=device),
        "lse": torch.empty((T, cfg.n_heads), dtype=torch.float32, device=device),
    }


# Context (keys per query row) from which the fused indexer + select is the
# faster way to run steps 1-2 on MI355X: as fast as the two calls on the last
# 2k chunk of a 17.5k prompt, about 10 % faster on an 8k chunk at a 49k
# context, slower on an 8k chunk at 16k.
FUSED_FROM_CONTEXT = 32768


def run_prefill(cfg, dev: Dict, chunk: int, outs: Dict, scores=None, stream=None,
                fused: Optional[bool] = None) -> None:
    """Runs the prompt ``dev`` (q, kv, qidx, w, kidx for all T tokens) in chunks of ``chunk``.

    ``outs`` comes from :func:`alloc_prompt_outputs`; ``scores`` is an optional
    [chunk][T] fp32 buffer reused by every chunk (allocated when needed).
    ``fused``: run steps 1-2 of every chunk fused (True), as two calls
    (False), or fused for the chunks whose context reaches
    FUSED_FROM_CONTEXT (None). The indices and outputs are the same either way.
    """
    import torch
    T = cfg.n_q
    if chunk <= 0:
        raise ValueError("chunk must be positive")
    plan = []
    for c0 in range(0, T, chunk):
        n = min(chunk, T - c0)
        use_fused = fused if fused is not None else c0 + n >= FUSED_FROM_CONTEXT
        plan.append((c0, n, use_fused))
    if any(not f for _, _, f in plan):
        if scores is None:
            scores = torch.empty((min(chunk, T), T), dtype=torch.float32, device=dev["q"].device)
        if scores.shape[1] < T or scores.shape[0] < min(chunk, T):
            raise ValueError("scores buffer too small for this prompt")
    ws_bytes = max([binding.indexer_topk_workspace_bytes(binding.make_dims(cfg, n_q=n, offset=c0))
                    for c0, n, f in plan if f] or [0])
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev["q"].device) if ws_bytes else None
    for c0, n, use_fused in plan:
        r = slice(c0, c0 + n)
        dims = binding.make_dims(cfg, n_q=n, offset=c0)
        binding.prefill_chunk(dims, dev["q"][r], dev["kv"][r], dev["qidx"][r], dev["w"][r], dev["kidx"][r],
                              outs["kv_cache"], outs["kidx_cache"], None if use_fused else scores[:n],
                              0 if use_fused else scores.shape[1], outs["idx"][r], outs["out"][r], outs["lse"][r],
                              ws if use_fused else None, stream)
