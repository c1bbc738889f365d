"""The fused indexer + select (dsa_indexer_topk) on the paths the workloads do
not reach: thresholds from the first 2,048 keys that are too high (fewer than
k candidates) or too low (more than fit), all-equal scores, shapes and context
lengths outside the fused kernels, rows no longer than k. Each case against
the two separate calls on every row (themselves checked against the oracle on
every row of every workload) and, where small enough, against the oracle."""
import numpy as np
import pytest

import oracle
from dsa_top_sparse_amd import binding, synth
from parity_checks import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    binding.lib()
    oracle.build(force=False)
    return torch


def _both(torch, cfg, inputs):
    dev = binding.to_device(inputs)
    outs = binding.alloc_outputs(cfg)
    dims = binding.make_dims(cfg)
    binding.indexer_scores(dims, dev["qidx"], dev["w"], dev["kidx"], outs["scores"], outs["ld"])
    binding.topk_select(dims, outs["scores"], outs["ld"], outs["idx"])
    ws = torch.empty(max(1, binding.indexer_topk_workspace_bytes(dims)), dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)  # whatever the workspace held before must not matter
    fidx = torch.full_like(outs["idx"], 12345)
    binding.indexer_topk(dims, dev["qidx"], dev["w"], dev["kidx"], fidx, ws)
    torch.cuda.synchronize()
    return outs["idx"].cpu().numpy(), fidx.cpu().numpy()


def _check(torch, cfg, inputs, label, with_oracle=True):
    say(f"fused: {label} {cfg}")
    two, fused = _both(torch, cfg, inputs)
    bad = np.flatnonzero(np.any(two != fused, axis=1))
    assert bad.size == 0, f"{label}: fused differs from the two calls on rows {bad[:8].tolist()}"
    if with_oracle:
        s = oracle.indexer_scores(cfg.n_q, cfg.offset, inputs["qidx"], inputs["w"], inputs["kidx"])
        ref = oracle.topk_select(cfg.n_q, cfg.offset, cfg.top_k, s)
        assert np.array_equal(fused, ref), f"{label}: fused differs from the oracle"


def _cfg(**kw):
    base = synth.CONFIGS["C2"].replace(name="fused", n_heads=1, d_latent=64, d_rope=0)
    return base.replace(**kw)


def test_fused_threshold_too_high(torch_cuda):
    # Every query's heads are the same all-ones vector, and the first 2,048
    # indexer keys hold 3 in their first c_j dims (c_j falling from 128 to 68
    # along the keys) while later keys are small: the row's top scores are the
    # first keys, so the sample's threshold keeps only a few hundred keys (fewer
    # than k) and every row is scored again and selected from the full row.
    cfg = _cfg(n_q=40, offset=9000, seed=71)
    inputs = synth.generate(cfg)
    rng = np.random.default_rng(1)
    inputs["qidx"] = synth.f32_to_bf16_bits(np.ones(inputs["qidx"].shape, np.float32))
    kid = rng.integers(-1, 2, size=(cfg.t_ctx, cfg.d_idx)).astype(np.float32)
    c = 128 - (np.arange(2048) * 60) // 2048
    kid[:2048] = 3.0 * (np.arange(cfg.d_idx)[None, :] < c[:, None])
    inputs["kidx"] = synth.f32_to_bf16_bits(kid)
    _check(torch_cuda, cfg, inputs, "threshold too high")


def test_fused_threshold_too_low(torch_cuda):
    # The first 2,048 keys all score 0 (zero indexer keys): the threshold is
    # 0, every causal key is a candidate, more than fit in LDS.
    cfg = _cfg(n_q=40, offset=9000, seed=72)
    inputs = synth.generate(cfg)
    inputs["kidx"][:2048] = 0
    _check(torch_cuda, cfg, inputs, "threshold too low")


@pytest.mark.parametrize("offset", [3000, 9000])
def test_fused_all_equal_scores(torch_cuda, offset):
    # q_idx = 0: every score is +0.0 and the k lowest indices win; 3,000-key
    # rows keep every key as a candidate (within LDS), 9,000-key rows do not.
    cfg = _cfg(n_q=24, offset=offset, seed=73)
    inputs = synth.generate(cfg)
    inputs["qidx"] = np.zeros_like(inputs["qidx"])
    _check(torch_cuda, cfg, inputs, f"all equal, offset {offset}")


def test_fused_short_rows_and_ragged(torch_cuda):
    # offset 0: rows 1 .. 2,100 keys long (no more than k for most: every
    # causal key, -1 padding); 70 queries (a partial 64-query block); top_k 100
    cfg = _cfg(n_q=2100, offset=0, seed=74)
    _check(torch_cuda, cfg, synth.generate(cfg), "offset 0, k 2048", with_oracle=False)
    cfg = _cfg(n_q=70, offset=1003, top_k=100, seed=75)
    _check(torch_cuda, cfg, synth.generate(cfg), "ragged, k 100")


@pytest.mark.parametrize("shape", [("bf16", 4, 64), ("f32", 2, 32), ("bf16", 4, 128, 66000)])
def test_fused_outside_the_fused_kernels(torch_cuda, shape):
    # other indexer shapes and dtypes, and a context past 65,536 keys: the call
    # runs the two steps with the scores in its workspace
    dt, h, d = shape[:3]
    off = shape[3] if len(shape) > 3 else 3000
    cfg = _cfg(n_q=8 if off > 60000 else 50, offset=off, n_idx_heads=h, d_idx=d, idx_dtype=dt, seed=76 + h)
    _check(torch_cuda, cfg, synth.generate(cfg), f"outside {shape}", with_oracle=off < 60000)


def test_prefill_chunk_fused_at_long_context(torch_cuda):
    # One chunk of 512 queries at a 34k-key context (where the prefill driver
    # runs steps 1-2 fused) through dsa_prefill_chunk, once with a score
    # matrix and once with NULL scores: caches, indices, outputs and lse
    # bit-identical; a few rows' indices against the oracle.
    torch = torch_cuda
    cfg = synth.CONFIGS["C3"].replace(name="fused_prefill", n_q=512, offset=33800, seed=11)
    say(f"fused prefill: generate {cfg}")
    inputs = synth.generate(cfg)
    dev = binding.to_device(inputs)
    dims = binding.make_dims(cfg)
    T = cfg.offset + cfg.n_q
    r = slice(cfg.offset, T)
    runs = {}
    for mode in ("scores", "fused"):
        kv = dev["kv"].clone()
        kx = dev["kidx"].clone()
        kv_chunk = dev["kv"][r].clone()
        kx_chunk = dev["kidx"][r].clone()
        kv[r] = 0  # the call appends the chunk's rows
        kx[r] = 0
        idx = torch.full((cfg.n_q, cfg.top_k), 12345, dtype=torch.int32, device="cuda")
        out = torch.empty((cfg.n_q, cfg.n_heads, cfg.d_latent), dtype=torch.float32, device="cuda")
        lse = torch.empty((cfg.n_q, cfg.n_heads), dtype=torch.float32, device="cuda")
        if mode == "scores":
            scores = torch.empty((cfg.n_q, T), dtype=torch.float32, device="cuda")
            binding.prefill_chunk(dims, dev["q"], kv_chunk, dev["qidx"], dev["w"], kx_chunk, kv, kx, scores, T,
                                  idx, out, lse)
        else:
            ws = torch.empty(binding.indexer_topk_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
            binding.prefill_chunk(dims, dev["q"], kv_chunk, dev["qidx"], dev["w"], kx_chunk, kv, kx, None, 0,
                                  idx, out, lse, ws)
        torch.cuda.synchronize()
        runs[mode] = (kv, kx, idx, out, lse)
    for a, b, what in zip(runs["scores"], runs["fused"], ("kv cache", "k_idx cache", "idx", "out", "lse")):
        assert torch.equal(a, b), what
    rows = [0, 255, 511]
    ref = oracle.full_path(cfg, inputs, rows=rows)
    assert np.array_equal(runs["fused"][2][rows].cpu().numpy(), ref["idx"])
