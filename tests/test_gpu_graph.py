"""The hot path under HIP graph capture (``-m gpu``).

The calls allocate nothing and synchronise only on a device's first use (the
matrix-core self-test, which is skipped while a stream is being captured), so
a serving loop can capture a step once and replay it. Each test captures
calls into a graph after an eager warm-up, then replays the graph several
times -- with the outputs overwritten and the program's own eager work and
synchronisations between the replays -- and compares every replay with the
eager result bit for bit.
"""
import numpy as np
import pytest

import oracle
from dsa_top_sparse_amd import binding, synth
from parity_checks import say

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    binding.lib()  # fails loudly when the HIP library is missing
    oracle.build(force=False)
    return torch


def _capture(torch, fn):
    """torch's recipe: warm up on a side stream, then capture fn into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replay_and_compare(torch, g, outs, ref, eager_between):
    for rep in range(REPLAYS):
        for t in outs.values():
            if t.dtype == torch.int32:
                t.fill_(-7)
            else:
                t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        eager_between()
        torch.cuda.synchronize()
        for k, r in ref.items():
            got = outs[k].cpu().numpy()
            assert np.array_equal(r.view(np.uint8), got.view(np.uint8)), f"replay {rep}: {k} differs"


def test_three_call_step_from_a_graph(torch_cuda):
    torch = torch_cuda
    cfg = synth.CONFIGS["C2"].replace(name="graph_step", n_q=300, offset=5000, seed=51)
    say(f"graph: {cfg}")
    dev = binding.to_device(synth.generate(cfg))
    eager = binding.alloc_outputs(cfg)
    binding.run_chunk(cfg, dev, eager)
    torch.cuda.synchronize()
    keys = ("scores", "idx", "out", "lse")
    ref = {k: eager[k].cpu().numpy() for k in keys}
    outs = binding.alloc_outputs(cfg)
    g = _capture(torch, lambda: binding.run_chunk(cfg, dev, outs))
    _replay_and_compare(torch, g, {k: outs[k] for k in keys}, ref, lambda: binding.run_chunk(cfg, dev, eager))


def test_fused_indexer_topk_from_a_graph(torch_cuda):
    torch = torch_cuda
    cfg = synth.CONFIGS["C2"].replace(name="graph_fused", n_q=260, offset=9000, seed=52)
    dev = binding.to_device(synth.generate(cfg))
    dims = binding.make_dims(cfg)
    ws = torch.empty(max(1, binding.indexer_topk_workspace_bytes(dims)), dtype=torch.uint8, device="cuda")
    idx_e = torch.empty((cfg.n_q, cfg.top_k), dtype=torch.int32, device="cuda")
    binding.indexer_topk(dims, dev["qidx"], dev["w"], dev["kidx"], idx_e, ws)
    torch.cuda.synchronize()
    ref = {"idx": idx_e.cpu().numpy()}
    idx = torch.empty_like(idx_e)
    ws_g = torch.empty_like(ws)
    g = _capture(torch, lambda: binding.indexer_topk(dims, dev["qidx"], dev["w"], dev["kidx"], idx, ws_g))
    _replay_and_compare(torch, g, {"idx": idx}, ref,
                        lambda: binding.indexer_topk(dims, dev["qidx"], dev["w"], dev["kidx"], idx_e, ws))


def test_allocation_free_decode_from_a_graph(torch_cuda):
    # the caller the allocation-free decode is for: a captured decode step
    torch = torch_cuda
    cfg = synth.CONFIGS["C4"].replace(name="graph_decode", n_q=4, offset=49148, seed=53, dup_frac=0.0)
    dev = binding.to_device(synth.generate(cfg))
    eager = binding.alloc_outputs(cfg)
    binding.run_chunk(cfg, dev, eager)  # indices for the decode queries
    torch.cuda.synchronize()
    dims = binding.make_dims(cfg)
    out_e, lse_e = torch.empty_like(eager["out"]), torch.empty_like(eager["lse"])
    binding.sparse_mla_decode_noalloc(dims, dev["q"], dev["kv"], eager["idx"], out_e, lse_e)
    torch.cuda.synchronize()
    ref = {"out": out_e.cpu().numpy(), "lse": lse_e.cpu().numpy()}
    out, lse = torch.empty_like(out_e), torch.empty_like(lse_e)
    g = _capture(torch, lambda: binding.sparse_mla_decode_noalloc(dims, dev["q"], dev["kv"], eager["idx"], out, lse))
    _replay_and_compare(torch, g, {"out": out, "lse": lse}, ref,
                        lambda: binding.sparse_mla_decode_noalloc(dims, dev["q"], dev["kv"], eager["idx"], out_e, lse_e))
