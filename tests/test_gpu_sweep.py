"""Seeded sweep of chunk shapes through the whole path (``-m gpu``).

Shapes come from a fixed seed: query counts from 1 to 640 (single queries,
partial and whole 64-query blocks), offsets from 0 to 60,000 (rows shorter
and longer than top_k, up to the filtered select's 65,536 keys), top_k from 4
to 4,096 (the fused path's largest), and score row strides with and
without padding (an odd stride takes the unaligned select and the indexer's
per-score stores). Every row is compared with the oracle: scores and indices
(two calls and the fused indexer + select) bit-exact, attention and lse
within the parity tolerance.
"""
import numpy as np
import pytest

import oracle
from dsa_top_sparse_amd import binding, synth
from parity_checks import check_attention, say

pytestmark = pytest.mark.gpu


def _shapes(count=24, seed=2024):
    rng = np.random.default_rng(seed)
    shapes = []
    for c in range(count):
        offset = int(rng.integers(0, 60000))
        n_q = int(rng.choice([1, 3, 63, 64, 65, 130, 257, 400, 640]))
        n_q = max(1, min(n_q, 8_000_000 // (offset + n_q)))  # keeps the oracle at seconds
        top_k = int(rng.choice([4, 64, 100, 256, 512, 1000, 2048, 2052, 4096]))
        pad = int(rng.choice([0, 0, 1, 4]))
        shapes.append((n_q, offset, top_k, pad, 900 + c))
    return shapes


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    binding.lib()  # fails loudly when the HIP library is missing
    oracle.build(force=False)
    return torch


@pytest.mark.parametrize("n_q,offset,top_k,pad,seed", _shapes())
def test_sweep_shape(torch_cuda, n_q, offset, top_k, pad, seed):
    torch = torch_cuda
    cfg = synth.CONFIGS["C2"].replace(name=f"sweep_{seed}", n_q=n_q, offset=offset, top_k=top_k, seed=seed)
    ld = cfg.t_ctx + pad
    say(f"sweep: {cfg} ld={ld}")
    inputs = synth.generate(cfg)
    dev = binding.to_device(inputs)
    outs = binding.alloc_outputs(cfg, ld=ld)
    binding.run_chunk(cfg, dev, outs)
    dims = binding.make_dims(cfg)
    ws = torch.empty(max(1, binding.indexer_topk_workspace_bytes(dims)), dtype=torch.uint8, device="cuda")
    fidx = torch.full_like(outs["idx"], 12345)
    binding.indexer_topk(dims, dev["qidx"], dev["w"], dev["kidx"], fidx, ws)
    torch.cuda.synchronize()
    ref = oracle.full_path(cfg, inputs)
    scores = outs["scores"].cpu().numpy()
    assert np.array_equal(scores[:, :cfg.t_ctx].view(np.uint32), ref["scores"].view(np.uint32)), "scores"
    assert np.all(scores[:, cfg.t_ctx:] == -np.inf), "padding columns"
    assert np.array_equal(outs["idx"].cpu().numpy(), ref["idx"]), "indices"
    assert np.array_equal(fidx.cpu().numpy(), ref["idx"]), "fused indices"
    check_attention(outs["out"].cpu().numpy(), outs["lse"].cpu().numpy(), ref["out"], ref["lse"], cfg.name)


def _other_dims(count=16, seed=4048):
    rng = np.random.default_rng(seed)
    shapes = []
    for c in range(count):
        act = str(rng.choice(["bf16", "bf16", "f32"]))
        shapes.append(dict(
            n_q=int(rng.choice([1, 33, 97])), offset=int(rng.integers(0, 4000)),
            n_heads=int(rng.choice([1, 4, 16, 64, 128])), d_latent=int(rng.choice([32, 64, 128, 512])),
            d_rope=int(rng.choice([0, 16, 64])), n_idx_heads=int(rng.choice([1, 2, 4, 8])),
            d_idx=int(rng.choice([16, 32, 48, 64, 128, 256])), top_k=int(rng.choice([1, 7, 64, 200, 1024])),
            act_dtype=act, idx_dtype=str(rng.choice(["bf16", "f32"])) if act == "f32" else "bf16",
            seed=1900 + c))
    return shapes


@pytest.mark.parametrize("shape", _other_dims(), ids=lambda d: "h{n_heads}_dl{d_latent}_dr{d_rope}_ih{n_idx_heads}_"
                         "di{d_idx}_k{top_k}_{act_dtype}_{idx_dtype}_q{n_q}_o{offset}".format(**d))
def test_sweep_other_dims(torch_cuda, shape):
    # Head counts, widths, top_k and dtypes away from the workloads' 64 x (512
    # + 64) attention and 4 x 128 indexer: the plain kernels, the MFMA indexer
    # for other widths, and the fused call's two-step fallback, every row
    # against the oracle.
    torch = torch_cuda
    cfg = synth.CONFIGS["C2"].replace(name="sweep_dims", **shape)
    say(f"sweep dims: {cfg}")
    inputs = synth.generate(cfg)
    dev = binding.to_device(inputs)
    outs = binding.alloc_outputs(cfg)
    binding.run_chunk(cfg, dev, outs)
    dims = binding.make_dims(cfg)
    ws = torch.empty(max(1, binding.indexer_topk_workspace_bytes(dims)), dtype=torch.uint8, device="cuda")
    fidx = torch.full_like(outs["idx"], 12345)
    binding.indexer_topk(dims, dev["qidx"], dev["w"], dev["kidx"], fidx, ws)
    torch.cuda.synchronize()
    ref = oracle.full_path(cfg, inputs)
    assert np.array_equal(outs["scores"].cpu().numpy().view(np.uint32), ref["scores"].view(np.uint32)), "scores"
    assert np.array_equal(outs["idx"].cpu().numpy(), ref["idx"]), "indices"
    assert np.array_equal(fidx.cpu().numpy(), ref["idx"]), "fused indices"
    check_attention(outs["out"].cpu().numpy(), outs["lse"].cpu().numpy(), ref["out"], ref["lse"], cfg.name)
