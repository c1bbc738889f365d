"""The LDS-poisoned debug build against the product build (``-m gpu``).

Every kernel of ``libdsa_amd_lds_poison.so`` (the same sources compiled with
``-DDSA_LDS_POISON``) fills its workgroup's LDS with a NaN pattern before its
body runs. Its results must equal the product library's bit for bit -- scores,
indices of both paths, attention and lse, split decode -- which shows that no
kernel reads LDS it has not written on these inputs (a stale value left by an
earlier workgroup would otherwise be replaced by NaN or a huge integer).
"""
import numpy as np
import pytest

import oracle
from dsa_top_sparse_amd import binding, synth
from dsa_top_sparse_amd import build as hip_build
from parity_checks import say

pytestmark = pytest.mark.gpu

CASES = [
    ("C1", {}),                                                    # 2,048 queries from empty caches (hi/lo P)
    ("C2", {"n_q": 520, "seed": 41}),                              # long rows, a partial query block
    ("C2", {"n_q": 77, "offset": 1003, "top_k": 100, "seed": 31}),  # ragged; k % 4 != 0: plain attention
    ("C4", {"n_q": 4, "offset": 49148, "seed": 44, "dup_frac": 0.0}),  # a decode step: split attention
    ("C0", {}),                                                    # fp32: the plain kernels
]


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    binding.lib()  # fails loudly when the HIP library is missing
    oracle.build(force=False)
    return torch


def _run_all(torch, cfg, dev):
    dims = binding.make_dims(cfg)
    outs = binding.alloc_outputs(cfg)
    binding.run_chunk(cfg, dev, outs)
    ws = torch.empty(max(1, binding.indexer_topk_workspace_bytes(dims)), dtype=torch.uint8, device="cuda")
    fidx = torch.full_like(outs["idx"], 12345)
    binding.indexer_topk(dims, dev["qidx"], dev["w"], dev["kidx"], fidx, ws)
    res = {"fused_idx": fidx}
    dws = binding.sparse_mla_decode_workspace_bytes(dims)
    if dws > 0:
        dw = torch.empty(dws, dtype=torch.uint8, device="cuda")
        res["dec_out"] = torch.empty_like(outs["out"])
        res["dec_lse"] = torch.empty_like(outs["lse"])
        binding.sparse_mla_decode(dims, dev["q"], dev["kv"], outs["idx"], res["dec_out"], res["dec_lse"], dw)
    torch.cuda.synchronize()
    res.update({k: outs[k] for k in ("scores", "idx", "out", "lse")})
    return {k: v.cpu().numpy() for k, v in res.items()}


@pytest.mark.parametrize("name,changes", CASES, ids=["C1", "C2_520q", "ragged_k100", "decode4", "C0_f32"])
def test_lds_poison_build_matches_product(torch_cuda, name, changes):
    torch = torch_cuda
    cfg = synth.CONFIGS[name].replace(name=f"poison_{name}", **changes)
    say(f"LDS poison: {cfg}")
    dev = binding.to_device(synth.generate(cfg))
    ref = _run_all(torch, cfg, dev)
    with binding.use_library(hip_build.LDS_POISON_LIB):
        got = _run_all(torch, cfg, dev)
    assert set(got) == set(ref)
    for k in ref:
        assert np.array_equal(ref[k].view(np.uint8), got[k].view(np.uint8)), f"{cfg.name}: {k} differs"
    assert not np.isnan(ref["out"]).any()
