"""The decode entry point that allocates nothing (dsa_sparse_mla_decode_noalloc)
against the one that takes a workspace (dsa_sparse_mla_decode), through the C
ABI: two calls in a row, the second with a smaller input, each to the
tolerance of the hot path; and the size limit of the library's scratch."""
import numpy as np
import pytest

from dsa_top_sparse_amd import binding, synth
from parity_checks import check_attention, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    binding.lib()
    return torch


def _decode_pair(torch, n_q, offset, seed):
    cfg = synth.CONFIGS["C4"].replace(name=f"noalloc{n_q}", n_q=n_q, offset=offset, seed=seed, dup_frac=0.0)
    inputs = synth.generate(cfg)
    dev = binding.to_device(inputs)
    outs = binding.alloc_outputs(cfg)
    dims = binding.make_dims(cfg)
    binding.indexer_scores(dims, dev["qidx"], dev["w"], dev["kidx"], outs["scores"], outs["ld"])
    binding.topk_select(dims, outs["scores"], outs["ld"], outs["idx"])
    ws_bytes = binding.sparse_mla_decode_workspace_bytes(dims)
    assert ws_bytes > 0, "the case must take the split path"
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    ref_out = torch.empty_like(outs["out"])
    ref_lse = torch.empty_like(outs["lse"])
    binding.sparse_mla_decode(dims, dev["q"], dev["kv"], outs["idx"], ref_out, ref_lse, ws)
    out = torch.full_like(outs["out"], 7.0)
    lse = torch.full_like(outs["lse"], 7.0)
    say(f"no-alloc decode: n_q={n_q} offset={offset} partial bytes={ws_bytes}")
    binding.sparse_mla_decode_noalloc(dims, dev["q"], dev["kv"], outs["idx"], out, lse)
    torch.cuda.synchronize()
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    check_attention(o, l, ref_out.cpu().numpy().astype(np.float64), ref_lse.cpu().numpy().astype(np.float64),
                    f"no-alloc n_q={n_q}")
    say(f"no-alloc n_q={n_q}: bit-identical to the workspace call: "
        f"{bool(torch.equal(out, ref_out) and torch.equal(lse, ref_lse))}")


def test_noalloc_decode_matches_workspace_decode(torch_cuda):
    torch = torch_cuda
    # 4 queries (64 split partials), then 2 (32): the second call reads only
    # what it wrote over the first call's scratch contents
    _decode_pair(torch, 4, 49148, seed=61)
    _decode_pair(torch, 2, 30000, seed=62)


def test_noalloc_decode_rejects_beyond_scratch(torch_cuda):
    torch = torch_cuda
    # 16 queries at 16 splits of 128 slots need 256 partials (33.6 MB) > 32 MiB
    cfg = synth.CONFIGS["C4"].replace(n_q=16, offset=49136, dup_frac=0.0)
    dims = binding.make_dims(cfg)
    assert binding.sparse_mla_decode_workspace_bytes(dims) > 32 << 20
    q = torch.zeros((16, 64, 576), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((49152, 576), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((16, 2048), dtype=torch.int32, device="cuda")
    out = torch.empty((16, 64, 512), dtype=torch.float32, device="cuda")
    with pytest.raises(binding.DsaError) as e:
        binding.sparse_mla_decode_noalloc(dims, q, kv, idx, out)
    assert e.value.status == -5  # DSA_ERR_WORKSPACE
