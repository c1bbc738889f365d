"""GPU parity of the HIP path against the CPU oracle (``-m gpu``, MI355X).

Every case calls the library through its C ABI (``dsa_top_sparse_amd.binding``)
on seeded synthetic inputs and compares with ``oracle``:
  * the five workloads C0-C4 on EVERY query row, in blocks of rows: indexer
    scores and top-k indices bit-exact (the indices of both the two-step path
    and the fused indexer + select), attention within max |out - ref| <=
    4e-3, relative L2 <= 5e-3 (per block, hence over the whole tensor too) and
    |lse - ref| <= 1e-3; the top-k properties also on every row against the
    GPU's scores;
  * edge cases (ragged sizes, other shapes, long rows, ties, padding, restart,
    decode splits, chunked prefill) on all rows of smaller inputs.
"""
import math

import numpy as np
import pytest

import golden_cases
import oracle
from dsa_top_sparse_amd import binding, synth
from parity_checks import ATOL, LSE_ATOL, attention_errors, check_attention, check_topk_properties, say

pytestmark = pytest.mark.gpu

_say = say


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X")
    binding.lib()  # fails loudly when the HIP library is missing
    oracle.build(force=False)
    return torch


def run_gpu(torch, cfg, inputs, ld=None, with_lse=True):
    dev = binding.to_device(inputs)
    outs = binding.alloc_outputs(cfg, ld=ld, with_lse=with_lse)
    binding.run_chunk(cfg, dev, outs)
    torch.cuda.synchronize()
    return dev, outs


# --------------------------------------------------------- every query row

ROW_BLOCK = 1024  # oracle rows per test: seconds of host time each
WORKLOADS = ["C0", "C1", "C2", "C3", "C4"]
BLOCKS = [(name, b) for name in WORKLOADS
          for b in range(math.ceil(synth.CONFIGS[name].n_q / ROW_BLOCK))]

_results = {}  # one workload's GPU results at a time (host copies)


def gpu_results(torch, name):
    """Runs the whole path once per workload; returns (cfg, inputs, host outputs, error sums)."""
    if name not in _results:
        _results.clear()
        cfg = synth.CONFIGS[name]
        say(f"{name}: generate {cfg}")
        inputs = synth.generate(cfg)
        say(f"{name}: run GPU path")
        dev, outs = run_gpu(torch, cfg, inputs)
        say(f"{name}: top-k properties on every row")
        check_topk_properties(torch, outs["scores"], outs["idx"], cfg.offset, cfg.top_k, name)
        host = {k: outs[k].cpu().numpy() for k in ("scores", "idx", "out", "lse")}
        say(f"{name}: fused indexer + select")
        dims = binding.make_dims(cfg)
        ws = torch.empty(binding.indexer_topk_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
        fidx = torch.full_like(outs["idx"], 12345)
        binding.indexer_topk(dims, dev["qidx"], dev["w"], dev["kidx"], fidx, ws)
        torch.cuda.synchronize()
        host["fused_idx"] = fidx.cpu().numpy()
        del ws, fidx
        del dev, outs
        torch.cuda.empty_cache()
        _results[name] = (cfg, inputs, host, {"se": 0.0, "sr": 0.0, "max_abs": 0.0, "blocks": 0})
    return _results[name]


@pytest.mark.parametrize("name,block", BLOCKS, ids=[f"{n}-rows{b * ROW_BLOCK}" for n, b in BLOCKS])
def test_config_parity(torch_cuda, name, block):
    # Rows [block * 1024, +1024) of the workload against the oracle: scores and
    # indices bit-exact, attention and lse within tolerance.
    cfg, inputs, host, acc = gpu_results(torch_cuda, name)
    r0, r1 = block * ROW_BLOCK, min(cfg.n_q, (block + 1) * ROW_BLOCK)
    rows = list(range(r0, r1))
    say(f"{name}: oracle on rows {r0}..{r1 - 1}")
    ref = oracle.full_path(cfg, inputs, rows=rows)
    g_scores = host["scores"][r0:r1]
    bad = np.flatnonzero(np.any(g_scores.view(np.uint32) != ref["scores"].view(np.uint32), axis=1))
    assert bad.size == 0, f"{name}: scores differ on rows {(bad[:8] + r0).tolist()}"
    g_idx = host["idx"][r0:r1]
    bad = np.flatnonzero(np.any(g_idx != ref["idx"], axis=1))
    assert bad.size == 0, f"{name}: indices differ on rows {(bad[:8] + r0).tolist()}"
    bad = np.flatnonzero(np.any(host["fused_idx"][r0:r1] != ref["idx"], axis=1))
    assert bad.size == 0, f"{name}: fused indexer + select differs on rows {(bad[:8] + r0).tolist()}"
    check_attention(host["out"][r0:r1], host["lse"][r0:r1], ref["out"], ref["lse"], f"{name} rows {r0}..{r1 - 1}",
                    row_ids=rows)
    max_abs, _, se, sr, _ = attention_errors(host["out"][r0:r1], ref["out"])
    acc["se"] += se
    acc["sr"] += sr
    acc["max_abs"] = max(acc["max_abs"], max_abs)
    acc["blocks"] += 1
    if acc["blocks"] * ROW_BLOCK >= cfg.n_q:
        say(f"{name}: all {cfg.n_q} rows: attention max_abs={acc['max_abs']:.3e} "
            f"rel_l2={math.sqrt(acc['se'] / acc['sr']):.3e}")


@pytest.mark.parametrize("ld_pad", [3, 0])
def test_ragged_fast_path_all_rows(torch_cuda, ld_pad):
    torch = torch_cuda
    cfg = synth.CONFIGS["C2"].replace(name="ragged", n_q=77, offset=1003, top_k=100, seed=31)
    inputs = synth.generate(cfg)
    # ld_pad 3: odd row stride (the select's unaligned path, one score per store
    # in the indexer, -inf padding columns); 0: t_ctx = 1,080 is a multiple of
    # 4, so full 32-key blocks take the indexer's 16-byte stores and the
    # partial last query block the per-score stores
    ld = cfg.t_ctx + ld_pad
    _say(f"ragged: {cfg} ld={ld}")
    dev, outs = run_gpu(torch, cfg, inputs, ld=ld)
    ref = oracle.full_path(cfg, inputs)
    ref_s = oracle.indexer_scores(cfg.n_q, cfg.offset, inputs["qidx"], inputs["w"], inputs["kidx"], ld=ld)
    assert np.array_equal(outs["scores"].cpu().numpy().view(np.uint32), ref_s.view(np.uint32))
    assert np.array_equal(outs["idx"].cpu().numpy(), ref["idx"])
    check_attention(outs["out"].cpu().numpy(), outs["lse"].cpu().numpy(), ref["out"], ref["lse"], "ragged")


@pytest.mark.parametrize("n_q,offset,d_idx", [
    (512, 0, 128),     # 8 query blocks, 4 key ranges: every XCD's walk starts at the first range
    (1024, 3000, 128),  # 16 query blocks, 32 key ranges: staggered walks, 2 blocks per XCD and range
    (576, 700, 128),    # 9 query blocks: contiguous runs of units per XCD
    (512, 2000, 64),    # the per-wave indexer (d_idx 64) on the staggered walk
])
def test_indexer_unit_walks(torch_cuda, n_q, offset, d_idx):
    # The indexer maps workgroups to (key range, query block) units by a
    # staggered walk per XCD when the query blocks are a multiple of 8 and by
    # contiguous runs otherwise. Every score of every row, bit-exact, on a
    # buffer filled with NaN first, so that a unit left out shows.
    torch = torch_cuda
    cfg = synth.CONFIGS["C2"].replace(name=f"units_{n_q}_{offset}_{d_idx}", n_q=n_q, offset=offset, d_idx=d_idx,
                                      seed=n_q + offset + d_idx)
    _say(f"indexer unit walk: {cfg}")
    inputs = synth.generate(cfg)
    dev = binding.to_device(inputs)
    ld = cfg.t_ctx
    scores = torch.full((cfg.n_q, ld), float("nan"), dtype=torch.float32, device="cuda")
    binding.indexer_scores(binding.make_dims(cfg), dev["qidx"], dev["w"], dev["kidx"], scores, ld)
    torch.cuda.synchronize()
    ref = oracle.indexer_scores(cfg.n_q, cfg.offset, inputs["qidx"], inputs["w"], inputs["kidx"], ld=ld)
    assert np.array_equal(scores.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("d_idx", [128, 64])
def test_indexer_negative_weights_and_zero_sums(torch_cuda, d_idx):
    # Weights in {-2, -1, 1, 2}: the small-integer indexer products stay exact,
    # so scores are still bit-exact; head sums cancel to exactly zero and
    # negative weights meet ReLU zeros, and every zero must come out as +0.
    # d_idx 128 runs the LDS-staged indexer, 64 the per-wave one.
    torch = torch_cuda
    cfg = synth.CONFIGS["C2"].replace(name=f"negw_{d_idx}", n_q=200, offset=900, d_idx=d_idx, top_k=256,
                                      seed=77 + d_idx)
    _say(f"negative weights: {cfg}")
    inputs = synth.generate(cfg)
    rng = np.random.default_rng(cfg.seed)
    inputs["w"] = rng.choice(np.array([-2.0, -1.0, 1.0, 2.0], dtype=np.float32), size=inputs["w"].shape)
    dev, outs = run_gpu(torch, cfg, inputs)
    dims = binding.make_dims(cfg)
    ws = torch.empty(max(1, binding.indexer_topk_workspace_bytes(dims)), dtype=torch.uint8, device="cuda")
    fidx = torch.full_like(outs["idx"], 12345)
    binding.indexer_topk(dims, dev["qidx"], dev["w"], dev["kidx"], fidx, ws)
    torch.cuda.synchronize()
    ref = oracle.full_path(cfg, inputs)
    s = outs["scores"].cpu().numpy()
    assert np.array_equal(s.view(np.uint32), ref["scores"].view(np.uint32))
    zeros = s == 0.0
    assert zeros.sum() > 1000 and not np.signbit(s[zeros]).any()
    assert (s < 0).any()  # negative scores occur and are kept as they are
    assert np.array_equal(outs["idx"].cpu().numpy(), ref["idx"])
    assert np.array_equal(fidx.cpu().numpy(), ref["idx"])
    check_attention(outs["out"].cpu().numpy(), outs["lse"].cpu().numpy(), ref["out"], ref["lse"], cfg.name)


def test_small_contexts_dense_and_hilo(torch_cuda):
    # offset 0, 100 queries, k = 2048: every row is dense causal with 1..100
    # keys, the few-key regime where P is split into hi + lo bf16 parts.
    torch = torch_cuda
    cfg = synth.CONFIGS["C1"].replace(name="dense_small", n_q=100, offset=0, seed=32)
    inputs = synth.generate(cfg)
    _say(f"dense_small: {cfg}")
    dev, outs = run_gpu(torch, cfg, inputs)
    ref = oracle.full_path(cfg, inputs)
    assert np.array_equal(outs["idx"].cpu().numpy(), ref["idx"])
    check_attention(outs["out"].cpu().numpy(), outs["lse"].cpu().numpy(), ref["out"], ref["lse"], "dense_small")
    # single key: query 0 attends to key 0 only -> its value row, exactly
    v0 = synth.bf16_bits_to_f32(inputs["kv"][0, : cfg.d_latent])
    assert np.array_equal(outs["out"][0].cpu().numpy(), np.tile(v0, (cfg.n_heads, 1)))


def test_topk_all_equal_scores_fallback(torch_cuda):
    # q_idx = 0 -> every causal score is +0.0, so the k lowest indices win and
    # the candidate set (the whole row) is larger than the select's LDS buffer.
    torch = torch_cuda
    cfg = synth.CONFIGS["C2"].replace(name="all_equal", n_q=40, offset=9000, seed=33)
    inputs = synth.generate(cfg)
    inputs["qidx"] = np.zeros_like(inputs["qidx"])
    _say("all_equal")
    dev, outs = run_gpu(torch, cfg, inputs)
    s = outs["scores"].cpu().numpy()
    for i in range(cfg.n_q):
        assert np.all(s[i, : cfg.offset + i + 1].view(np.uint32) == 0)
    exp = np.tile(np.arange(cfg.top_k, dtype=np.int32), (cfg.n_q, 1))
    assert np.array_equal(outs["idx"].cpu().numpy(), exp)


def test_topk_strictly_increasing_rows(torch_cuda):
    # Distinct scores increasing with the key index: the last k causal keys win.
    torch = torch_cuda
    n_q, off, k = 33, 5000, 2048
    ld = off + n_q
    scores = torch.arange(ld, dtype=torch.float32, device="cuda").repeat(n_q, 1).contiguous()
    idx = torch.empty((n_q, k), dtype=torch.int32, device="cuda")
    cfg = synth.CONFIGS["C2"].replace(n_q=n_q, offset=off)
    binding.topk_select(binding.make_dims(cfg), scores, ld, idx)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for i in range(n_q):
        p = off + i
        assert np.array_equal(got[i], np.arange(p - k + 1, p + 1, dtype=np.int32))


def test_topk_random_floats_and_negative_zero(torch_cuda):
    # General fp32 scores (negatives, -0.0, +0.0, wide exponents) vs Python's sort.
    torch = torch_cuda
    rng = np.random.default_rng(77)
    n_q, off, k = 24, 3000, 700
    ld = off + n_q
    s = (rng.standard_normal((n_q, ld)) * np.exp(rng.uniform(-20, 20, size=(n_q, ld)))).astype(np.float32)
    s[rng.random(s.shape) < 0.05] = 0.0
    s[rng.random(s.shape) < 0.05] = -0.0
    s[:, 100:130] = 7.0  # a block of ties
    for i in range(n_q):
        s[i, off + i + 1:] = -np.inf
    st = torch.from_numpy(s).cuda()
    idx = torch.empty((n_q, k), dtype=torch.int32, device="cuda")
    cfg = synth.CONFIGS["C2"].replace(n_q=n_q, offset=off, top_k=k)
    binding.topk_select(binding.make_dims(cfg), st, ld, idx)
    torch.cuda.synchronize()
    ref = oracle.topk_select(n_q, off, k, s)
    assert np.array_equal(idx.cpu().numpy(), ref)


@pytest.mark.parametrize("shape", [
    # (n_heads, d_latent, d_rope, n_idx_heads, d_idx, top_k): which kernels run
    (16, 128, 32, 4, 64, 96),    # MFMA indexer for d_idx 64; plain attention in bf16
    (64, 512, 64, 4, 256, 130),  # MFMA indexer for d_idx 256; top_k % 4 != 0: plain attention
    (8, 64, 0, 2, 48, 50),       # plain indexer in bf16 (2 heads, width 48); plain attention
    (64, 512, 64, 4, 32, 64),    # MFMA indexer for d_idx 32; fast attention with a short index row
])
def test_other_shapes_bf16(torch_cuda, shape):
    # Every step on bf16 inputs whose shapes leave the 4 x 128 indexer and the
    # 64-head 512 + 64 attention: scores and indices bit-exact, attention
    # within tolerance, every row against the oracle.
    torch = torch_cuda
    h, dl, dr, hi_, di, k = shape
    cfg = synth.CONFIGS["C2"].replace(name=f"shape{shape}", n_q=70, offset=301, n_heads=h, d_latent=dl,
                                      d_rope=dr, n_idx_heads=hi_, d_idx=di, top_k=k, seed=sum(shape))
    inputs = synth.generate(cfg)
    _say(f"other shape: {shape}")
    dev, outs = run_gpu(torch, cfg, inputs)
    ref = oracle.full_path(cfg, inputs)
    assert np.array_equal(outs["scores"][:, : cfg.t_ctx].cpu().numpy().view(np.uint32),
                          oracle.indexer_scores(cfg.n_q, cfg.offset, inputs["qidx"], inputs["w"],
                                                inputs["kidx"]).view(np.uint32))
    assert np.array_equal(outs["idx"].cpu().numpy(), ref["idx"])
    check_attention(outs["out"].cpu().numpy(), outs["lse"].cpu().numpy(), ref["out"], ref["lse"], f"{shape}")


@pytest.mark.parametrize("off", [30000, 70000])
@pytest.mark.parametrize("order", ["increasing", "decreasing", "random"])
def test_topk_long_rows_speculation(torch_cuda, order, off):
    # Both select kernels guess from the start of each row: the filtered one a
    # threshold from its first 2,048 keys, the streamed one a bucket from its
    # first 8,192. Increasing scores make the guess far too low (the candidates
    # overflow LDS), decreasing scores make it too high (fewer than k keys pass
    # it); both must fall back to a second read. Random integer scores take the
    # one-pass path. Ties at several places; 30,000-key rows (filtered kernel)
    # and 70,000-key rows (streamed kernel); every row against the oracle.
    torch = torch_cuda
    rng = np.random.default_rng(len(order))
    n_q, k = 10, 2048
    ld = off + n_q
    j = np.arange(ld, dtype=np.float64)
    if order == "increasing":
        base = np.floor(j / 3)
    elif order == "decreasing":
        base = ld - j  # the k-th key's bucket lies below the guessed one
    else:
        base = rng.integers(0, 400, size=ld).astype(np.float64)
    s = np.tile(base, (n_q, 1)).astype(np.float32)
    s[:, 5000:5100] = s[0, 5000]  # a block of equal scores
    for i in range(n_q):
        s[i, off + i + 1:] = -np.inf
    _say(f"topk long rows: {order} offset={off}")
    st = torch.from_numpy(s).cuda()
    idx = torch.empty((n_q, k), dtype=torch.int32, device="cuda")
    cfg = synth.CONFIGS["C2"].replace(n_q=n_q, offset=off, top_k=k)
    binding.topk_select(binding.make_dims(cfg), st, ld, idx)
    torch.cuda.synchronize()
    ref = oracle.topk_select(n_q, off, k, s)
    assert np.array_equal(idx.cpu().numpy(), ref)


@pytest.mark.parametrize("off,k", [(12000, 4096), (12000, 9000), (40000, 10000)])
def test_topk_large_k(torch_cuda, off, k):
    # k above the select's LDS candidate capacity (6,144): the refinement and
    # the emit re-read the row from global memory, in both select kernels;
    # integer-valued scores with ties on even rows, random floats on odd rows.
    torch = torch_cuda
    rng = np.random.default_rng(off + k)
    n_q = 8
    ld = off + n_q
    s = rng.integers(0, 200, size=(n_q, ld)).astype(np.float32)
    s[1::2] = rng.standard_normal((n_q // 2, ld)).astype(np.float32)
    for i in range(n_q):
        s[i, off + i + 1:] = -np.inf
    _say(f"topk large k: offset={off} k={k}")
    st = torch.from_numpy(s).cuda()
    idx = torch.empty((n_q, k), dtype=torch.int32, device="cuda")
    cfg = synth.CONFIGS["C2"].replace(n_q=n_q, offset=off, top_k=k)
    binding.topk_select(binding.make_dims(cfg), st, ld, idx)
    torch.cuda.synchronize()
    ref = oracle.topk_select(n_q, off, k, s)
    assert np.array_equal(idx.cpu().numpy(), ref)


@pytest.mark.parametrize("off", [9000, 30000])
def test_topk_constant_low_bits(torch_cuda, off):
    # Scores 1 + m/8 + 2^-20 (m random in [0, 8)): every score has the same
    # exponent and the same nonzero low mantissa bits, so the select's second
    # refinement level is skipped with a threshold whose last bits are not 0;
    # and 2 + m/8 (low bits 0). Register and streaming kernels, vs the oracle.
    torch = torch_cuda
    rng = np.random.default_rng(off)
    n_q, k = 12, 2048
    ld = off + n_q
    m = rng.integers(0, 8, size=(n_q, ld)).astype(np.float64)
    s = (1.0 + m / 8 + 2.0 ** -20).astype(np.float32)
    s[1::2] = (2.0 + m[1::2] / 8).astype(np.float32)
    assert np.all(s[0].view(np.uint32) & 0x3FF == s[0, 0].view(np.uint32) & 0x3FF)
    for i in range(n_q):
        s[i, off + i + 1:] = -np.inf
    _say(f"topk constant low bits: offset={off}")
    st = torch.from_numpy(s).cuda()
    idx = torch.empty((n_q, k), dtype=torch.int32, device="cuda")
    cfg = synth.CONFIGS["C2"].replace(n_q=n_q, offset=off, top_k=k)
    binding.topk_select(binding.make_dims(cfg), st, ld, idx)
    torch.cuda.synchronize()
    ref = oracle.topk_select(n_q, off, k, s)
    assert np.array_equal(idx.cpu().numpy(), ref)


@pytest.mark.parametrize("off,k,ld_pad", [(7000, 2048, 0), (17000, 2048, 0), (30000, 2048, 4), (60000, 1500, 0),
                                          (65520, 2048, 0), (65521, 2048, 0), (70000, 2048, 0), (5000, 999, 1),
                                          (2040, 2000, 0), (4090, 2048, 0), (16368, 2048, 0)])
def test_topk_row_lengths(torch_cuda, off, k, ld_pad):
    # Row lengths across the select kernels: the filtered kernel up to 65,536
    # keys (that limit hit exactly and passed by one key), rows shorter than
    # its 2,048-key threshold sample, rows around its candidate capacity, the
    # streamed kernel beyond, and unaligned leading dimensions (streamed
    # kernel); integer-valued scores with many ties plus random floats, vs
    # the oracle.
    torch = torch_cuda
    rng = np.random.default_rng(off + k)
    n_q = 16
    ld = off + n_q + ld_pad
    s = rng.integers(0, 300, size=(n_q, ld)).astype(np.float32)
    s[::2] = rng.standard_normal((n_q // 2, ld)).astype(np.float32)
    for i in range(n_q):
        s[i, off + i + 1:] = -np.inf
    _say(f"topk rows: offset={off} k={k} ld={ld}")
    st = torch.from_numpy(s).cuda()
    idx = torch.empty((n_q, k), dtype=torch.int32, device="cuda")
    cfg = synth.CONFIGS["C2"].replace(n_q=n_q, offset=off, top_k=k)
    binding.topk_select(binding.make_dims(cfg), st, ld, idx)
    torch.cuda.synchronize()
    ref = oracle.topk_select(n_q, off, k, s)
    assert np.array_equal(idx.cpu().numpy(), ref)


def test_topk_kth_far_above_sample_threshold(torch_cuda):
    # The row's first 2,048 keys (the filtered select's threshold sample) are
    # small, and k keys far larger sit later in the row: the threshold from the
    # sample keeps a candidate set that holds the top k, but the k-th key lies
    # far above the threshold, so the select finds its top digit from the
    # candidates instead of the threshold-relative histogram. Ties among the
    # large keys on some rows. Every row vs the oracle.
    torch = torch_cuda
    rng = np.random.default_rng(11)
    n_q, off, k = 12, 14000, 2048
    ld = off + n_q
    s = rng.random((n_q, ld)).astype(np.float32)
    s[:, 2048:] *= 0.5  # below the sample's threshold (about 0.8)
    for i in range(n_q):
        big = rng.choice(np.arange(2048, off), size=k + 40, replace=False)
        s[i, big] = (1000.0 + rng.integers(0, 50 if i % 2 else 5000, size=big.size)).astype(np.float32)
        s[i, off + i + 1:] = -np.inf
    _say("topk k-th far above the sample threshold")
    st = torch.from_numpy(s).cuda()
    idx = torch.empty((n_q, k), dtype=torch.int32, device="cuda")
    cfg = synth.CONFIGS["C2"].replace(n_q=n_q, offset=off, top_k=k)
    binding.topk_select(binding.make_dims(cfg), st, ld, idx)
    torch.cuda.synchronize()
    ref = oracle.topk_select(n_q, off, k, s)
    assert np.array_equal(idx.cpu().numpy(), ref)


def test_attention_arbitrary_slots(torch_cuda):
    # -1 padding anywhere, out-of-causal-range indices, a query with no valid
    # slot (out = 0, lse = -inf), unsorted and repeated keys.
    torch = torch_cuda
    cfg = synth.CONFIGS["C2"].replace(name="slots", n_q=6, offset=3000, top_k=96, seed=34)
    inputs = synth.generate(cfg)
    rng = np.random.default_rng(5)
    idx = rng.integers(0, cfg.offset, size=(cfg.n_q, cfg.top_k)).astype(np.int32)
    idx[0, :] = -1
    idx[1, rng.random(cfg.top_k) < 0.5] = -1
    idx[2, :] = -1
    idx[2, 50] = 17
    idx[3, 10:20] = cfg.offset + 3 + 1  # one past query 3's position: skipped
    idx[4, :] = 5  # the same key 96 times
    dev = binding.to_device(inputs)
    out = torch.empty((cfg.n_q, cfg.n_heads, cfg.d_latent), dtype=torch.float32, device="cuda")
    lse = torch.empty((cfg.n_q, cfg.n_heads), dtype=torch.float32, device="cuda")
    gidx = torch.from_numpy(idx).cuda()
    binding.sparse_mla_fwd(binding.make_dims(cfg), dev["q"], dev["kv"], gidx, out, lse)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.sparse_mla(cfg.n_q, cfg.offset, cfg.sm_scale, cfg.d_latent, inputs["q"],
                                     inputs["kv"], idx)
    assert np.all(out[0].cpu().numpy() == 0.0) and np.all(np.isneginf(lse[0].cpu().numpy()))
    check_attention(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, "slots")


def test_attention_long_rows_and_late_first_tile(torch_cuda):
    # Rows longer than the 2,048 of the workloads (the index ring is refilled
    # many times), a partial last tile (top_k = 4100), a first valid slot
    # beyond tile 8 and one only in the last slot, and a bf16 row length that
    # is not a multiple of 4 (plain kernel).
    torch = torch_cuda
    for top_k in (4100, 99):
        cfg = synth.CONFIGS["C2"].replace(name=f"long{top_k}", n_q=6, offset=20000, top_k=top_k, seed=35)
        inputs = synth.generate(cfg)
        rng = np.random.default_rng(6)
        idx = rng.integers(0, cfg.offset, size=(cfg.n_q, cfg.top_k)).astype(np.int32)
        idx[1, :300] = -1                      # first valid tile 9
        idx[2, :-1] = -1                       # only the last slot
        idx[3, rng.random(cfg.top_k) < 0.9] = -1
        idx[4, : cfg.top_k // 2] = cfg.offset + 4 + 7  # beyond query 4's position
        dev = binding.to_device(inputs)
        out = torch.empty((cfg.n_q, cfg.n_heads, cfg.d_latent), dtype=torch.float32, device="cuda")
        lse = torch.empty((cfg.n_q, cfg.n_heads), dtype=torch.float32, device="cuda")
        _say(f"long rows: top_k={top_k}")
        binding.sparse_mla_fwd(binding.make_dims(cfg), dev["q"], dev["kv"], torch.from_numpy(idx).cuda(), out, lse)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle.sparse_mla(cfg.n_q, cfg.offset, cfg.sm_scale, cfg.d_latent, inputs["q"],
                                         inputs["kv"], idx)
        check_attention(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, f"long{top_k}")


def test_chunk_invariance_and_determinism(torch_cuda):
    # The 8k chunk of C3 as four 2k chunks (offsets 8192, 10240, 12288, 14336)
    # gives the same scores, index sets, outputs and lse, bit for bit;
    # repeating a call is bitwise stable.
    torch = torch_cuda
    cfg = synth.CONFIGS["C3"]
    inputs = synth.generate(cfg)
    _say("chunk invariance: whole chunk")
    dev, outs = run_gpu(torch, cfg, inputs)
    whole_idx = outs["idx"].clone()
    whole_out = outs["out"].clone()
    whole_lse = outs["lse"].clone()
    binding.run_chunk(cfg, dev, outs)
    torch.cuda.synchronize()
    assert torch.equal(outs["idx"], whole_idx) and torch.equal(outs["out"], whole_out)
    for c in range(4):
        sub = cfg.replace(n_q=2048, offset=cfg.offset + 2048 * c)
        rows = slice(2048 * c, 2048 * (c + 1))
        sdev = {"qidx": dev["qidx"][rows].contiguous(), "w": dev["w"][rows].contiguous(),
                "q": dev["q"][rows].contiguous(), "kidx": dev["kidx"][: sub.t_ctx].contiguous(),
                "kv": dev["kv"][: sub.t_ctx].contiguous()}
        souts = binding.alloc_outputs(sub)
        _say(f"chunk invariance: sub-chunk {c}")
        binding.run_chunk(sub, sdev, souts)
        torch.cuda.synchronize()
        assert torch.equal(souts["idx"], whole_idx[rows])
        assert torch.equal(souts["scores"], outs["scores"][rows, : sub.t_ctx])
        # attention outputs are chunk-invariant too (each query's work depends only on its own row)
        assert torch.equal(souts["out"], whole_out[rows])
        assert torch.equal(souts["lse"], whole_lse[rows])


def test_chunked_prefill_replay(torch_cuda):
    # The pages' 8,192-token prefill from empty caches, in 2,048-token chunks
    # (offsets 0 / 2,048 / 4,096 / 6,144) through dsa_prefill_chunk, against
    # the same prompt as one 8,192-token chunk: caches, index sets, outputs
    # and lse are bit-identical; sampled rows (around chunk edges) match the
    # oracle.
    from dsa_top_sparse_amd import prefill
    torch = torch_cuda
    cfg = synth.PROMPTS["P8K"]
    inputs = synth.generate(cfg)
    dev = binding.to_device(inputs)
    runs = {}
    for chunk in (8192, 2048, 1000):
        _say(f"prefill replay: chunk {chunk}")
        o = prefill.alloc_prompt_outputs(cfg)
        prefill.run_prefill(cfg, dev, chunk, o)
        torch.cuda.synchronize()
        runs[chunk] = o
    whole = runs[8192]
    assert torch.equal(whole["kv_cache"].view(torch.int16), dev["kv"].view(torch.int16))
    assert torch.equal(whole["kidx_cache"].view(torch.int16), dev["kidx"].view(torch.int16))
    for chunk in (2048, 1000):
        for key in ("idx", "out", "lse"):
            assert torch.equal(runs[chunk][key], whole[key]), (chunk, key)
    rows = [0, 1, 999, 1000, 2047, 2048, 2049, 4095, 4096, 6143, 6144, 8191]
    ref = oracle.full_path(cfg, inputs, rows=rows)
    assert np.array_equal(whole["idx"][rows].cpu().numpy(), ref["idx"])
    check_attention(whole["out"][rows].cpu().numpy(), whole["lse"][rows].cpu().numpy(), ref["out"], ref["lse"],
                    "prefill replay")


def test_prefill_replay_17k_prompt_2k_chunks(torch_cuda):
    # The pages' 17.5k-token prompt (17,536 tokens) from empty caches in
    # 2,048-token chunks (nine calls, the last of 1,152 tokens; once more with
    # the indexer and select fused) and in 8,192-token chunks, against the
    # whole prompt as one chunk: index sets,
    # outputs and lse bit-identical; rows on both sides of every chunk edge
    # against the oracle.
    from dsa_top_sparse_amd import prefill
    torch = torch_cuda
    cfg = synth.PROMPTS["P17K"]
    say(f"prefill 17k: generate {cfg}")
    inputs = synth.generate(cfg)
    dev = binding.to_device(inputs)
    T = cfg.n_q
    scores = torch.empty((T, T), dtype=torch.float32, device="cuda")
    runs = {}
    for chunk in (T, 8192, 2048):
        say(f"prefill 17k: chunk {chunk}")
        o = prefill.alloc_prompt_outputs(cfg)
        prefill.run_prefill(cfg, dev, chunk, o, scores=scores)
        torch.cuda.synchronize()
        runs[chunk] = {k: o[k] for k in ("idx", "out", "lse")}
    # 2k chunks again with steps 1-2 fused (no score matrix)
    say("prefill 17k: chunk 2048, indexer + select fused")
    o = prefill.alloc_prompt_outputs(cfg)
    prefill.run_prefill(cfg, dev, 2048, o, fused=True)
    torch.cuda.synchronize()
    runs["2048-fused"] = {k: o[k] for k in ("idx", "out", "lse")}
    for chunk in (8192, 2048, "2048-fused"):
        for key in ("idx", "out", "lse"):
            assert torch.equal(runs[chunk][key], runs[T][key]), (chunk, key)
    edges = sorted({r for c in range(0, T, 2048) for r in (c - 1, c, c + 1) if 0 <= r < T} | {T - 1})
    say(f"prefill 17k: oracle on {len(edges)} chunk-edge rows")
    ref = oracle.full_path(cfg, inputs, rows=edges)
    got = runs[2048]
    assert np.array_equal(got["idx"][edges].cpu().numpy(), ref["idx"])
    check_attention(got["out"][edges].cpu().numpy(), got["lse"][edges].cpu().numpy(), ref["out"], ref["lse"],
                    "prefill 17k", row_ids=edges)


def test_self_test_and_launch_limits(torch_cuda):
    # The matrix-core layout self-test passes on this device (and is cached),
    # and every entry point's launch-limit check lets the workloads' kernels run
    # (the config parity tests above already launched them).
    binding.self_test()
    binding.self_test()


@pytest.mark.parametrize("n_q", [1, 3, 4, 40])
def test_decode_step(torch_cuda, n_q):
    # A decode step (1-4 tokens, and a 40-token draft) against a ~49k-token
    # cache: indexer -> top-k -> split attention, vs the oracle and vs the
    # unsplit attention call.
    torch = torch_cuda
    cfg = synth.CONFIGS["C4"].replace(name=f"decode{n_q}", n_q=n_q, offset=49152 - n_q, seed=40 + n_q,
                                      dup_frac=0.0)
    inputs = synth.generate(cfg)
    dev, outs = run_gpu(torch, cfg, inputs)  # indexer + top-k + unsplit attention
    dims = binding.make_dims(cfg)
    ws_bytes = binding.sparse_mla_decode_workspace_bytes(dims)
    assert ws_bytes > 0
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    out = torch.empty_like(outs["out"])
    lse = torch.empty_like(outs["lse"])
    _say(f"decode: n_q={n_q} ws={ws_bytes}")
    binding.sparse_mla_decode(dims, dev["q"], dev["kv"], outs["idx"], out, lse, ws)
    torch.cuda.synchronize()
    ref = oracle.full_path(cfg, inputs)
    assert np.array_equal(outs["idx"].cpu().numpy(), ref["idx"])
    check_attention(out.cpu().numpy(), lse.cpu().numpy(), ref["out"], ref["lse"], f"decode{n_q}")
    # splits of <= 128 slots take the hi/lo-P path, so the split result is the
    # more accurate one; the two agree to the parity tolerance
    assert float((out - outs["out"]).abs().max()) <= ATOL
    assert float((lse - outs["lse"]).abs().max()) <= LSE_ATOL


def test_decode_empty_and_partial_splits(torch_cuda):
    # Index rows whose first half (eight whole splits) holds no valid slot, a
    # row with a single valid slot, and a row with none.
    torch = torch_cuda
    cfg = synth.CONFIGS["C4"].replace(name="decode_pad", n_q=3, offset=20000, seed=47, dup_frac=0.0)
    inputs = synth.generate(cfg)
    rng = np.random.default_rng(8)
    idx = rng.integers(0, cfg.offset, size=(cfg.n_q, cfg.top_k)).astype(np.int32)
    idx[0, :1024] = -1
    idx[1, :] = -1
    idx[1, 1500] = 777
    idx[2, :] = -1
    dev = binding.to_device(inputs)
    dims = binding.make_dims(cfg)
    ws = torch.empty(binding.sparse_mla_decode_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    out = torch.empty((cfg.n_q, cfg.n_heads, cfg.d_latent), dtype=torch.float32, device="cuda")
    lse = torch.empty((cfg.n_q, cfg.n_heads), dtype=torch.float32, device="cuda")
    binding.sparse_mla_decode(dims, dev["q"], dev["kv"], torch.from_numpy(idx).cuda(), out, lse, ws)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.sparse_mla(cfg.n_q, cfg.offset, cfg.sm_scale, cfg.d_latent, inputs["q"], inputs["kv"], idx)
    check_attention(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, "decode_pad")
    assert np.all(out[2].cpu().numpy() == 0.0) and np.all(np.isneginf(lse[2].cpu().numpy()))


def test_attention_reference_restart(torch_cuda):
    # One selected key, in a late tile, is aligned with head 5's query so that
    # its logit exceeds every logit of the first tile by ~60 (natural log):
    # far beyond the lag the kernel lets its per-head reference maximum keep,
    # so the query must restart with a raised reference.
    torch = torch_cuda
    cfg = synth.CONFIGS["C2"].replace(name="restart", n_q=4, offset=3000, seed=35)
    inputs = synth.generate(cfg)
    rng = np.random.default_rng(9)
    idx = np.sort(rng.choice(cfg.offset, size=(cfg.n_q, cfg.top_k), replace=True), axis=1).astype(np.int32)
    j = int(idx[0, 700])  # tile 21 of query 0
    q5 = synth.bf16_bits_to_f32(inputs["q"][0, 5]).astype(np.float64)
    kvj = 60.0 * q5 / (np.linalg.norm(q5) ** 2) / cfg.sm_scale  # q5 . kvj * scale = 60
    inputs["kv"][j] = synth.f32_to_bf16_bits(kvj.astype(np.float32))
    dev = binding.to_device(inputs)
    out = torch.empty((cfg.n_q, cfg.n_heads, cfg.d_latent), dtype=torch.float32, device="cuda")
    lse = torch.empty((cfg.n_q, cfg.n_heads), dtype=torch.float32, device="cuda")
    binding.sparse_mla_fwd(binding.make_dims(cfg), dev["q"], dev["kv"], torch.from_numpy(idx).cuda(), out, lse)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.sparse_mla(cfg.n_q, cfg.offset, cfg.sm_scale, cfg.d_latent, inputs["q"], inputs["kv"], idx)
    assert ref_l[0, 5] > 55.0  # the planted logit dominates head 5
    check_attention(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, "restart")


def test_golden_fixtures_through_the_abi(torch_cuda):
    # The hand-worked fixtures of tests/golden (fp32 inputs, so the general
    # kernels run) through the C ABI: scores and indices exact, attention to
    # fp32 rounding. Each top-k case runs at its own (unaligned) leading
    # dimension and padded with -inf to a multiple of 4, so both the streamed
    # and the register-resident select see it.
    torch = torch_cuda
    F32 = binding.DSA_F32
    _say("golden fixtures")
    g = golden_cases.load("indexer_hand.json")
    q_idx = torch.from_numpy(golden_cases.array(g["q_idx"])).cuda()
    n_h, d_i = q_idx.shape[1], q_idx.shape[2]
    dims = binding.Dims(g["n_q"], g["offset"], 1, 1, 0, n_h, d_i, 1, 1.0, F32, F32)
    scores = torch.full((g["n_q"], g["ld"]), 7.0, dtype=torch.float32, device="cuda")
    binding.indexer_scores(dims, q_idx, torch.from_numpy(golden_cases.array(g["w_idx"])).cuda(),
                           torch.from_numpy(golden_cases.array(g["k_idx"])).cuda(), scores, g["ld"])
    torch.cuda.synchronize()
    got, want = scores.cpu().numpy(), golden_cases.array(g["scores"])
    assert np.array_equal(got, want) and np.array_equal(np.signbit(got), np.signbit(want))

    for case in golden_cases.load("topk_hand.json")["cases"]:
        s = golden_cases.array(case["scores"])
        for ld in (s.shape[1], (s.shape[1] + 3) // 4 * 4):
            sp = np.full((case["n_q"], ld), -np.inf, dtype=np.float32)
            sp[:, : s.shape[1]] = s
            dims = binding.Dims(case["n_q"], case["offset"], 1, 1, 0, 1, 1, case["k"], 1.0, F32, F32)
            idx = torch.full((case["n_q"], case["k"]), 12345, dtype=torch.int32, device="cuda")
            binding.topk_select(dims, torch.from_numpy(sp).cuda(), ld, idx)
            torch.cuda.synchronize()
            assert idx.cpu().tolist() == case["idx"], (case["offset"], ld)

    g = golden_cases.load("attention_hand.json")
    dims = binding.Dims(g["n_q"], g["offset"], g["n_heads"], g["d_latent"], g["d_rope"], 1, 1,
                        len(g["idx"][0]), g["sm_scale"], F32, F32)
    out = torch.full((g["n_q"], g["n_heads"], g["d_latent"]), 7.0, dtype=torch.float32, device="cuda")
    lse = torch.full((g["n_q"], g["n_heads"]), 7.0, dtype=torch.float32, device="cuda")
    binding.sparse_mla_fwd(dims, torch.from_numpy(golden_cases.array(g["q"])).cuda(),
                           torch.from_numpy(golden_cases.array(g["kv"])).cuda(),
                           torch.from_numpy(golden_cases.array(g["idx"], np.int32)).cuda(), out, lse)
    torch.cuda.synchronize()
    assert np.max(np.abs(out.cpu().numpy() - np.array(g["out"]))) < g["tol"]
    assert np.max(np.abs(lse.cpu().numpy() - np.array(g["lse"]))) < g["tol"]
