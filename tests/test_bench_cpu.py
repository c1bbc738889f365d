"""bench.py's host-side arithmetic and its one-GPU contract (CPU tier)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from dsa_top_sparse_amd import synth  # noqa: E402


def _causal(cfg):
    return [cfg.offset + i + 1 for i in range(cfg.n_q)]


@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4"])
def test_algorithmic_work_closed_forms(name):
    # per-launch work from the definitions: the indexer's 2 H_I D_I flop and
    # 4-byte score per causal pair, the select's causal scores above k read
    # plus k indices written per query, the attention's 2 H (D_qk + D_v) flop
    # and one 1,152-byte row gathered per selected pair
    cfg = synth.CONFIGS[name]
    n = _causal(cfg)
    idx, topk, attn = bench.algorithmic_work(cfg)
    pairs = sum(n)
    sel = sum(min(cfg.top_k, x) for x in n)
    assert idx["flops"] == 2 * 4 * 128 * pairs
    assert topk["bytes"] == 4 * sum(x for x in n if x > cfg.top_k) + 4 * cfg.n_q * cfg.top_k
    assert attn["flops"] == 2 * 64 * (576 + 512) * sel
    assert attn["gathered_bytes"] == 1152 * sel


def test_algorithmic_work_headline_figures():
    # the figures the measurement section quotes for the 8k chunk at offset 8k
    idx, topk, attn = bench.algorithmic_work(synth.CONFIGS["C3"])
    assert abs(attn["flops"] - 2.336e12) / 2.336e12 < 1e-3  # 8,192 x 2,048 selected pairs
    assert abs(idx["flops"] - 1.031e11) / 1.031e11 < 1e-3   # 1.007e8 causal pairs
    assert abs(topk["bytes"] - 470e6) / 470e6 < 5e-3
    assert abs(attn["gathered_bytes"] - 19.33e9) / 19.33e9 < 1e-3
    # every C4 query has more than k keys too: the same attention work
    assert bench.algorithmic_work(synth.CONFIGS["C4"])[2]["flops"] == attn["flops"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
