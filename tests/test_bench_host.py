"""Host-side checks of bench.py (no GPU): the algorithmic byte and FLOP
figures its roofline divides by, against figures worked out by hand from the
workload definitions (KV, Q, output, mask and page-table bytes; one read of
the logits), and the one-GPU guard."""
import os
import subprocess
import sys

import numpy as np
import pytest

import tvgen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("cfg,mb", [(1, 0.060), (2, 81.8), (3, 639.2), (4, 544.2)])
def test_attention_bytes_match_hand_figures(cfg, mb):
    w = tvgen.make_workload(cfg, with_kv=False, with_logits=False)
    assert bench.attention_bytes(w) / 1e6 == pytest.approx(mb, abs=0.05 if mb > 1 else 0.001)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_attention_flops_between_prefix_only_and_dense_tree(cfg):
    # every row sees its whole prefix and at least itself, at most every node
    w = tvgen.make_workload(cfg, with_kv=False, with_logits=False)
    depth = np.stack([tvgen.tree_depths(p) for p in w.parents])
    f = bench.attention_flops(w, depth)
    per_key = w.Hq * 4 * w.D
    lo = sum(int(L) * w.N + w.N for L in w.prefix_lens) * per_key
    hi = sum((int(L) + w.N) * w.N for L in w.prefix_lens) * per_key
    assert lo <= f <= hi
    # the tree part is exactly the visible (ancestor-or-self) pairs
    tree = f - sum(int(L) * w.N for L in w.prefix_lens) * per_key
    assert tree == int((depth + 1).sum()) * per_key


@pytest.mark.parametrize("cfg,mb", [(1, 0.061), (2, 262.7), (3, 985.0), (4, 131.3)])
def test_greedy_accept_bytes_are_one_read_of_the_logits(cfg, mb):
    w = tvgen.make_workload(cfg, with_kv=False, with_logits=False)
    # the logits once, plus each row's draft token and parent in and argmax out
    assert bench.accept_bytes(w) == w.B * w.N * (w.V * 4 + 12)
    assert bench.accept_bytes(w) / 1e6 == pytest.approx(mb, abs=0.05 if mb > 1 else 0.001)


def test_node_counts_shrink_the_figures():
    w = tvgen.make_workload(2, with_kv=False, with_logits=False)
    sizes = np.full(w.B, w.N // 2, np.int32)
    assert bench.present(w, sizes).sum() == w.B * w.N // 2
    assert bench.accept_bytes(w, sizes) * 2 == bench.accept_bytes(w)
    assert bench.attention_bytes(w, sizes) < bench.attention_bytes(w)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
