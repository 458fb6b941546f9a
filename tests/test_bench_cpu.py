"""Host-side checks of bench.py: the one-GPU contract and the algorithmic
counts its roofline divides by (no GPU needed)."""
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=300, env=env)


def test_more_than_one_gpu_is_refused():
    r = _run_bench(["--gpus", "2"])
    assert r.returncode == 2 and "one GPU only" in r.stderr, (r.returncode, r.stderr[-300:])
    r = _run_bench([], {"WORLD_SIZE": "2"})
    assert r.returncode == 2 and "one GPU only" in r.stderr, (r.returncode, r.stderr[-300:])


def test_tree_depths():
    # chain: depths 1..T; star below the root: 1 then 2s; the hand-worked
    # tree of the oracle pins (node 2 a sibling of node 1 under node 0)
    assert list(bench.tree_depths(np.array([-1, 0, 1, 2]))) == [1, 2, 3, 4]
    assert list(bench.tree_depths(np.array([-1, 0, 0, 0]))) == [1, 2, 2, 2]
    assert list(bench.tree_depths(np.array([-1, 0, 0]))) == [1, 2, 2]
    assert list(bench.tree_depths(np.array([-1, -1, 1]))) == [1, 1, 2]


def test_algorithmic_counts_by_hand():
    # Two sequences, H = 2, bf16: sequence 0 has 3 prefix keys and the tree
    # 0 <- 1 (node 1's parent is node 0), sequence 1 no prefix and one node.
    # Visible (row, key) pairs per head: node 0 of seq 0 sees 3 + 1 keys,
    # node 1 sees 3 + 2, node 0 of seq 1 sees 0 + 1: 10 in all.
    x = SimpleNamespace(cfg=SimpleNamespace(dtype="bf16", heads=2, batch=2),
                        parents=np.array([-1, 0, -1], np.int32), tree_indptr=np.array([0, 2, 3]),
                        prefix_lens=np.array([3, 0]), kv_lens=np.array([5, 1]))
    flops, bytes_, kv_tokens, pairs = bench.algorithmic_counts(x)
    assert pairs == 10 and kv_tokens == 6
    assert flops == 2 * 2 * (576 + 512) * 10
    # KV rows (576 bf16 + a 4-byte page-table entry each), Q (3 nodes x 2
    # heads x 576 bf16), out + lse (513 fp32 per row) and the 3 parents
    assert bytes_ == 6 * (576 * 2 + 4) + 6 * 576 * 2 + 6 * 513 * 4 + 3 * 4
