"""Host-side logic of bench.py (CPU only): the one-GPU guard, the tree
workload's path lengths and the source hash that ties committed counter
summaries to the kernel sources."""

import os
import subprocess
import sys

import numpy as np

import oracle
from gated_delta_rule_79_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args,
                          capture_output=True, text=True, env=env, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run_bench(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_several_ranks_are_refused():
    r = _run_bench(["--gpus", "1"], {"WORLD_SIZE": "2"})
    assert r.returncode == 2


def test_tree_depths_match_oracle_paths():
    _, par, _ = synth.make_tree_inputs(5, 23, 1, 16, 16, seed=5)
    depth = bench.tree_depths(par.numpy(), 23)
    for b in range(5):
        for i in range(23):
            assert depth[b][i] == len(oracle.tree_path(par.numpy()[b], i))


def test_tree_depths_chain_and_star():
    n = 9
    chain = np.arange(-1, n - 1)[None, :]
    star = np.full((1, n), -1)
    assert bench.tree_depths(chain, n)[0] == list(range(1, n + 1))
    assert bench.tree_depths(star, n)[0] == [1] * n


def test_source_hash_ignores_comments_only(tmp_path):
    a = tmp_path / "a.hip"
    a.write_text("int f() {  // first\n  return 1;\n}\n")
    h0 = bench.source_hash([str(a)])
    a.write_text("// header\nint f() {  // changed\n\n  return 1;\n}\n")
    assert bench.source_hash([str(a)]) == h0
    a.write_text("int f() {\n  return 2;\n}\n")
    assert bench.source_hash([str(a)]) != h0


def test_algorithmic_bytes_of_the_headline_forward():
    # B=1, T=4096, H=16, d=128, bf16 q/k/v/o, bf16 beta and scalar log alpha,
    # no state in or out: 4 rows of 128 bf16 and two gate scalars per
    # (token, head)
    _, byts = bench.algorithmic(1, 4096, 16, 128, 128, 64, 2, 2, "scalar", 1, False, False)
    assert byts == 4096 * 16 * (4 * 128 * 2 + 2 * 2)
