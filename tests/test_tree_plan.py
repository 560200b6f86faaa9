"""Tree decode plans (host only): shared segments with many rows go to MFMA
items as partial states, every other key to path items of at most 16 rows
whose steps carry the mask of the queries that see them.  A C++ driver
(tests/native/tree_plan_check.cpp, built here with g++ against the host
sources) replays workloads and checks every plan against the block tables:
each query's keys covered exactly once, its merge row listing exactly its
partial rows, steps inside their blocks."""

import math
import os
import shutil
import subprocess

import pytest

import synth
from synth import Shape

from test_plan_patch import ops_text

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "paged_kv_cache_204_amd", "csrc")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if not gxx:
        pytest.skip("g++ not found")
    exe = str(tmp_path_factory.mktemp("tree") / "tree_plan_check")
    subprocess.run([gxx, "-O1", "-std=c++17", f"-I{CSRC}", os.path.join(HERE, "native", "tree_plan_check.cpp"),
                    os.path.join(CSRC, "host", "plan.cpp"), os.path.join(CSRC, "host", "tree.cpp"),
                    os.path.join(CSRC, "host", "pool.cpp"), "-o", exe], check=True)
    return exe


def run(driver, wl, **env):
    e = dict(os.environ, **{f"TREE_CHECK_{k.upper()}": str(v) for k, v in env.items()})
    r = subprocess.run([driver], input=ops_text(wl), capture_output=True, text=True, env=e, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    trees, others = (int(x) for x in r.stdout.split()[1::2])
    return trees, others


CASES = {
    "c4_mcts": lambda: synth.named("c4_mcts"),
    "c3_dendrite": lambda: synth.named("c3_dendrite"),
    "c2_trellis": lambda: synth.named("c2_trellis"),
    # ragged 21-token edges (partial blocks at every level), G 4
    "mcts_ragged": lambda: synth.mcts_workload(
        "mcts_ragged", 14, Shape(32, 8, 128, 16, 1, 512), root_len=300, depth=3, fanout=3, edge_len=21,
        k_scale=1 / math.sqrt(128)),
    # 64-token blocks, G 8, wide fan-out
    "mcts_b64": lambda: synth.mcts_workload(
        "mcts_b64", 31, Shape(32, 4, 64, 64, 1, 512), root_len=700, depth=2, fanout=7, edge_len=90),
    # G 1: sixteen queries per path item
    "mcts_g1": lambda: synth.mcts_workload(
        "mcts_g1", 32, Shape(8, 8, 64, 32, 1, 1024), root_len=333, depth=3, fanout=4, edge_len=40),
    # shared prompt with repeated decode rounds (appends between)
    "trellis_small": lambda: synth.shared_prompt_workload(
        "trellis_small", 12, Shape(32, 4, 64, 32, 3, 128), prompt_len=200, n_sessions=5, shared_blocks=3,
        decode_steps=6),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_tree_plans_cover_every_key_once(driver, name):
    trees, _ = run(driver, CASES[name]())
    assert trees > 0


@pytest.mark.parametrize("name", ["c4_mcts", "mcts_ragged", "c3_dendrite"])
def test_tree_plans_under_other_cut_rules(driver, name):
    # everything shared through MFMA items / nothing but long runs / two parts
    # / long runs under many rows
    for env in ({"wide_rows": 1, "wide_tokens": 1}, {"wide_rows": 1 << 20, "path_tokens": 1 << 20},
                {"wide_rows": 4, "wide_tokens": 16, "max_parts": 2},
                {"wide_rows": 128, "wide_tokens": 256, "path_tokens": 1024}):
        trees, others = run(driver, CASES[name](), **env)
        assert trees + others > 0
