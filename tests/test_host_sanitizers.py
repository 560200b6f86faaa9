"""The host sources (pool, planners, prefix cache) built with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer, driven by the native
checkers over the benchmark workloads and random traffic: any out-of-bounds
access, use after free, leak or undefined operation fails the run."""

import os
import shutil
import subprocess

import pytest

import synth
from synth import Shape
from test_plan_patch import ops_text

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "paged_kv_cache_204_amd", "csrc")
HOST = [os.path.join(CSRC, "host", f) for f in ("plan.cpp", "tree.cpp", "pool.cpp", "radix.cpp")]
FLAGS = ["-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


@pytest.fixture(scope="module")
def build(tmp_path_factory):
    gxx = shutil.which("g++")
    if not gxx:
        pytest.skip("g++ not found")
    out = tmp_path_factory.mktemp("sanitized")
    built = {}

    def make(name):
        if name not in built:
            exe = str(out / name)
            subprocess.run([gxx, *FLAGS, f"-I{CSRC}", os.path.join(HERE, "native", name + ".cpp"), *HOST, "-o", exe],
                           check=True)
            built[name] = exe
        return built[name]
    return make


def run(exe, args=(), stdin=None, env=None):
    r = subprocess.run([exe, *map(str, args)], input=stdin, capture_output=True, text=True, timeout=600,
                       env=dict(ENV, **(env or {})))
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    return r.stdout


def small(name):
    """Reduced forms of the configurations (the planners' code paths, in seconds)."""
    return {
        "c4_mcts": lambda: synth.named("c4_mcts"),
        "c1_tiny_fork": lambda: synth.named("c1_tiny_fork"),
        "dendrite": lambda: synth.fork_workload("san_dendrite", 51, Shape(32, 4, 64, 16, 1, 256), prefix_len=777,
                                                n_branches=6, branch_len=50, decode_steps=20),
        "trellis": lambda: synth.shared_prompt_workload("san_trellis", 52, Shape(32, 4, 64, 32, 3, 128),
                                                        prompt_len=200, n_sessions=5, shared_blocks=3,
                                                        decode_steps=6),
    }[name]()


@pytest.mark.parametrize("name", ["c4_mcts", "dendrite", "trellis", "c1_tiny_fork"])
def test_tree_planner(build, name):
    exe = build("tree_plan_check")
    wl = small(name)
    for env in ({"TREE_CHECK_MIN_WGS": "0"},
                {"TREE_CHECK_MIN_WGS": "0", "TREE_CHECK_WIDE_ROWS": "16", "TREE_CHECK_PATH_TOKENS": "128"}):
        run(exe, stdin=ops_text(wl), env=env)


@pytest.mark.parametrize("name", ["dendrite", "c1_tiny_fork"])
def test_decode_planner_and_patching(build, name):
    run(build("plan_patch_check"), stdin=ops_text(small(name)))


def test_prefill_planner(build):
    out = run(build("prefill_plan_check"), args=(7, 40))
    assert out.startswith("ok")


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_prefix_cache(build, seed):
    out = run(build("radix_drive"), args=(seed, 300))
    assert out.startswith("ok")
