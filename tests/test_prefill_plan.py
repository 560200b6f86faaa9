"""Prefill planning (host only).  A C++ driver (tests/native/prefill_plan_check.cpp,
built here with g++ against the host sources) plans random prefill calls --
shared roots, forks with their own prompts, ragged and zero counts, every
block size and head grouping, planner settings -- and checks that the items
let through exactly the causal (query, key) pairs, each once, with in-range
mask shifts, kernel-sized items and the sequences' own blocks."""

import os
import shutil
import subprocess

import pytest

import paged_kv_cache_204_amd as pkv

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "paged_kv_cache_204_amd", "csrc")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if not gxx:
        pytest.skip("g++ not found")
    exe = str(tmp_path_factory.mktemp("prefill") / "prefill_plan_check")
    subprocess.run([gxx, "-O1", "-std=c++17", f"-I{CSRC}",
                    os.path.join(HERE, "native", "prefill_plan_check.cpp"),
                    os.path.join(CSRC, "host", "plan.cpp"), os.path.join(CSRC, "host", "tree.cpp"),
                    os.path.join(CSRC, "host", "pool.cpp"),
                    "-o", exe], check=True)
    return exe


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_prefill_plans_cover_exactly_the_causal_pairs(driver, seed):
    r = subprocess.run([driver, str(seed), "150"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr


def test_prefill_on_a_host_only_pool_is_an_argument_error():
    desc = dict(num_blocks=8, block_size=4, num_layers=1, num_q_heads=4, num_kv_heads=2, head_dim=8)
    pool = pkv.kv_pool_create(desc, None, None)
    try:
        s = pkv.seq_allocate(pool)
        pkv.kv_append(pool, [s], 5, None, None, None)
        with pytest.raises(pkv.PkvError) as e:
            pkv.paged_attn_prefill(pool, 0, [s], [5], None, 0.5, None)
        assert e.value.code == pkv.PKV_ERR_ARG
        assert pkv.seq_block_table(pool, s) == ([0, 1], 5)
    finally:
        pkv.kv_pool_destroy(pool)
