"""Pools over a caller-owned device workspace (kv_workspace_bytes of the
calls' limits): the calls give the oracle's results from the workspace
alone, the coarsest plans (what a call that does not fit falls back to) too,
and calls past the limits fail before any device work."""

import numpy as np
import pytest

import paged_kv_cache_204_amd as pkv
import synth
from synth import Shape

from test_gpu_parity import REDUCED, parity, sample_ops
from test_workspace import desc_of, replay_calls

pytestmark = pytest.mark.gpu


def limits(wl):
    calls = list(replay_calls(wl))
    return max(c[1] for c in calls), max(c[2] for c in calls)


@pytest.mark.parametrize("name", ["mcts_small", "verify_small", "prefill_small", "commit_small", "dendrite_small"])
def test_reduced_workloads_in_a_workspace(dev, name):
    wl = REDUCED[name]
    parity(wl, ws_limits=limits(wl), label=f"{name}[workspace]")


@pytest.mark.parametrize("name,every", [("c4_mcts", 1), ("c5_verify", 1), ("c2_trellis_prefill", 1), ("c3_dendrite", 31)])
def test_configurations_in_a_workspace(dev, name, every):
    wl = synth.named(name)
    parity(wl, want=sample_ops(wl, every), ws_limits=limits(wl), label=f"{name}[workspace]")


@pytest.mark.parametrize("name", ["mcts_small", "verify_small", "prefill_small", "dendrite_small", "c4_mcts",
                                  "c5_verify"])
def test_coarse_plans(dev, name, monkeypatch):
    # every call planned as the coarsest plan a tight workspace falls back to
    monkeypatch.setenv("PKV_COARSE_PLANS", "1")
    wl = REDUCED[name] if name in REDUCED else synth.named(name)
    parity(wl, ws_limits=limits(wl), label=f"{name}[coarse]")


def test_calls_past_the_limits_fail_before_any_work(dev):
    import torch
    s = Shape(8, 2, 64, 16, 1, 64)
    d = desc_of(s)
    n = pkv.kv_pool_bytes(d) // 2
    k = torch.zeros(n, dtype=torch.int16, device="cuda")
    v = torch.zeros(n, dtype=torch.int16, device="cuda")
    need = pkv.kv_workspace_bytes(d, 2, 4)
    ws = torch.empty(need + 512, dtype=torch.uint8, device="cuda")
    # too small, misaligned
    for kw in (dict(workspace=ws, workspace_bytes=need - 1), dict(workspace=ws.data_ptr() + 16, workspace_bytes=need)):
        with pytest.raises(pkv.PkvError) as e:
            pkv.kv_pool_create(d, k, v, max_seqs=2, max_tree_nodes=4, **kw)
        assert e.value.code == pkv.PKV_ERR_ARG
    pool = pkv.kv_pool_create(d, k, v, workspace=ws, workspace_bytes=need, max_seqs=2, max_tree_nodes=4)
    st = torch.cuda.current_stream().cuda_stream
    try:
        ids = [pkv.seq_allocate(pool) for _ in range(3)]
        kv = torch.zeros(3 * 20 * 2 * 64, dtype=torch.int16, device="cuda")
        pkv.kv_append(pool, ids, 20, kv, kv, st)
        q = torch.zeros(3 * 8 * 64 * 8, dtype=torch.int16, device="cuda")
        out = torch.full((3 * 8, 8, 64), 7.0, device="cuda")
        calls = [
            lambda: pkv.paged_attn_decode(pool, 0, ids, q, 0.125, out, None, st),   # 3 sequences
            lambda: pkv.paged_attn_tree_verify(pool, 0, ids[:1], 5, [[-1, 0, 1, 2, 3]], q, 0.125, out, None, st),
            lambda: pkv.paged_attn_prefill(pool, 0, ids[:2], [5, 1], q, 0.125, out, None, st),
        ]
        for call in calls:
            with pytest.raises(pkv.PkvError) as e:
                call()
            assert e.value.code == pkv.PKV_ERR_ARG
        torch.cuda.synchronize()
        assert bool((out == 7.0).all())
        # within the limits the same pool works
        pkv.paged_attn_decode(pool, 0, ids[:2], q, 0.125, out, None, st)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(out[:2]).all())
    finally:
        pkv.kv_pool_destroy(pool)
