"""paged_attn_decode_layers: the decode calls of a step over all layers in
one C-ABI call (one launch for the direct plan of short queries) give the
oracle's result for every layer, and per-layer paged_attn_decode's bit for
bit."""

import numpy as np
import pytest

import paged_kv_cache_204_amd as pkv
import synth
from synth import Shape

from gpu_harness import GpuPool, to_dev
from test_gpu_parity import Agg, oracle_run

pytestmark = pytest.mark.gpu


def layer_groups(wl):
    """Runs of decode ops over the same sequences at layers 0 .. L-1."""
    groups, cur = [], []
    for idx, op in enumerate(wl.ops):
        if op[0] == "decode" and (not cur or (op[1] == wl.ops[cur[0]][1] and op[2] == len(cur))):
            cur.append(idx)
        else:
            if cur:
                groups.append(cur)
            cur = [idx] if op[0] == "decode" and op[2] == 0 else []
    if cur:
        groups.append(cur)
    return [g for g in groups if len(g) == wl.shape.num_layers]


def run_batched(wl, want, monkeypatch=None):
    import torch
    s = wl.shape
    gp = GpuPool(s, wl.free_order())
    h, got = {}, {}
    groups = {g[0]: g for g in layer_groups(wl)}
    try:
        idx = 0
        while idx < len(wl.ops):
            op = wl.ops[idx]
            if op[0] == "alloc":
                h[op[1]] = pkv.seq_allocate(gp.pool)
            elif op[0] == "fork":
                h[op[2]] = pkv.seq_fork(gp.pool, h[op[1]])
            elif op[0] == "free":
                pkv.seq_free(gp.pool, h.pop(op[1]))
            elif op[0] == "append":
                k, v = wl.append_data(op[3], len(op[1]), op[2])
                pkv.kv_append(gp.pool, [h[x] for x in op[1]], op[2], to_dev(k), to_dev(v), gp.stream)
            elif op[0] == "decode":
                g = groups[idx]
                ids = [h[x] for x in op[1]]
                L, n = len(g), len(ids)
                q = torch.cat([to_dev(wl.decode_query(wl.ops[j][3], n)) for j in g])
                out = torch.empty((L, n, s.num_q_heads, s.head_dim), device="cuda")
                lse = torch.empty((L, n, s.num_q_heads), device="cuda")
                pkv.paged_attn_decode_layers(gp.pool, 0, L, ids, q, wl.sm_scale, out, lse, gp.stream)
                if any(j in want for j in g):
                    # the same calls one layer at a time, bit for bit
                    for l, j in enumerate(g):
                        o1 = torch.empty((n, s.num_q_heads, s.head_dim), device="cuda")
                        l1 = torch.empty((n, s.num_q_heads), device="cuda")
                        pkv.paged_attn_decode(gp.pool, l, ids, q[l * n:(l + 1) * n], wl.sm_scale, o1, l1,
                                              gp.stream)
                        torch.cuda.synchronize()
                        assert torch.equal(o1, out[l]) and torch.equal(l1, lse[l]), (wl.name, j)
                        got[j] = (out[l].cpu().numpy(), lse[l].cpu().numpy())
                idx = g[-1]
            idx += 1
        torch.cuda.synchronize()
    finally:
        gp.close()
    return got


@pytest.mark.parametrize("name,every,env", [
    ("trellis_layers", 1, {}),
    ("trellis_layers", 1, {"PKV_DIRECT_MAX_TOKENS": "0"}),   # segment plan: a launch per layer
    ("c2_trellis", 23, {}),
])
def test_layer_batched_decode(dev, name, every, env, monkeypatch):
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    if name == "trellis_layers":
        wl = synth.shared_prompt_workload("trellis_layers", 41, Shape(32, 4, 64, 32, 5, 128), prompt_len=200,
                                          n_sessions=5, shared_blocks=3, decode_steps=4)
    else:
        wl = synth.named(name)
    groups = layer_groups(wl)
    assert groups
    want = {j for g in groups[::every] + [groups[-1]] for j in g}
    exp, _, _ = oracle_run(wl, want=want)
    got = run_batched(wl, want)
    agg = Agg()
    for j in sorted(want):
        agg.add(got[j], exp[j], f"{name} op {j}")
    agg.done(f"{name}[layers{'/' + ','.join(env) if env else ''}]")
