"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Attention outputs: max |d| <= 4e-3 and mean |d| <= 5e-4 against the float64
oracle, over every compared element of a workload; lse within 4e-3.
Pool contents after copy-on-write and the K/V scatter: bit-exact against the
oracle's own pool copy, on every filled slot of every held block.
Invariants that must hold bit for bit on the GPU: a forked child reads
exactly what its parent reads, and physical block placement does not change
any output.
"""

import math

import numpy as np
import pytest

import synth
from synth import Shape
from oracle import run_program

pytestmark = pytest.mark.gpu

TOL_MAX = 4e-3
TOL_MEAN = 5e-4


def oracle_run(wl, want=None, free_order="default"):
    kw = {} if isinstance(free_order, str) else {"free_order": free_order}
    results = {}
    last = None
    for idx, op, pool, handles, r in run_program(wl, want=want, **kw):
        if r is not None:
            results[idx] = r
        last = (pool, handles)
    return results, last[0], last[1]


class Agg:
    def __init__(self):
        self.n = 0
        self.sum = 0.0
        self.max = 0.0

    def add(self, got, want, label):
        out_g, lse_g = got
        out_w, lse_w = want
        assert out_g.shape == out_w.shape, label
        assert np.isfinite(out_g).all(), f"{label}: non-finite output"
        d = np.abs(out_g.astype(np.float64) - out_w)
        dl = np.abs(lse_g.astype(np.float64) - lse_w)
        assert d.max() <= TOL_MAX, f"{label}: max |d| {d.max():.3e}"
        assert dl.max() <= TOL_MAX, f"{label}: lse max |d| {dl.max():.3e}"
        self.n += d.size
        self.sum += d.sum()
        self.max = max(self.max, d.max())

    def done(self, label):
        assert self.n > 0
        mean = self.sum / self.n
        print(f"[parity] {label}: max |d| {self.max:.3e} mean |d| {mean:.3e}", flush=True)
        from conftest import record_margin
        record_margin(label, self.max, mean, self.n, TOL_MAX, TOL_MEAN)
        assert mean <= TOL_MEAN, f"{label}: mean |d| {mean:.3e}"
        return mean


def check_pool_contents(oracle_pool):
    """pool_cb for run_gpu: device pool bits == oracle pool bits on filled slots."""
    def cb(gp, handles):
        k, v = gp.pool_bits()
        om = oracle_pool
        held = [b for b in range(om.N) if om.rc[b] > 0]
        assert held
        for b in held:
            n = om.filled[b]
            # device [L][N][Hkv][B][D] vs oracle [N][B][L][Hkv][D]
            kd = k[:, b, :, :n, :].transpose(2, 0, 1, 3)
            vd = v[:, b, :, :n, :].transpose(2, 0, 1, 3)
            assert np.array_equal(kd, om.kbits[b, :n]), f"K block {b}"
            assert np.array_equal(vd, om.vbits[b, :n]), f"V block {b}"
    return cb


def parity(wl, want=None, check_pool=True, label=None, ws_limits=None, ws_bytes=None):
    from gpu_harness import run_gpu, log
    label = label or wl.name
    log(f"[gpu] parity {label}: oracle")
    exp, opool, _ = oracle_run(wl, want=want)
    log(f"[gpu] parity {label}: device run ({len(wl.ops)} ops)")
    got = run_gpu(wl, want=set(exp), pool_cb=check_pool_contents(opool) if check_pool else None,
                  ws_limits=ws_limits, ws_bytes=ws_bytes)
    agg = Agg()
    for idx in exp:
        agg.add(got[idx], exp[idx], f"{label} op {idx}")
    mean = agg.done(label)
    log(f"[gpu] parity {label}: ok, {len(exp)} calls, max {agg.max:.2e} mean {mean:.2e}")
    return got, exp


# ------------------------------------------------ reduced workloads (fast)

def reduced():
    return {
        # shared prompt, ragged prompt end (200 % 32 != 0), 3 layers
        "trellis_small": synth.shared_prompt_workload(
            "trellis_small", 12, Shape(32, 4, 64, 32, 3, 128), prompt_len=200,
            n_sessions=5, shared_blocks=3, decode_steps=6),
        # fork at a half-filled block: every branch copies it on first append
        "dendrite_small": synth.fork_workload(
            "dendrite_small", 13, Shape(32, 4, 64, 16, 1, 256), prefix_len=777,
            n_branches=6, branch_len=50, decode_steps=5, permute=True),
        # search tree with ragged 21-token edges (copies at every level)
        "mcts_small": synth.mcts_workload(
            "mcts_small", 14, Shape(32, 8, 128, 16, 1, 512), root_len=300, depth=3,
            fanout=3, edge_len=21, k_scale=1 / math.sqrt(128)),
        # draft-tree verify, context not block aligned
        "verify_small": synth.verify_workload(
            "verify_small", 15, Shape(32, 8, 128, 16, 1, 256), n_seqs=3, ctx_len=333,
            n_nodes=17, tree_depth=5, permute=True),
        "verify_ctx0": synth.verify_workload(
            "verify_ctx0", 16, Shape(8, 2, 64, 8, 1, 64), n_seqs=2, ctx_len=0,
            n_nodes=64, tree_depth=10),
        "verify_one_node": synth.verify_workload(
            "verify_one_node", 17, Shape(8, 8, 64, 16, 1, 64), n_seqs=4, ctx_len=100,
            n_nodes=1, tree_depth=1),
        "c1_tiny_fork": synth.named("c1_tiny_fork"),
        # causal prefill after a cached prefix: ragged counts (one window,
        # exactly one, just over one, several), a count of 0
        "prefill_small": synth.prefill_workload(
            "prefill_small", 18, Shape(32, 8, 128, 16, 1, 256), shared_len=77,
            own_lens=[1, 63, 64, 65, 130, 0, 200]),
        # whole prompts new (no cached prefix), G 4 at D 64, 32-token blocks
        "prefill_ctx0": synth.prefill_workload(
            "prefill_ctx0", 19, Shape(32, 4, 64, 32, 2, 128), shared_len=0,
            own_lens=[300, 5, 64]),
        # speculative rounds: verify a draft tree, commit the accepted paths
        # (pool contents checked bit for bit), decode after the commit
        "commit_small": synth.verify_commit_workload(
            "commit_small", 21, Shape(32, 8, 128, 16, 2, 256), n_seqs=3, ctx_len=77, n_nodes=20,
            tree_depth=5, rounds=2, permute=True),
        # forks share the tree blocks: commits copy the blocks they write
        "commit_forked": synth.verify_commit_workload(
            "commit_forked", 22, Shape(32, 4, 64, 8, 1, 256), n_seqs=4, ctx_len=45, n_nodes=33,
            tree_depth=7, rounds=2, fork_after=True),
        # a sequence and its fork commit different paths of the tree they
        # share in one call: the second writes in place blocks the first
        # reads, so the commit runs the sequences one after the other
        "commit_shared": synth.Workload(
            "commit_shared", 23, Shape(16, 4, 64, 4, 1, 128),
            [("alloc", 0), ("append", (0,), 50, 1), ("append", (0,), 16, 2), ("fork", 0, 1),
             ("verify", (0, 1), 0, 16, 2), ("commit", (0, 1), 16, 2, 10), ("append", (0, 1), 1, 6),
             ("decode", (0, 1), 0, 7)],
            1.0 / math.sqrt(64), tree_depth=6),
        # repeated prefill calls: the same call at the next layer (plan reused),
        # the same arguments after an append (pool changed: planned afresh),
        # other counts
        "prefill_repeat": synth.Workload(
            "prefill_repeat", 20, Shape(32, 8, 128, 16, 2, 128),
            [("alloc", 0), ("append", (0,), 40, 1), ("fork", 0, 1), ("fork", 0, 2), ("fork", 0, 3),
             ("append", (1, 2, 3), 20, 5),
             ("prefill", (1, 2, 3), 0, (20, 20, 20), 6), ("prefill", (1, 2, 3), 1, (20, 20, 20), 7),
             ("append", (1, 2, 3), 5, 8),
             ("prefill", (1, 2, 3), 0, (20, 20, 20), 9), ("prefill", (1, 2, 3), 1, (25, 5, 0), 10),
             ("prefill", (3, 1), 1, (45, 1), 11)],
            1.0 / math.sqrt(128)),
    }


REDUCED = reduced()

# Decode calls of few, short queries run the direct kernel (one workgroup per
# query and kv head over all its keys); the same calls can be forced onto the
# split path (shared-prefix items, partial states, merge) or, past the default
# limits, onto the direct kernel.  Planner settings are read from the
# environment when a pool is created.
PATHS = {
    "auto": {},
    "split": {"PKV_DIRECT_MAX_TOKENS": "0"},
    "direct": {"PKV_DIRECT_MAX_TOKENS": "100000", "PKV_DIRECT_MAX_WGS": "100000"},
    # split path with the chunk lengths picked for parallelism alone: long
    # shared prefixes give queries more partial states than a merge row
    # carries inline, so the merge walks its part list
    "manyparts": {"PKV_DIRECT_MAX_TOKENS": "0", "PKV_MAX_PARTS": "0"},
    # tree decode plans for batches of any size: path items over the trie
    # (shared runs re-read by every item below them) ...
    "tree": {"PKV_DIRECT_MAX_TOKENS": "0", "PKV_TREE_MIN_WGS": "0"},
    # ... and with shared runs through MFMA items (partial states in a launch
    # before the path items, which merge them)
    "treewide": {"PKV_DIRECT_MAX_TOKENS": "0", "PKV_TREE_MIN_WGS": "0", "PKV_TREE_WIDE_ROWS": "16",
                 "PKV_TREE_WIDE_TOKENS": "32", "PKV_TREE_PATH_TOKENS": "256"},
    # the wide-run rule the MCTS tree met before: the root as MFMA items
    "treeroot": {"PKV_TREE_WIDE_ROWS": "128", "PKV_TREE_WIDE_TOKENS": "256", "PKV_TREE_PATH_TOKENS": "1024"},
}


def set_path(monkeypatch, path):
    for k, v in PATHS[path].items():
        monkeypatch.setenv(k, v)


@pytest.mark.parametrize("path", ["auto", "split", "tree", "treewide"])
@pytest.mark.parametrize("name", list(REDUCED))
def test_reduced_workload_parity(dev, name, path, monkeypatch):
    set_path(monkeypatch, path)
    parity(REDUCED[name], label=f"{name}[{path}]")


# Shapes at the edges of what the kernels take: block sizes 1..128, GQA group
# 1..16 (and a non-power-of-two group), head_dim 64 / 128, ragged lengths.
SHAPES = [
    (Shape(4, 4, 64, 1, 1, 700), "B1_G1"),
    (Shape(8, 1, 64, 2, 2, 400), "B2_G8"),
    (Shape(16, 1, 128, 4, 1, 200), "B4_G16"),
    (Shape(12, 4, 128, 8, 1, 128), "B8_G3"),
    (Shape(32, 4, 64, 64, 1, 32), "B64_G8"),
    (Shape(32, 8, 128, 128, 1, 16), "B128_G4"),
]


@pytest.mark.parametrize("path", ["auto", "split"])
@pytest.mark.parametrize("shape,label", SHAPES, ids=[s[1] for s in SHAPES])
def test_shape_edges(dev, shape, label, path, monkeypatch):
    set_path(monkeypatch, path)
    wl = synth.fork_workload(f"edge_{label}", 20 + SHAPES.index((shape, label)), shape,
                             prefix_len=131, n_branches=3, branch_len=67, decode_steps=2,
                             permute=True)
    parity(wl, label=f"edge_{label}[{path}]")
    if path == "auto":
        tree = synth.verify_workload(f"edge_tree_{label}", 40 + SHAPES.index((shape, label)),
                                     shape, n_seqs=2, ctx_len=70, n_nodes=9, tree_depth=4)
        parity(tree)
        pre = synth.prefill_workload(f"edge_prefill_{label}", 50 + SHAPES.index((shape, label)),
                                     shape, shared_len=70, own_lens=[9, 70, 1])
        parity(pre)


# Direct decode at its edges: fewer 32-token steps than waves (1..9 keys),
# ragged lengths within one call, lengths around the step size, G 1 / 3 / 16
# at both head dims (eight- and four-wave kernels).  At head_dim 64 calls of
# at most 768 keys load every step of a wave in one round and longer ones
# roll two steps ahead: the fifth case's calls hold 765 .. 769 keys (both
# forms, 768 the last one-round call); the sixth has 16-token blocks (two
# per step) and G 16, the seventh 64-token blocks (half a block per step).
# Calls of more workgroups than CUs at head_dim 64 and at most 576 keys run
# two workgroups per CU with step-indexed V tiles: the eighth case (320
# workgroups, 514 .. 516 keys), the ninth (300, ragged 21 .. 469 keys, so
# some waves have no step), the tenth (280 workgroups at 651 .. 720 keys,
# past the step-indexed tiles: the one-round form again).
DIRECT_CASES = [
    # shape, prefix, own keys of branch i = base + i * inc, branches[, decode steps]
    (Shape(8, 8, 64, 16, 1, 64), 1, 0, 1, 6),
    (Shape(24, 8, 64, 4, 1, 256), 31, 1, 16, 5),
    (Shape(16, 1, 128, 16, 1, 256), 64, 0, 31, 4),
    (Shape(32, 4, 128, 32, 1, 512), 200, 290, 9, 7),
    (Shape(32, 4, 64, 32, 1, 256), 760, 4, 0, 3, 5),
    (Shape(16, 1, 64, 16, 1, 256), 40, 0, 100, 6),
    (Shape(32, 4, 64, 64, 1, 64), 100, 3, 50, 5),
    (Shape(32, 4, 64, 32, 1, 1024), 256, 257, 0, 80, 3),
    (Shape(16, 2, 64, 16, 1, 4096), 20, 0, 3, 150, 2),
    (Shape(32, 4, 64, 32, 1, 2048), 600, 50, 1, 70, 2),
]


def ragged_fork(name, cfg_id, shape, prefix, base, inc, n, decode_steps=3):
    ops = [("alloc", 0), ("append", (0,), prefix, 1)]
    kids = tuple(range(1, n + 1))
    for c in kids:
        ops.append(("fork", 0, c))
    for i, c in enumerate(kids):
        if base + i * inc:
            ops.append(("append", (c,), base + i * inc, len(ops)))
    for _ in range(decode_steps):
        ops.append(("append", kids, 1, len(ops)))
        ops.append(("decode", kids, 0, len(ops)))
    return synth.Workload(name, cfg_id, shape, ops, 1.0 / math.sqrt(shape.head_dim),
                          permute_free_list=True)


@pytest.mark.parametrize("case", range(len(DIRECT_CASES)))
def test_direct_decode_edges(dev, case, monkeypatch):
    set_path(monkeypatch, "direct")
    shape, prefix, base, inc, n, *steps = DIRECT_CASES[case]
    parity(ragged_fork(f"direct_{case}", 70 + case, shape, prefix, base, inc, n, *steps),
           label=f"direct_{case}")


# Planner settings (read from the environment when a pool is created) pick
# different kernel variants for the same call: four- or eight-wave MFMA
# workgroups, one or two row tiles per wave, few or many key chunks, the
# VALU path for everything it can take.  Every setting must keep parity.
# (the split-path settings also turn direct decode plans off)
_SPLIT = {"PKV_DIRECT_MAX_TOKENS": "0"}
KNOBS = [
    {"PKV_MFMA_WAVES": "4", "PKV_MFMA_ROW_TILES": "2", **_SPLIT},
    {"PKV_MFMA_WAVES": "8", "PKV_MFMA_ROW_TILES": "2", **_SPLIT},
    {"PKV_MFMA_ROW_TILES": "1", **_SPLIT},
    {"PKV_TARGET_MFMA_WGS": "16", "PKV_TARGET_WGS": "16", **_SPLIT},
    {"PKV_TARGET_MFMA_WGS": "4096", "PKV_TARGET_WGS": "4096", "PKV_MAX_CHUNK": "64", "PKV_MAX_PARTS": "0",
     **_SPLIT},
    {"PKV_MFMA_MIN_ROWS": "0", **_SPLIT},
    {"PKV_UNSHARE_MAX_QUERIES": "0", **_SPLIT},
    {"PKV_UNSHARE_MAX_QUERIES": "64", "PKV_UNSHARE_MAX_TOKENS": "100000", **_SPLIT},
    PATHS["direct"],
]


@pytest.mark.parametrize("knobs", KNOBS, ids=["-".join(f"{k[4:].lower()}{v}" for k, v in kn.items())
                                              for kn in KNOBS])
def test_planner_settings_keep_parity(dev, knobs, monkeypatch):
    for k, v in knobs.items():
        monkeypatch.setenv(k, v)
    tag = "-".join(f"{k[4:].lower()}{v}" for k, v in knobs.items())
    # 64 nodes x G 4 = 256 rows per sequence: eight-wave tiles are possible
    parity(synth.verify_workload(f"knob_verify_{tag}", 60, Shape(32, 8, 128, 16, 1, 128), n_seqs=2,
                                 ctx_len=301, n_nodes=64, tree_depth=6), check_pool=False)
    # G 16 (MFMA only) with 16 branches over one prefix: a 256-row shared tile
    parity(synth.fork_workload(f"knob_fork_{tag}", 61, Shape(16, 1, 128, 16, 1, 256),
                               prefix_len=203, n_branches=16, branch_len=29, decode_steps=2,
                               permute=True), check_pool=False)
    # G 4 decode with a prefix shared by 3 branches: VALU and MFMA items mixed
    parity(synth.fork_workload(f"knob_mixed_{tag}", 62, Shape(32, 8, 64, 16, 1, 256),
                               prefix_len=260, n_branches=12, branch_len=41, decode_steps=2),
           check_pool=False)
    # causal prefill of ragged prompts after a shared prefix
    parity(synth.prefill_workload(f"knob_prefill_{tag}", 63, Shape(32, 4, 64, 16, 1, 256),
                                  shared_len=150, own_lens=[100, 7, 64, 260]), check_pool=False)


# ------------------------------------------------------- full-size workloads

def sample_ops(wl, every):
    idx = [i for i, op in enumerate(wl.ops) if op[0] in ("decode", "verify", "prefill")]
    keep = set(idx[::every])
    keep.add(idx[-1])
    return keep


@pytest.mark.parametrize("name,every,path", [
    ("c1_tiny_fork", 1, "auto"), ("c1_tiny_fork", 1, "split"),
    ("c2_trellis", 23, "auto"), ("c2_trellis", 23, "split"),
    ("c3_dendrite", 9, "auto"), ("c3_dendrite", 31, "direct"), ("c3_dendrite", 31, "manyparts"),
    ("c3_dendrite_aligned", 31, "auto"),
    ("c3_dendrite", 31, "tree"),
    ("c4_mcts", 1, "auto"), ("c4_mcts", 1, "treeroot"), ("c4_mcts_folded", 1, "auto"), ("c5_verify", 1, "auto"),
    ("c2_trellis_prefill", 1, "auto"), ("c5_verify_commit", 1, "auto"),
])
def test_full_workload_parity(dev, name, every, path, monkeypatch):
    """The five workloads at full size, launched as the benchmark launches
    them (path "auto"), and the small-batch decode ones also on the other
    decode path; every call runs on the GPU, the oracle checks a sample of
    calls (all of them for single-call workloads)."""
    set_path(monkeypatch, path)
    wl = synth.named(name)
    parity(wl, want=sample_ops(wl, every), check_pool=name != "c2_trellis", label=f"{name}[{path}]")


# ---------------------------------------------------------------- edges

def small_shape():
    return Shape(8, 2, 64, 16, 1, 64)


def test_empty_and_noop_calls(dev):
    import torch
    import paged_kv_cache_204_amd as pkv
    from gpu_harness import GpuPool, log
    log("[gpu] empty / no-op calls")
    gp = GpuPool(small_shape())
    try:
        s = pkv.seq_allocate(gp.pool)
        q = torch.zeros((1, 8, 64), dtype=torch.int16, device="cuda")
        out = torch.full((1, 8, 64), 7.0, device="cuda")
        with pytest.raises(pkv.PkvError) as e:
            pkv.paged_attn_decode(gp.pool, 0, [s], q, 0.125, out, None, gp.stream)
        assert e.value.code == pkv.PKV_ERR_EMPTY
        pkv.paged_attn_decode(gp.pool, 0, [], q, 0.125, out, None, gp.stream)
        pkv.kv_append(gp.pool, [s], 0, None, None, gp.stream)
        pkv.kv_append(gp.pool, [], 5, None, None, gp.stream)
        with pytest.raises(pkv.PkvError) as e:
            pkv.paged_attn_decode(gp.pool, 1, [s], q, 0.125, out, None, gp.stream)
        assert e.value.code == pkv.PKV_ERR_ARG
        torch.cuda.synchronize()
        assert bool((out == 7.0).all())
    finally:
        gp.close()


def test_single_key_returns_v_exactly(dev):
    """len 1: softmax weight exactly 1, so out equals the stored V bits."""
    import torch
    import paged_kv_cache_204_amd as pkv
    from gpu_harness import GpuPool, to_dev, log
    log("[gpu] single key")
    shape = small_shape()
    wl = synth.fork_workload("single", 60, shape, prefix_len=1, n_branches=1, branch_len=0)
    gp = GpuPool(shape)
    try:
        s = pkv.seq_allocate(gp.pool)
        k, v = wl.append_data(1, 1, 1)
        pkv.kv_append(gp.pool, [s], 1, to_dev(k), to_dev(v), gp.stream)
        q = to_dev(wl.decode_query(2, 1))
        out = torch.empty((1, 8, 64), device="cuda")
        lse = torch.empty((1, 8), device="cuda")
        pkv.paged_attn_decode(gp.pool, 0, [s], q, 0.125, out, lse, gp.stream)
        o = out.cpu().numpy()
        vf = (v.astype(np.uint32) << 16).view(np.float32)[0, 0, 0]   # [Hkv][D]
        for h in range(8):
            assert np.array_equal(o[0, h], vf[h // 4])
    finally:
        gp.close()


def test_fork_and_duplicates_read_identically(dev):
    """A forked child and its parent, and a sequence listed twice, give
    bit-identical outputs for the same query."""
    import torch
    import paged_kv_cache_204_amd as pkv
    from gpu_harness import GpuPool, to_dev, log
    log("[gpu] fork equality")
    shape = Shape(32, 4, 64, 16, 1, 256)
    wl = synth.fork_workload("forkeq", 61, shape, prefix_len=1000, n_branches=1, branch_len=0)
    gp = GpuPool(shape)
    try:
        p = pkv.seq_allocate(gp.pool)
        k, v = wl.append_data(1, 1, 1000)
        pkv.kv_append(gp.pool, [p], 1000, to_dev(k), to_dev(v), gp.stream)
        c = pkv.seq_fork(gp.pool, p)
        q1 = to_dev(wl.decode_query(5, 1))
        q3 = torch.cat([q1, q1, q1])
        outs = []
        for seqs, q in (([p], q1), ([c], q1), ([p, c, p], q3)):
            o = torch.empty((len(seqs), 32, 64), device="cuda")
            pkv.paged_attn_decode(gp.pool, 0, seqs, q, 0.125, o, None, gp.stream)
            outs.append(o.cpu().numpy())
        assert np.array_equal(outs[0][0], outs[1][0])
        assert np.array_equal(outs[2][0], outs[2][1])
        assert np.array_equal(outs[2][0], outs[2][2])
    finally:
        gp.close()


def test_physical_placement_is_invisible(dev):
    """Same program, different free-list orders: bit-identical outputs."""
    from gpu_harness import run_gpu, log
    log("[gpu] placement invariance")
    wl = REDUCED["dendrite_small"]
    n = wl.shape.num_blocks
    a = run_gpu(wl, free_order=None)
    b = run_gpu(wl, free_order=np.random.default_rng(5).permutation(n).astype(np.int32))
    assert a.keys() == b.keys()
    for i in a:
        assert np.array_equal(a[i][0], b[i][0]) and np.array_equal(a[i][1], b[i][1])
