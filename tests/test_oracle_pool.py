"""Pins of the oracle's block-pool model (CPU only).

* the hand-derived trace in tests/golden (rules from the Dendrite, Trellis
  and SGLang pages, worked out by hand);
* structural invariants after every op of random programs;
* transactional errors;
* block counts the workload definitions fix in closed form, and the
  shared-prefix rule and memory figure the pages print.
"""

import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import synth
from oracle import PoolModel, OOMError, SeqError, ArgError, run_program
from trace_format import parse_trace, check_expectations


def run_trace_on_model(steps, B=4, N=8):
    pool = PoolModel(N, B, num_layers=1, num_kv_heads=1, head_dim=1)
    names = {}
    for op, expect in steps:
        slots = cow = None
        if op[0] == "alloc":
            names[op[1]] = pool.allocate()
        elif op[0] == "fork":
            names[op[2]] = pool.fork(names[op[1]])
        elif op[0] == "free":
            pool.free(names.pop(op[1]))
        elif op[0] == "append":
            sl, cw = pool.append([names[op[1]]], int(op[2]))
            slots, cow = sl[0], cw
        check_expectations(
            expect, table=lambda n: pool.table(names[n]),
            length=lambda n: pool.length(names[n]), live=list(names),
            rc_all=pool.rc, fifo=pool.free_list(), slots=slots, cow=cow,
            label=" ".join(op))
    return pool, names


def test_hand_trace():
    steps = parse_trace("pool_trace_b4_n8.txt")
    assert len(steps) == 10
    pool, names = run_trace_on_model(steps)
    assert pool.table(names["s2"]) == [0, 2, 4]


def test_hand_trace_cow_moves_the_right_data():
    """Copy-on-write copies only the shared filled slots; the writer's new
    token lands in the copy and the original keeps its own data."""
    pool = PoolModel(8, 4, num_layers=1, num_kv_heads=1, head_dim=2)

    def data(vals):
        a = np.array(vals, dtype=np.uint16).reshape(1, 1, len(vals), 1, 1)
        return np.repeat(a, 2, axis=-1), np.repeat(a + 100, 2, axis=-1)

    s0 = pool.allocate()
    pool.append([s0], 6, *data([10, 11, 12, 13, 14, 15]))
    s1 = pool.fork(s0)
    pool.append([s1], 1, *data([20]))
    pool.append([s0], 1, *data([16]))
    k1, _ = pool.gather_bits(s1, 0)
    k0, v0 = pool.gather_bits(s0, 0)
    assert k1[:, 0, 0].tolist() == [10, 11, 12, 13, 14, 15, 20]
    assert k0[:, 0, 0].tolist() == [10, 11, 12, 13, 14, 15, 16]
    assert v0[:, 0, 0].tolist() == [110, 111, 112, 113, 114, 115, 116]
    # block 2 is s1's copy of block 1: slots 0..1 copied, slot 2 its own token
    assert pool.kbits[2, :3, 0, 0, 0].tolist() == [14, 15, 20]
    assert pool.kbits[1, :3, 0, 0, 0].tolist() == [14, 15, 16]


# ---------------------------------------------------------------- invariants

def check_invariants(pool):
    live_refs = sum(len(t) for t in pool.tables.values())
    assert sum(pool.rc) == live_refs
    held = {b for b, c in enumerate(pool.rc) if c > 0}
    assert len(pool.fifo) + len(held) == pool.N
    assert not held & set(pool.fifo)
    assert len(set(pool.fifo)) == len(pool.fifo)
    for sid, t in pool.tables.items():
        n = pool.lens[sid]
        if n == 0:
            assert t == []
        else:
            assert (len(t) - 1) * pool.B < n <= len(t) * pool.B
        for b in t:
            assert pool.rc[b] >= 1


ops_strategy = st.lists(
    st.tuples(st.sampled_from(["alloc", "fork", "free", "append", "append2"]),
              st.integers(0, 7), st.integers(0, 7), st.integers(0, 9)),
    min_size=1, max_size=40)


@settings(max_examples=300, deadline=None)
@given(ops=ops_strategy, B=st.sampled_from([1, 2, 4]), N=st.integers(1, 12),
       seed=st.integers(0, 2**16))
def test_random_programs_keep_invariants_and_contents(ops, B, N, seed):
    """After every op: refcount/free-list invariants hold, every live
    sequence reads back exactly the tokens appended to it (in order), and
    a failing op changes nothing."""
    rng = np.random.default_rng(seed)
    order = rng.permutation(N)
    pool = PoolModel(N, B, num_layers=1, num_kv_heads=1, head_dim=1,
                     free_order=order)
    logical = {}        # sid -> list of token values, kept independently
    counter = [1]
    for kind, a, b, n in ops:
        live = sorted(logical)
        before = pool.snapshot()
        try:
            if kind == "alloc":
                sid = pool.allocate()
                logical[sid] = []
            elif kind == "fork" and live:
                p = live[a % len(live)]
                sid = pool.fork(p)
                logical[sid] = list(logical[p])
            elif kind == "free" and live:
                s = live[a % len(live)]
                pool.free(s)
                del logical[s]
            elif kind in ("append", "append2") and live:
                seqs = [live[a % len(live)]]
                if kind == "append2" and len(live) > 1:
                    other = live[b % len(live)]
                    if other != seqs[0]:
                        seqs.append(other)
                vals = np.arange(counter[0], counter[0] + len(seqs) * n,
                                 dtype=np.uint16).reshape(1, len(seqs), n, 1, 1)
                counter[0] += len(seqs) * n
                pool.append(seqs, n, vals, vals + 1)
                for i, s in enumerate(seqs):
                    logical[s] += vals[0, i, :, 0, 0].tolist()
        except OOMError:
            assert pool.snapshot() == before
        check_invariants(pool)
        for s, toks in logical.items():
            k, v = pool.gather_bits(s, 0)
            assert k[:, 0, 0].tolist() == toks
            assert (v[:, 0, 0].astype(int) - 1).tolist() == toks


def test_errors_are_transactional():
    pool = PoolModel(3, 2)
    s = pool.allocate()
    pool.append([s], 3)
    t = pool.fork(s)
    before = pool.snapshot()
    # t needs a CoW copy (1 block) + 2 new blocks for 4 more tokens: 3 > 1 free
    with pytest.raises(OOMError):
        pool.append([t], 4)
    assert pool.snapshot() == before
    with pytest.raises(ArgError):
        pool.append([s, s], 1)
    with pytest.raises(SeqError):
        pool.append([s, 99], 1)
    with pytest.raises(SeqError):
        pool.fork(99)
    with pytest.raises(SeqError):
        pool.free(99)
    assert pool.snapshot() == before
    # a multi-sequence append that fits for the first sequence but not the
    # second must not apply the first either
    u = pool.allocate()
    before = pool.snapshot()
    with pytest.raises(OOMError):
        pool.append([t, u], 2)
    assert pool.snapshot() == before


def test_fork_moves_no_data_and_takes_no_blocks():
    pool = PoolModel(16, 4)
    s = pool.allocate()
    pool.append([s], 10)
    fifo = pool.free_list()
    c = pool.fork(s)
    assert pool.free_list() == fifo
    assert pool.table(c) == pool.table(s)
    assert all(pool.rc[b] == 2 for b in pool.table(s))


# --------------------------------------------------- numbers the pages fix

def unique_blocks(pool):
    return sum(1 for c in pool.rc if c > 0)


def final_pool(wl):
    last = None
    for _, _, pool, handles, _ in run_program(wl, store_data=False):
        last = (pool, handles)
    return last


def test_trellis_shared_prefix_blocks():
    """Trellis benchmark definitions: the shared region is
    round(phi * L / 32) whole 32-token blocks -> 8 blocks at L = 512,
    phi = 0.5, and every session acquires them instead of allocating."""
    wl = synth.named("c2_trellis")
    assert wl.meta["shared_blocks"] == 8 == round(0.5 * 512 / 32)
    pool, handles = final_pool(wl)
    shared = pool.table(handles[0])
    assert len(shared) == 8
    for h in range(1, 17):
        t = pool.table(handles[h])
        assert t[:8] == shared
        assert len(set(t[8:]) & set(shared)) == 0
        assert pool.length(handles[h]) == 512 + 64
    assert all(pool.rc[b] == 17 for b in shared)
    # 8 shared + 16 sessions x (8 prompt blocks + 2 blocks of decoded tokens)
    assert unique_blocks(pool) == 8 + 16 * (8 + 2) == 168


def test_dendrite_memory_figure():
    """Dendrite evidence: a 4K prefix with 6 branches takes 1.1 GB against
    6 GB when every branch holds a full copy (a saving of about 80 % or
    more).  With 16-token blocks and 80 own tokens per branch, unique pool
    blocks over per-branch blocks must land on 1.1 / 6."""
    shape = synth.Shape(8, 2, 64, 16, 1, 512)
    wl = synth.fork_workload("dendrite_mem", 90, shape, prefix_len=4096,
                             n_branches=6, branch_len=80, decode_steps=0)
    pool, handles = final_pool(wl)
    unique = unique_blocks(pool)
    logical = sum(len(pool.table(handles[h])) for h in range(1, 7))
    assert unique == 4096 // 16 + 6 * 5
    assert logical == 6 * (4096 // 16 + 5)
    assert abs(unique / logical - 1.1 / 6) < 0.005
    assert 1 - unique / logical >= 0.8


@pytest.mark.parametrize("name,unique,cows", [
    ("c1_tiny_fork", 128 // 16 + 4 * 1, 0),
    ("c3_dendrite", 4104 // 16 + 1 + 6 * 25, 6),
    ("c3_dendrite_aligned", 4096 // 16 + 6 * 24, 0),
    ("c4_mcts", 2048 // 16 + 4 * 4 + 16 * 4 + 64 * 4 + 256 * 4, 0),
    ("c5_verify", 8 * (2048 // 16 + 64 // 16), 0),
    ("c2_trellis_prefill", 256 // 32 + 16 * (256 // 32), 0),
])
def test_workload_block_counts(name, unique, cows):
    """Closed-form block counts of each workload's construction.  The
    half-filled shared block of the 4104-token prefix is copied once by each
    of the 6 branches on their first append."""
    wl = synth.named(name)
    s = wl.shape
    model = PoolModel(s.num_blocks, s.block_size, free_order=wl.free_order())
    hmap = {}
    n_cow = 0
    for op in wl.ops:
        if op[0] == "alloc":
            hmap[op[1]] = model.allocate()
        elif op[0] == "fork":
            hmap[op[2]] = model.fork(hmap[op[1]])
        elif op[0] == "append":
            _, cw = model.append([hmap[h] for h in op[1]], op[2])
            n_cow += len(cw)
    assert unique_blocks(model) == unique
    assert n_cow == cows


def test_c5_trees_have_depth_six():
    wl = synth.named("c5_verify")
    op = [o for o in wl.ops if o[0] == "verify"][0]
    parents = wl.tree_parents(op[4], 8, 64)
    for p in parents:
        depth = [1] * 64
        for i in range(1, 64):
            assert 0 <= p[i] < i
            depth[i] = depth[p[i]] + 1
        assert max(depth) == 6
        assert p[0] == -1
