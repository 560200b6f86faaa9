"""Pins of the oracle's draft-tree commit (CPU only).

* Rebuild: after a commit, every sequence reads back (bit for bit) exactly
  the K/V of a sequence built from scratch by appending the context and then
  the accepted nodes' K/V in path order -- taken from the test's own copy of
  what was appended, not from the pool; decode over both is identical.
* Special cases: a chain tree accepted whole changes nothing; an empty path
  leaves the context; a full path of a branchy tree moves only off-path
  slots.
* A hand-derived trace of tables, refcounts, free list and copies.
* Shared tree blocks (a fork taken after the tree was appended): the commit
  copies the blocks it writes and the fork reads what it read before.
* Errors change nothing: a path that skips a parent link, an unknown
  sequence, a copy that would need a block this call released.
"""

import numpy as np
import pytest

import synth
from oracle import PoolModel, decode
from oracle.pool import ArgError, OOMError


def bits(rng, shape):
    return synth.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def invariants(pool):
    assert sum(pool.rc) == sum(len(t) for t in pool.tables.values())
    assert len(pool.fifo) + sum(1 for r in pool.rc if r > 0) == pool.N
    for s, t in pool.tables.items():
        n = pool.lens[s]
        assert len(t) == -(-n // pool.B)


def rebuild(pool_args, ctx_k, ctx_v, tree_k, tree_v, path):
    """A fresh pool holding context + accepted nodes, appended in order."""
    p = PoolModel(*pool_args)
    s = p.allocate()
    if ctx_k.shape[2]:
        p.append([s], ctx_k.shape[2], ctx_k, ctx_v)
    if path:
        p.append([s], len(path), tree_k[:, :, path], tree_v[:, :, path])
    return p, s


@pytest.mark.parametrize("B,ctx,T,depth,seed", [(1, 5, 7, 3, 1), (2, 9, 12, 4, 2), (4, 0, 16, 5, 3),
                                                (16, 37, 40, 6, 4), (4, 13, 64, 8, 5), (8, 16, 1, 1, 6)])
def test_commit_equals_a_rebuilt_sequence(B, ctx, T, depth, seed):
    rng = np.random.default_rng(seed)
    L, Hkv, D = 2, 2, 8
    args = (512, B, L, Hkv, D)
    pool = PoolModel(*args, free_order=rng.permutation(512))
    seqs = [pool.allocate() for _ in range(3)]
    ck, cv = bits(rng, (L, 3, ctx, Hkv, D)), bits(rng, (L, 3, ctx, Hkv, D))
    tk, tv = bits(rng, (L, 3, T, Hkv, D)), bits(rng, (L, 3, T, Hkv, D))
    if ctx:
        pool.append(seqs, ctx, ck, cv)
    pool.append(seqs, T, tk, tv)
    parents = np.stack([synth.draw_tree(rng, T, depth) for _ in seqs])
    wl = synth.Workload("t", 90 + seed, synth.Shape(4, Hkv, D, B, L, 512), [], 1.0)
    paths = wl.accept_paths(seed, parents)
    paths[0] = []                                   # one rejects everything
    pool.tree_commit(seqs, T, parents, paths)
    invariants(pool)
    q = bits(rng, (1, 4, D))
    for i, s in enumerate(seqs):
        fresh, f = rebuild(args, ck[:, i:i + 1], cv[:, i:i + 1], tk[:, i:i + 1], tv[:, i:i + 1], paths[i])
        assert pool.length(s) == ctx + len(paths[i])
        for layer in range(L):
            a, b = pool.gather_bits(s, layer), fresh.gather_bits(f, layer)
            assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
            if pool.length(s):
                oa, la = decode(pool, layer, [s], q, 0.3)
                ob, lb = decode(fresh, layer, [f], q, 0.3)
                assert np.array_equal(oa, ob) and np.array_equal(la, lb)


def test_chain_accepted_whole_changes_nothing():
    rng = np.random.default_rng(7)
    pool = PoolModel(32, 4, 1, 1, 4)
    s = pool.allocate()
    pool.append([s], 10, bits(rng, (1, 1, 10, 1, 4)), bits(rng, (1, 1, 10, 1, 4)))
    before = (pool.table(s), pool.length(s), pool.gather_bits(s, 0), list(pool.rc), pool.free_list())
    chain = np.arange(-1, 5, dtype=np.int32)
    cow = pool.tree_commit([s], 6, [chain], [list(range(6))])
    assert cow == []
    after = (pool.table(s), pool.length(s), pool.gather_bits(s, 0), list(pool.rc), pool.free_list())
    assert before[0] == after[0] and before[1] == after[1] and before[3:] == after[3:]
    assert np.array_equal(before[2][0], after[2][0])


def test_hand_trace():
    """B = 4, N = 8, identity free list.

    s = alloc; append 6 context tokens -> blocks [0, 1], len 6.
    Tree of 7 nodes appended: len 13, blocks [0, 1, 2, 3]; free [4..7].
    parent = [-1, 0, 0, 1, 1, 2, 4]; path [0, 1, 4, 6] (node 6 under 4).
    New length 6 + 4 = 10 -> 3 blocks: block 3 (positions 12..15) released
    -> free [4, 5, 6, 7, 3].  Moves: k=2 reads position 6+4=10, writes 8;
    k=3 reads 12, writes 9 (nodes 0, 1 stay where they are).  Block 2 is
    held once: written in place, no copy.
    t = fork(s) (rc 2 on blocks 0, 1, 2); a second 4-node chain tree is
    appended to t: position 10 in block 2 is shared -> append copies it to
    block 4 (slots 0..1), t = [0, 1, 4, 5], len 14; free [6, 7, 3].
    Commit t with path [0, 2]? Not a parent chain of a chain tree -> error.
    Commit t with path [0, 1] of parent [-1, 0, 1, 2]: nothing moves
    (positions 10, 11 keep nodes 0, 1); new length 12 -> block 5 released;
    free [6, 7, 3, 5].
    """
    pool = PoolModel(8, 4)
    s = pool.allocate()
    pool.append([s], 6)
    pool.append([s], 7)
    assert pool.table(s) == [0, 1, 2, 3] and pool.free_list() == [4, 5, 6, 7]
    par = [-1, 0, 0, 1, 1, 2, 4]
    assert pool.tree_commit([s], 7, [par], [[0, 1, 4, 6]]) == []
    assert pool.table(s) == [0, 1, 2] and pool.length(s) == 10
    assert pool.free_list() == [4, 5, 6, 7, 3]
    t = pool.fork(s)
    _, cow = pool.append([t], 4)
    assert cow == [(2, 4, 2)] and pool.table(t) == [0, 1, 4, 5] and pool.length(t) == 14
    assert pool.free_list() == [6, 7, 3]
    with pytest.raises(ArgError):
        pool.tree_commit([t], 4, [[-1, 0, 1, 2]], [[0, 2]])
    assert pool.table(t) == [0, 1, 4, 5] and pool.free_list() == [6, 7, 3]
    assert pool.tree_commit([t], 4, [[-1, 0, 1, 2]], [[0, 1]]) == []
    assert pool.table(t) == [0, 1, 4] and pool.length(t) == 12
    assert pool.free_list() == [6, 7, 3, 5]
    assert pool.rc[:6] == [2, 2, 1, 0, 1, 0]
    invariants(pool)


def test_shared_tree_blocks_are_copied_before_writing():
    rng = np.random.default_rng(8)
    L, Hkv, D, B = 1, 1, 4, 4
    pool = PoolModel(32, B, L, Hkv, D)
    s = pool.allocate()
    pool.append([s], 5, bits(rng, (L, 1, 5, Hkv, D)), bits(rng, (L, 1, 5, Hkv, D)))
    pool.append([s], 8, bits(rng, (L, 1, 8, Hkv, D)), bits(rng, (L, 1, 8, Hkv, D)))
    f = pool.fork(s)                          # shares every tree block
    ref = pool.gather_bits(f, 0)
    par = [-1, 0, 0, 2, 3, 3, 5, 6]
    cow = pool.tree_commit([s], 8, [par], [[0, 2, 3, 5, 6]])
    # writes land at positions 6, 7, 8, 9 (blocks 1 and 2): both copied
    assert [(c[0], c[2]) for c in cow] == [(pool.table(f)[1], 4), (pool.table(f)[2], 2)]
    got = pool.gather_bits(f, 0)
    assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])
    invariants(pool)


def test_commit_of_two_sequences_sharing_a_tree():
    """Both the fork and its parent commit, in one call, different paths of
    the tree they share: each equals its own rebuild."""
    rng = np.random.default_rng(9)
    L, Hkv, D, B = 1, 1, 4, 2
    args = (64, B, L, Hkv, D)
    pool = PoolModel(*args)
    ck, cv = bits(rng, (L, 1, 3, Hkv, D)), bits(rng, (L, 1, 3, Hkv, D))
    tk, tv = bits(rng, (L, 1, 9, Hkv, D)), bits(rng, (L, 1, 9, Hkv, D))
    s = pool.allocate()
    pool.append([s], 3, ck, cv)
    pool.append([s], 9, tk, tv)
    f = pool.fork(s)
    par = [-1, 0, 0, 1, 2, 3, 4, 5, 6]
    paths = [[0, 2, 4, 6, 8], [0, 1, 3, 5, 7]]
    pool.tree_commit([f, s], 9, [par, par], paths)
    for sid, path in zip([f, s], paths):
        fresh, g = rebuild(args, ck, cv, tk, tv, path)
        a, b = pool.gather_bits(sid, 0), fresh.gather_bits(g, 0)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    invariants(pool)


def test_errors_change_nothing():
    pool = PoolModel(6, 2)
    s = pool.allocate()
    pool.append([s], 2)
    pool.append([s], 4)                 # s = [0, 1, 2]: 2 context tokens + 4 tree nodes
    t = pool.allocate()
    pool.append([t], 2)
    pool.append([t], 4)                 # t = [3, 4, 5]
    u = pool.fork(t)                    # t's blocks shared; the pool is full
    snap = pool.snapshot()
    par = [-1, 0, 0, 2]
    with pytest.raises(ArgError):
        pool.tree_commit([s], 4, [par], [[2, 3]])       # does not start at the root
    with pytest.raises(ArgError):
        pool.tree_commit([s], 4, [par], [[0, 1, 3]])    # 3 is not a child of 1
    with pytest.raises(ArgError):
        pool.tree_commit([s, s], 4, [par, par], [[0], [0]])
    with pytest.raises(ArgError):
        pool.tree_commit([s], 7, [par + [3, 4, 5]], [[0]])
    # s keeps only its root (block 2 is released); t writes position 3 into
    # block 4, which u shares: its copy may not take block 2, which still
    # holds tokens of this call, and no other block is free
    with pytest.raises(OOMError):
        pool.tree_commit([s, t], 4, [par, par], [[0], [0, 2]])
    assert pool.snapshot() == snap
    assert u in pool.tables
