"""Pins of the oracle's attention (CPU only).

Each pin is something other than the oracle itself:
* closed forms (one key, equal keys, equal values, zero query);
* a library routine: ``torch.nn.functional.scaled_dot_product_attention`` in
  float64 on the CPU (``enable_gqa`` for the head grouping) and
  ``torch.logsumexp`` for the log-sum-exp, run on the test's own contiguous
  copy of each sequence, with tree masks built by boolean transitive closure
  of the parent matrix (not by walking parents);
* invariants the pages imply: a forked child reads what its parent reads,
  physical block ids do not matter, paged equals contiguous, a chain tree is
  causal attention, a tree node equals a decode along its root path;
* brute-force enumeration of every block placement on tiny pools.
"""

import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import synth
from oracle import (PoolModel, attend, bf16_bits_to_f64, decode, prefill, tree_verify,
                    tree_key_positions, run_program, ArgError, EmptyError)


def rand_bits(rng, shape, scale=1.0):
    return synth.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(scale))


def t64(bits):
    return torch.from_numpy(bf16_bits_to_f64(bits))


def sdpa(q_bits, k_bits, v_bits, scale, mask=None):
    """Library attention: q [R][Hq][D], k/v [n][Hkv][D] -> out [R][Hq][D], lse [R][Hq]."""
    q = t64(q_bits).permute(1, 0, 2)[None]          # [1][Hq][R][D]
    k = t64(k_bits).permute(1, 0, 2)[None]
    v = t64(v_bits).permute(1, 0, 2)[None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    out = F.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=scale,
                                         enable_gqa=True)[0].permute(1, 0, 2)
    g = q.shape[1] // k.shape[1]
    kk = k.repeat_interleave(g, dim=1)
    z = scale * (q @ kk.transpose(-1, -2))
    if m is not None:
        z = z.masked_fill(~m, float("-inf"))
    lse = torch.logsumexp(z, dim=-1)[0].permute(1, 0)
    return out.numpy(), lse.numpy()


# ------------------------------------------------------------ closed forms

def test_single_key_returns_v_exactly():
    rng = np.random.default_rng(1)
    q = bf16_bits_to_f64(rand_bits(rng, (4, 64)))
    k = bf16_bits_to_f64(rand_bits(rng, (1, 64)))
    v = bf16_bits_to_f64(rand_bits(rng, (1, 64)))
    out, lse = attend(q, k, v, 0.125)
    assert np.array_equal(out, np.repeat(v, 4, axis=0))
    for r in range(4):
        z = 0.125 * math.fsum(q[r] * k[0])
        assert abs(lse[r] - z) <= 1e-13 * max(1.0, abs(z))


def test_equal_keys_give_mean_of_values():
    rng = np.random.default_rng(2)
    q = bf16_bits_to_f64(rand_bits(rng, (3, 32)))
    k = np.repeat(bf16_bits_to_f64(rand_bits(rng, (1, 32))), 37, axis=0)
    v = bf16_bits_to_f64(rand_bits(rng, (37, 32)))
    out, lse = attend(q, k, v, 0.3)
    assert np.allclose(out, v.mean(axis=0)[None], rtol=0, atol=1e-13)
    z = 0.3 * np.array([math.fsum(q[r] * k[0]) for r in range(3)])
    assert np.allclose(lse, z + math.log(37), rtol=0, atol=1e-12)


def test_equal_values_give_that_value():
    rng = np.random.default_rng(3)
    q = bf16_bits_to_f64(rand_bits(rng, (5, 16)))
    k = bf16_bits_to_f64(rand_bits(rng, (50, 16), 3.0))
    v = np.repeat(bf16_bits_to_f64(rand_bits(rng, (1, 16))), 50, axis=0)
    out, _ = attend(q, k, v, 1.0)
    assert np.allclose(out, v[:5], rtol=0, atol=1e-13)


def test_zero_query_gives_mean_and_log_length():
    rng = np.random.default_rng(4)
    k = bf16_bits_to_f64(rand_bits(rng, (29, 64)))
    v = bf16_bits_to_f64(rand_bits(rng, (29, 64)))
    out, lse = attend(np.zeros((2, 64)), k, v, 0.125)
    assert np.allclose(out, v.mean(axis=0)[None], rtol=0, atol=1e-13)
    assert np.allclose(lse, math.log(29), rtol=0, atol=1e-14)


def test_empty_key_set_is_an_error():
    with pytest.raises(EmptyError):
        attend(np.zeros((1, 4)), np.zeros((0, 4)), np.zeros((0, 4)), 1.0)
    pool = PoolModel(4, 2, 1, 1, 4)
    s = pool.allocate()
    with pytest.raises(EmptyError):
        decode(pool, 0, [s], np.zeros((1, 1, 4), np.uint16), 1.0)


# ------------------------------------------------- library routine (SDPA)

class Tracked:
    """A pool plus the test's own contiguous copy of every sequence."""

    def __init__(self, N, B, L, Hkv, D, free_order=None):
        self.pool = PoolModel(N, B, L, Hkv, D, free_order=free_order)
        self.L, self.Hkv, self.D = L, Hkv, D
        self.data = {}

    def alloc(self):
        s = self.pool.allocate()
        self.data[s] = (np.zeros((self.L, 0, self.Hkv, self.D), np.uint16),) * 2
        return s

    def fork(self, p):
        s = self.pool.fork(p)
        self.data[s] = self.data[p]
        return s

    def append(self, seqs, n, rng, kscale=1.0):
        k = rand_bits(rng, (self.L, len(seqs), n, self.Hkv, self.D), kscale)
        v = rand_bits(rng, (self.L, len(seqs), n, self.Hkv, self.D))
        self.pool.append(seqs, n, k, v)
        for i, s in enumerate(seqs):
            ok, ov = self.data[s]
            self.data[s] = (np.concatenate([ok, k[:, i]], axis=1),
                            np.concatenate([ov, v[:, i]], axis=1))
        return k, v


@pytest.mark.parametrize("hq,hkv,d,B", [(8, 2, 64, 16), (32, 4, 64, 32),
                                        (32, 8, 128, 16), (4, 4, 16, 4),
                                        (6, 1, 8, 1)])
def test_decode_matches_library_attention(hq, hkv, d, B):
    rng = np.random.default_rng(hq * 1000 + d + B)
    N = 128
    tp = Tracked(N, B, 2, hkv, d, free_order=rng.permutation(N))
    root = tp.alloc()
    tp.append([root], 37, rng)
    kids = [tp.fork(root) for _ in range(3)]
    tp.append(kids, 5, rng)
    extra = tp.fork(kids[1])
    tp.append([extra, kids[0]], 11, rng)
    seqs = [root] + kids + [extra]
    for layer in range(2):
        q = rand_bits(rng, (len(seqs), hq, d))
        out, lse = decode(tp.pool, layer, seqs, q, 1 / math.sqrt(d))
        for i, s in enumerate(seqs):
            k, v = tp.data[s]
            ro, rl = sdpa(q[i:i + 1], k[layer], v[layer], 1 / math.sqrt(d))
            assert np.allclose(out[i], ro[0], rtol=0, atol=1e-12)
            assert np.allclose(lse[i], rl[0], rtol=0, atol=1e-12)


def closure_mask(parent, ctx):
    """Attention mask of a draft tree from the reachability matrix.

    A[i][j] = 1 when j is the parent of i; (I + A)^(T) > 0 marks every
    ancestor-or-self pair.  Context columns are all visible.
    """
    t = len(parent)
    a = np.zeros((t, t), dtype=np.int64)
    for i in range(1, t):
        a[i, parent[i]] = 1
    reach = np.eye(t, dtype=np.int64)
    step = np.eye(t, dtype=np.int64) + a
    for _ in range(t):
        reach = np.minimum(reach @ step, 1)
    mask = np.ones((t, ctx + t), dtype=bool)
    mask[:, ctx:] = reach > 0
    return mask


@pytest.mark.parametrize("ctx,T,depth", [(40, 9, 4), (0, 7, 3), (130, 16, 6), (5, 1, 1)])
def test_tree_verify_matches_library_attention(ctx, T, depth):
    rng = np.random.default_rng(ctx * 7 + T)
    hq, hkv, d, B = 8, 2, 32, 16
    tp = Tracked(64, B, 1, hkv, d, free_order=rng.permutation(64))
    seqs = [tp.alloc() for _ in range(3)]
    if ctx:
        tp.append(seqs, ctx, rng)
    tp.append(seqs, T, rng)
    parents = np.stack([synth.draw_tree(rng, T, depth) for _ in seqs])
    q = rand_bits(rng, (3, T, hq, d))
    out, lse = tree_verify(tp.pool, 0, seqs, parents, q, 0.2)
    for i, s in enumerate(seqs):
        k, v = tp.data[s]
        mask = closure_mask(parents[i], ctx)
        ro, rl = sdpa(q[i], k[0], v[0], 0.2, mask)
        assert np.allclose(out[i], ro, rtol=0, atol=1e-12)
        assert np.allclose(lse[i], rl, rtol=0, atol=1e-12)


def test_chain_tree_is_causal_attention():
    rng = np.random.default_rng(11)
    ctx, T = 23, 12
    tp = Tracked(32, 4, 1, 2, 16)
    s = tp.alloc()
    tp.append([s], ctx + T, rng)
    parent = np.arange(-1, T - 1, dtype=np.int32)[None]
    q = rand_bits(rng, (1, T, 4, 16))
    out, lse = tree_verify(tp.pool, 0, [s], parent, q, 0.25)
    causal = np.tril(np.ones((T, ctx + T), dtype=bool), k=ctx)
    k, v = tp.data[s]
    ro, rl = sdpa(q[0], k[0], v[0], 0.25, causal)
    assert np.allclose(out[0], ro, rtol=0, atol=1e-12)
    assert np.allclose(lse[0], rl, rtol=0, atol=1e-12)


def test_key_positions_of_a_small_tree():
    #      0
    #     / \
    #    1   2
    #   /     \
    #  3       4
    parent = [-1, 0, 0, 1, 2]
    assert tree_key_positions(parent, 0, 3) == [0, 1, 2, 3]
    assert tree_key_positions(parent, 3, 3) == [0, 1, 2, 3, 4, 6]
    assert tree_key_positions(parent, 4, 0) == [0, 2, 4]


# ------------------------------------------------------------ invariants

def test_single_node_tree_equals_decode():
    rng = np.random.default_rng(12)
    tp = Tracked(32, 8, 1, 2, 32)
    s = tp.alloc()
    tp.append([s], 45, rng)
    q = rand_bits(rng, (1, 1, 8, 32))
    out_t, lse_t = tree_verify(tp.pool, 0, [s], np.array([[-1]]), q, 0.17)
    out_d, lse_d = decode(tp.pool, 0, [s], q[:, 0], 0.17)
    assert np.array_equal(out_t[:, 0], out_d) and np.array_equal(lse_t[:, 0], lse_d)


def test_tree_node_equals_decode_along_its_path():
    """Cross-check of the tree mask with the pool: node i's output equals a
    plain decode on a sequence forked from the context that appends the
    root..i path tokens in order."""
    rng = np.random.default_rng(13)
    ctx, T = 33, 10
    B, hkv, d, hq = 4, 2, 16, 4
    tp = Tracked(128, B, 1, hkv, d)
    s = tp.alloc()
    tp.append([s], ctx, rng)
    base = tp.fork(s)
    k_tree, v_tree = tp.append([s], T, rng)
    parent = synth.draw_tree(rng, T, 4)
    q = rand_bits(rng, (1, T, hq, d))
    out, lse = tree_verify(tp.pool, 0, [s], parent[None], q, 0.3)
    for i in range(T):
        path = []
        j = i
        while j != -1:
            path.append(j)
            j = parent[j]
        path.reverse()
        br = tp.pool.fork(base)
        kk = k_tree[:, :, path]
        vv = v_tree[:, :, path]
        tp.pool.append([br], len(path), kk, vv)
        od, ld = decode(tp.pool, 0, [br], q[:, i], 0.3)
        assert np.allclose(out[0, i], od[0], rtol=0, atol=1e-13)
        assert np.allclose(lse[0, i], ld[0], rtol=0, atol=1e-13)
        tp.pool.free(br)


def test_forked_child_equals_parent_until_it_diverges():
    rng = np.random.default_rng(14)
    tp = Tracked(64, 16, 1, 2, 64)
    p = tp.alloc()
    tp.append([p], 100, rng)
    c = tp.fork(p)
    q = rand_bits(rng, (1, 8, 64))
    op, lp = decode(tp.pool, 0, [p], q, 0.125)
    oc, lc = decode(tp.pool, 0, [c], q, 0.125)
    assert np.array_equal(op, oc) and np.array_equal(lp, lc)
    tp.append([c], 1, rng)
    oc2, _ = decode(tp.pool, 0, [c], q, 0.125)
    assert not np.array_equal(op, oc2)
    op2, _ = decode(tp.pool, 0, [p], q, 0.125)
    assert np.array_equal(op, op2)     # the parent is untouched by the child's write


def test_physical_placement_does_not_matter():
    """Same program, different free-list orders: identical outputs."""
    wl = synth.named("c1_tiny_fork")
    ref = None
    for seed in range(4):
        order = np.random.default_rng(100 + seed).permutation(wl.shape.num_blocks)
        outs = [r for *_, r in run_program(wl, free_order=order) if r is not None]
        if ref is None:
            ref = outs
        else:
            for (o1, l1), (o2, l2) in zip(ref, outs):
                assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_lse_merge_identity():
    """Softmax states over disjoint key sets merge by log-sum-exp into the
    state over their union."""
    rng = np.random.default_rng(15)
    q = bf16_bits_to_f64(rand_bits(rng, (6, 64)))
    k = bf16_bits_to_f64(rand_bits(rng, (300, 64)))
    v = bf16_bits_to_f64(rand_bits(rng, (300, 64)))
    full, lf = attend(q, k, v, 0.125)
    cuts = [0, 17, 130, 131, 300]
    parts = [attend(q, k[a:b], v[a:b], 0.125) for a, b in zip(cuts, cuts[1:])]
    m = np.max([l for _, l in parts], axis=0)
    w = [np.exp(l - m) for _, l in parts]
    tot = np.sum(w, axis=0)
    merged = sum(o * wi[:, None] for (o, _), wi in zip(parts, w)) / tot[:, None]
    assert np.allclose(merged, full, rtol=0, atol=1e-13)
    assert np.allclose(m + np.log(tot), lf, rtol=0, atol=1e-13)


# ------------------------------------------------------------ brute force

@pytest.mark.parametrize("B", [2, 16])
def test_brute_force_tiny_pools(B):
    """Pool of 4 blocks, at most 2 logical blocks per sequence: every
    placement (all 24 free-list orders, covering the 12 injective placements
    of 2 logical blocks), every length 1..2B, every fork point, both append
    orders of two branches.  Every output must equal the library attention
    on the contiguous data, and placements must agree bit for bit."""
    rng = np.random.default_rng(B)
    hkv, hq, d = 1, 2, 8
    total = 2 * B
    k_all = rand_bits(rng, (1, 2, total, hkv, d))
    v_all = rand_bits(rng, (1, 2, total, hkv, d))
    q = rand_bits(rng, (2, hq, d))
    lib = {}
    lens = range(1, total + 1) if B == 2 else [1, B - 1, B, B + 1, total]
    for n in lens:
        forks = range(0, n + 1) if B == 2 else [0, n // 2, n]
        for f in forks:
            for order_first in (0, 1):
                key = (n, f, order_first)
                results = []
                for perm in itertools.permutations(range(4)):
                    pool = PoolModel(4, B, 1, hkv, d, free_order=perm)
                    p = pool.allocate()
                    if f:
                        pool.append([p], f, k_all[:, :1, :f], v_all[:, :1, :f])
                    c = pool.fork(p)
                    rest = n - f
                    # branch 0 = parent continues with row 0, branch 1 = child with row 1
                    conts = [(p, 0), (c, 1)]
                    if order_first:
                        conts.reverse()
                    try:
                        for s, row in conts:
                            if rest:
                                pool.append([s], rest, k_all[:, row:row + 1, f:n],
                                            v_all[:, row:row + 1, f:n])
                    except Exception:
                        results.append(None)
                        continue
                    out, lse = decode(pool, 0, [p, c], q, 0.5)
                    results.append((out, lse))
                ok = [r for r in results if r is not None]
                assert ok, key
                for r in ok[1:]:
                    assert np.array_equal(r[0], ok[0][0]) and np.array_equal(r[1], ok[0][1])
                for i, row in enumerate((0, 1)):
                    kk = np.concatenate([k_all[0, 0, :f], k_all[0, row, f:n]])
                    vv = np.concatenate([v_all[0, 0, :f], v_all[0, row, f:n]])
                    if key not in lib:
                        lib[key] = {}
                    ro, rl = sdpa(q[i:i + 1], kk, vv, 0.5)
                    assert np.allclose(ok[0][0][i], ro[0], rtol=0, atol=1e-13)
                    assert np.allclose(ok[0][1][i], rl[0], rtol=0, atol=1e-13)


# ------------------------------------------------------------ causal prefill

def sdpa_causal(q_bits, k_bits, v_bits, scale):
    """Library causal attention over a whole sequence: q/k/v [n][H][D], query
    i sees keys 0..i (``is_causal``); lse by ``torch.logsumexp`` over a
    ``tril`` of ones."""
    q = t64(q_bits).permute(1, 0, 2)[None]
    k = t64(k_bits).permute(1, 0, 2)[None]
    v = t64(v_bits).permute(1, 0, 2)[None]
    out = F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=scale,
                                         enable_gqa=True)[0].permute(1, 0, 2)
    g = q.shape[1] // k.shape[1]
    z = scale * (q @ k.repeat_interleave(g, dim=1).transpose(-1, -2))
    n = z.shape[-1]
    keep = torch.ones(n, n, dtype=torch.bool).tril()
    lse = torch.logsumexp(z.masked_fill(~keep, float("-inf")), dim=-1)[0].permute(1, 0)
    return out.numpy(), lse.numpy()


@pytest.mark.parametrize("hq,hkv,d,B", [(8, 2, 64, 16), (32, 4, 64, 32), (6, 1, 8, 1),
                                        (4, 4, 16, 4)])
def test_prefill_matches_library_causal_attention(hq, hkv, d, B):
    """The new tokens' rows equal the last rows of the library's causal
    attention over the whole sequence (the earlier rows get queries of their
    own, which the prefill does not compute).  Covers a shared prefix, ragged
    counts, a count of 0 and a whole sequence new."""
    rng = np.random.default_rng(hq * 100 + d + B)
    tp = Tracked(256, B, 2, hkv, d, free_order=rng.permutation(256))
    root = tp.alloc()
    tp.append([root], 29, rng)
    kids = [tp.fork(root) for _ in range(3)]
    tp.append(kids, 7, rng)
    tp.append([kids[0]], 66, rng)
    tp.append([kids[2]], 1, rng)
    seqs = kids + [root]
    n_new = [66 + 7, 0, 8, 29]       # kids[0]: 73 new; root: all of it new
    lens = [29 + 7 + 66, 29 + 7, 29 + 7 + 1, 29]
    for layer in range(2):
        q_new = rand_bits(rng, (sum(n_new), hq, d))
        out, lse = prefill(tp.pool, layer, seqs, n_new, q_new, 1 / math.sqrt(d))
        row = 0
        for s_, n, ln in zip(seqs, n_new, lens):
            k, v = tp.data[s_]
            assert k.shape[1] == ln
            q_all = np.concatenate([rand_bits(rng, (ln - n, hq, d)), q_new[row:row + n]])
            ro, rl = sdpa_causal(q_all, k[layer], v[layer], 1 / math.sqrt(d))
            assert np.allclose(out[row:row + n], ro[ln - n:], rtol=0, atol=1e-12)
            assert np.allclose(lse[row:row + n], rl[ln - n:], rtol=0, atol=1e-12)
            row += n


def test_prefill_query_equals_decode_on_the_prefix_it_sees():
    """Query j of the new tokens reads what a decode reads on a sequence
    holding only the first len - n + j + 1 tokens (built by appending exactly
    those tokens to a fresh pool)."""
    rng = np.random.default_rng(21)
    B, hkv, d, hq = 4, 2, 16, 4
    tp = Tracked(64, B, 1, hkv, d)
    s = tp.alloc()
    tp.append([s], 13, rng)
    tp.append([s], 9, rng)
    k, v = tp.data[s]
    q = rand_bits(rng, (9, hq, d))
    out, lse = prefill(tp.pool, 0, [s], [9], q, 0.4)
    for j in range(9):
        solo = PoolModel(64, B, 1, hkv, d)
        t = solo.allocate()
        n = 13 + j + 1
        solo.append([t], n, k[:, None, :n], v[:, None, :n])
        od, ld = decode(solo, 0, [t], q[j:j + 1], 0.4)
        assert np.array_equal(out[j], od[0]) and np.array_equal(lse[j], ld[0])


def test_prefill_equals_chain_tree_verify():
    """A chain-shaped draft tree is causal attention over its tokens."""
    rng = np.random.default_rng(22)
    tp = Tracked(64, 8, 1, 2, 32)
    seqs = [tp.alloc() for _ in range(2)]
    tp.append(seqs, 19, rng)
    tp.append(seqs, 11, rng)
    q = rand_bits(rng, (2, 11, 8, 32))
    chain = np.tile(np.arange(-1, 10, dtype=np.int32), (2, 1))
    out_t, lse_t = tree_verify(tp.pool, 0, seqs, chain, q, 0.3)
    out_p, lse_p = prefill(tp.pool, 0, seqs, [11, 11], q.reshape(22, 8, 32), 0.3)
    assert np.array_equal(out_t.reshape(22, 8, 32), out_p)
    assert np.array_equal(lse_t.reshape(22, 8), lse_p)


def test_prefill_zero_query_gives_running_means():
    """q = 0: every visible key weighs the same, so query j's output is the
    mean of V over tokens 0..ctx+j and its lse is ln(ctx + j + 1)."""
    rng = np.random.default_rng(23)
    tp = Tracked(32, 4, 1, 1, 8)
    s = tp.alloc()
    tp.append([s], 10, rng)
    out, lse = prefill(tp.pool, 0, [s], [6], np.zeros((6, 2, 8), np.uint16), 0.7)
    v = bf16_bits_to_f64(tp.data[s][1][0, :, 0])    # [10][8]
    for j in range(6):
        seen = 4 + j + 1
        assert np.allclose(out[j, 0], v[:seen].mean(axis=0), rtol=0, atol=1e-15)
        assert math.isclose(lse[j, 1], math.log(seen), abs_tol=1e-15)


def test_prefill_argument_errors():
    rng = np.random.default_rng(24)
    tp = Tracked(16, 4, 1, 1, 8)
    s = tp.alloc()
    tp.append([s], 5, rng)
    with pytest.raises(ArgError):
        prefill(tp.pool, 0, [s], [6], np.zeros((6, 1, 8), np.uint16), 1.0)
    with pytest.raises(ArgError):
        prefill(tp.pool, 0, [s], [2], np.zeros((3, 1, 8), np.uint16), 1.0)
    out, lse = prefill(tp.pool, 0, [s], [0], np.zeros((0, 1, 8), np.uint16), 1.0)
    assert out.shape == (0, 1, 8) and lse.shape == (0, 1)
