"""Pins of the oracle's radix prefix cache (CPU only).

* The pages' own examples: the Trellis page's "hello my name is Alice" /
  "hello my name is Bob" tree of three entries; the SGLang page's split of
  an edge [A, B, C, D] by a request [A, B, E, F] into a parent [A, B] over
  [C, D] and [E, F], done by slicing pages (no page copied); the Trellis
  benchmark's hit-rate ceiling (L/32 - 1)/(L/32) for a probe that differs
  in the warm prompt's last 32-token block.
* A hand-derived trace of locks and leaf-first LRU eviction (worked out from
  the SGLang page's rules, written below with the reasoning).
* Brute force: the matched length of every probe equals the longest
  whole-block common prefix with any inserted prompt, the blocks returned
  are those of the first prompt inserted with that prefix, and lock counts
  equal the number of unreleased matches that reach into each edge.
* Pool invariants after every operation: refcounts = table references +
  cached pages, free list + held blocks = pool size.
"""

import random

import pytest

from oracle import PoolModel, RadixModel
from oracle.pool import ArgError, SeqError


def run_prompt(pool, cache, tokens, insert=True, release=True):
    """A request: match, append the rest, (insert), (release); returns the sequence."""
    sid, matched = cache.match(tokens)
    if len(tokens) > matched:
        pool.append([sid], len(tokens) - matched)
    if insert:
        cache.insert(sid, tokens)
    if release:
        cache.release(sid)
    return sid, matched


def check_invariants(pool, cache):
    held = sum(len(t) for t in pool.tables.values()) + cache.cached_pages()
    assert sum(pool.rc) == held
    assert len(pool.fifo) + sum(1 for r in pool.rc if r > 0) == pool.N
    assert not set(pool.fifo) & {b for b in range(pool.N) if pool.rc[b] > 0}
    for depth, toks, lock, pages in cache.dump():
        assert len(toks) == len(pages) * pool.B and pages
        assert lock >= 0


# ------------------------------------------------------- the pages' examples

def text(s):
    return [ord(c) for c in s]


def test_alice_and_bob_make_three_entries():
    pool = PoolModel(64, 1)
    cache = RadixModel(pool)
    for prompt in ("hello my name is Alice", "hello my name is Bob"):
        sid, _ = run_prompt(pool, cache, text(prompt))
        pool.free(sid)
    d = cache.dump()
    assert [(depth, "".join(map(chr, toks))) for depth, toks, _, _ in d] == [
        (1, "hello my name is "), (2, "Alice"), (2, "Bob")]
    # the shared entry is stored once: 17 + 5 + 3 blocks for 22 + 20 tokens
    assert cache.cached_pages() == 25
    check_invariants(pool, cache)


def test_edge_split_slices_pages_without_copying():
    A, B_, C, D, E, F = 1, 2, 3, 4, 5, 6
    pool = PoolModel(16, 1)
    cache = RadixModel(pool)
    s1, m1 = run_prompt(pool, cache, [A, B_, C, D])
    assert m1 == 0 and pool.table(s1) == [0, 1, 2, 3]
    s2, m2 = cache.match([A, B_, E, F])
    # the common prefix's pages are acquired, not recomputed
    assert m2 == 2 and pool.table(s2) == [0, 1]
    pool.append([s2], 2)
    assert pool.table(s2) == [0, 1, 4, 5]
    cache.insert(s2, [A, B_, E, F])
    assert cache.dump() == [
        (1, [A, B_], 1, [0, 1]),    # s2's match ended at the cut: it locks [A, B] only
        (2, [C, D], 0, [2, 3]),
        (2, [E, F], 0, [4, 5]),
    ]
    cache.release(s2)
    assert [n[2] for n in cache.dump()] == [0, 0, 0]
    # pages 0, 1: s1, s2 and the cache; nothing was copied: 6 blocks in use
    assert pool.rc[:6] == [3, 3, 2, 2, 2, 2]
    assert len(pool.fifo) == 10
    check_invariants(pool, cache)


@pytest.mark.parametrize("L", [128, 512, 2048])
def test_hit_rate_ceiling_when_the_last_block_differs(L):
    B = 32
    pool = PoolModel(2 * L // B + 4, B)
    cache = RadixModel(pool)
    rng = random.Random(L)
    warm = [rng.randrange(1000) for _ in range(L)]
    s, _ = run_prompt(pool, cache, warm)
    pool.free(s)
    for flip in (L - B, L - 1, L - B // 2):      # any token of the last block
        probe = list(warm)
        probe[flip] += 1000
        sid, matched = cache.match(probe)
        assert matched / L == (L / 32 - 1) / (L / 32)
        cache.release(sid)
        pool.free(sid)
    sid, matched = cache.match(warm)
    assert matched == L
    check_invariants(pool, cache)


# ---------------------------------------------- hand-derived eviction trace

def test_lock_and_lru_eviction_trace():
    """B = 2, 16 blocks, identity free list.

    1. P1 = [1,2,3,4,5,6]: fresh sequence, blocks 0,1,2; insert -> node X
       (pages 0,1,2, stamp 1); free the sequence -> rc 1 (the cache).
    2. P2 = [1,2,3,4,7,8]: match -> 4 tokens, pages 0,1, X locked (stamp
       2); append -> block 3; insert: X touched (3) and split after 2
       blocks: M = [1,2,3,4] (pages 0,1, lock 1, stamp 3) over X' = [5,6]
       (page 2) and a new leaf Y = [7,8] (page 3, stamp 4); release -> all
       locks 0; free the sequence.
    3. P3 = [9,9]: block 4, leaf Z (stamp 5); free the sequence.
       Free list: 5..15 (11 blocks).
    4. evict(12): oldest unlocked leaf X' (3) -> block 2 freed; 12 free.
    5. evict(14): Y (4) -> block 3; now M is a leaf (3) and older than Z (5)
       -> blocks 0, 1; 15 free.  Z stays.
    6. A request [9,9,1] matches Z (2 tokens) and locks it: evict(16)
       fails and changes nothing.
    7. Released, evict(16) drops Z, but the request still holds block 4:
       15 free, fails; freeing the request returns block 4: 16 free.
    """
    pool = PoolModel(16, 2)
    cache = RadixModel(pool)
    s1, _ = run_prompt(pool, cache, [1, 2, 3, 4, 5, 6])
    pool.free(s1)
    s2, m2 = run_prompt(pool, cache, [1, 2, 3, 4, 7, 8])
    assert m2 == 4
    pool.free(s2)
    s3, _ = run_prompt(pool, cache, [9, 9])
    pool.free(s3)
    assert cache.dump() == [(1, [1, 2, 3, 4], 0, [0, 1]), (2, [5, 6], 0, [2]),
                            (2, [7, 8], 0, [3]), (1, [9, 9], 0, [4])]
    assert list(pool.fifo) == list(range(5, 16))
    assert cache.evict(12)
    assert list(pool.fifo) == list(range(5, 16)) + [2]
    assert cache.evict(14)
    assert list(pool.fifo) == list(range(5, 16)) + [2, 3, 0, 1]
    assert cache.dump() == [(1, [9, 9], 0, [4])]
    s4, m4 = cache.match([9, 9, 1])
    assert m4 == 2 and cache.dump() == [(1, [9, 9], 1, [4])]
    assert not cache.evict(16)
    assert cache.dump() == [(1, [9, 9], 1, [4])] and len(pool.fifo) == 15
    cache.release(s4)
    assert not cache.evict(16)
    assert cache.dump() == [] and len(pool.fifo) == 15 and pool.rc[4] == 1
    pool.free(s4)
    assert len(pool.fifo) == 16 and pool.fifo[-1] == 4
    check_invariants(pool, cache)


def test_errors():
    pool = PoolModel(8, 2)
    cache = RadixModel(pool)
    s = pool.allocate()
    pool.append([s], 3)
    with pytest.raises(ArgError):
        cache.insert(s, [1, 2, 3, 4])
    with pytest.raises(SeqError):
        cache.release(s)
    m, _ = cache.match([1, 2])
    cache.release(m)
    with pytest.raises(SeqError):
        cache.release(m)


# ------------------------------------------------------------- brute force

def whole_block_lcp(a, b, B):
    n = 0
    while n + B <= min(len(a), len(b)) and a[n:n + B] == b[n:n + B]:
        n += B
    return n


@pytest.mark.parametrize("B,seed", [(1, 1), (2, 2), (4, 3), (4, 4), (8, 5)])
def test_matches_equal_brute_force(B, seed):
    rng = random.Random(seed)
    pool = PoolModel(4096, B)
    cache = RadixModel(pool)
    inserted = []          # (tokens, table) in insertion order
    live = {}              # unreleased matches: sequence -> (tokens, matched)
    for step in range(120):
        if inserted and rng.random() < 0.7:
            base = rng.choice(inserted)[0]
            cut = rng.randrange(len(base) + 1)
            tokens = base[:cut] + [rng.randrange(3) for _ in range(rng.randrange(0, 12))]
        else:
            tokens = [rng.randrange(3) for _ in range(rng.randrange(0, 20))]
        sid, matched = cache.match(tokens)
        best = max([whole_block_lcp(tokens, t, B) for t, _ in inserted] + [0])
        assert matched == best
        # blocks: those of the first inserted prompt sharing each whole block
        for i in range(matched // B):
            first = next(tab for t, tab in inserted if whole_block_lcp(tokens, t, B) > i * B)
            assert pool.table(sid)[i] == first[i]
        if len(tokens) > matched:
            pool.append([sid], len(tokens) - matched)
        if rng.random() < 0.8:
            cache.insert(sid, tokens)
            inserted.append((tokens, pool.table(sid)))
        live[sid] = (tokens, matched)
        if rng.random() < 0.5:
            victim = rng.choice(sorted(live))
            cache.release(victim)
            del live[victim]
            if rng.random() < 0.5:
                pool.free(victim)
        # lock of a node = unreleased matches whose matched tokens reach into its edge
        pos = {}
        for depth, toks, lock, pages in cache.dump():
            pos[depth] = pos.get(depth - 1, []) + toks
            start = len(pos[depth]) - len(toks)
            want = sum(1 for t, m in live.values()
                       if m > start and t[:start + B] == pos[depth][:start + B])
            assert lock == want
        check_invariants(pool, cache)
