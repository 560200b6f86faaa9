"""Plain model of a refcounted, copy-on-write block pool (test infrastructure).

Rules, and where they come from:

* K/V live in fixed-size token blocks drawn from one shared pool, and each
  sequence holds an ordered list of block ids instead of a contiguous array
  ("Introducing RadixAttention into Trellis", section *RadixAttention in
  Trellis*; the Dendrite page, section details, 16-token PagedAttention
  blocks).
* A sequence that shares a prefix *acquires* the existing blocks by raising
  their refcounts instead of allocating new ones (Trellis page, same
  section).  Forking copies the parent's block-table pointers, not K/V data
  (Dendrite page, section details: copy-on-write fork; glossary entry
  *Copy-on-Write*: share until a modification, copy only then).
* The free list starts as every block id in order and freed pages are
  appended at its end (SGLang RadixAttention page, source-level sketch:
  ``free_page_pool`` built from ``range`` and ``extend`` on reclaim).
  Allocation takes the head of the list -- the pages do not show allocation;
  this is the plain reading.  A caller may give another initial order.
* The cache is append-only: cached K/V never change once written (Trellis
  page, section *LLM prefill and KV cache*), so a block that several
  sequences hold must be copied before one of them writes into it.

Append, for each sequence in call order and each new token in order:
if ``len % B == 0`` take a fresh block; otherwise, if the last block's
refcount is above one, copy its filled slots into a fresh block, hand the
sequence the copy and drop one reference from the original; then write the
token at ``(table[len // B], len % B)`` and increment ``len``.  A call that
cannot get every block it needs changes nothing.
"""

from __future__ import annotations

from collections import deque

import numpy as np


class PoolError(Exception):
    """Base class; every error leaves the model exactly as it was."""


class ArgError(PoolError):
    pass


class OOMError(PoolError):
    pass


class SeqError(PoolError):
    pass


class EmptyError(PoolError):
    pass


class PoolModel:
    def __init__(self, num_blocks, block_size, num_layers=1, num_kv_heads=1,
                 head_dim=1, free_order=None, store_data=True):
        if num_blocks <= 0 or block_size <= 0:
            raise ArgError("pool needs blocks and a positive block size")
        self.N = int(num_blocks)
        self.B = int(block_size)
        self.L = int(num_layers)
        self.Hkv = int(num_kv_heads)
        self.D = int(head_dim)
        if free_order is None:
            order = list(range(self.N))
        else:
            order = [int(b) for b in free_order]
            if sorted(order) != list(range(self.N)):
                raise ArgError("free order must be a permutation of the block ids")
        self.fifo = deque(order)
        self.rc = [0] * self.N
        self.tables: dict[int, list[int]] = {}
        self.lens: dict[int, int] = {}
        self.next_id = 0
        self.store_data = store_data
        if store_data:
            # block-major copy of the pool: [block][slot][layer][kv head][dim]
            shape = (self.N, self.B, self.L, self.Hkv, self.D)
            self.kbits = np.zeros(shape, dtype=np.uint16)
            self.vbits = np.zeros(shape, dtype=np.uint16)
        # number of slots ever written in each block (for content checks)
        self.filled = [0] * self.N

    # ---------------------------------------------------------------- ops
    def allocate(self) -> int:
        sid = self.next_id
        self.next_id += 1
        self.tables[sid] = []
        self.lens[sid] = 0
        return sid

    def _check(self, sid):
        if sid not in self.tables:
            raise SeqError(f"unknown sequence {sid}")

    def fork(self, parent: int) -> int:
        self._check(parent)
        sid = self.next_id
        self.next_id += 1
        self.tables[sid] = list(self.tables[parent])
        self.lens[sid] = self.lens[parent]
        for b in self.tables[sid]:
            self.rc[b] += 1
        return sid

    def free(self, sid: int) -> None:
        self._check(sid)
        for b in self.tables[sid]:
            self.rc[b] -= 1
            if self.rc[b] == 0:
                self.fifo.append(b)
                self.filled[b] = 0
        del self.tables[sid]
        del self.lens[sid]

    def adopt(self, blocks, length: int) -> int:
        """New sequence over blocks someone already holds (a prefix-cache
        hit): the table is ``blocks``, the length ``length``, and each block
        gains a reference ("Introducing RadixAttention into Trellis",
        section "RadixAttention in Trellis": a session sharing a prefix
        acquires the existing blocks, refcount + 1)."""
        blocks = [int(b) for b in blocks]
        if blocks and not (len(blocks) - 1) * self.B < length <= len(blocks) * self.B:
            raise ArgError("length does not fit the block count")
        if not blocks and length != 0:
            raise ArgError("length does not fit the block count")
        for b in blocks:
            if self.rc[b] < 1:
                raise ArgError(f"block {b} is not held")
        sid = self.next_id
        self.next_id += 1
        self.tables[sid] = list(blocks)
        self.lens[sid] = length
        for b in blocks:
            self.rc[b] += 1
        return sid

    def hold(self, block: int) -> None:
        """One more reference held outside any sequence (a cache's own)."""
        if self.rc[block] < 1:
            raise ArgError(f"block {block} is not held")
        self.rc[block] += 1

    def unhold(self, block: int) -> None:
        """Drop a reference taken by :meth:`hold`; zero -> tail of the free list."""
        self.rc[block] -= 1
        if self.rc[block] == 0:
            self.fifo.append(block)
            self.filled[block] = 0

    def append(self, seqs, n_tok, k_bits=None, v_bits=None):
        """Append ``n_tok`` tokens to each sequence in ``seqs``.

        ``k_bits``/``v_bits``: uint16 ``[L][len(seqs)][n_tok][Hkv][D]`` or None
        (bookkeeping only).  Returns ``(slots, cow)`` where ``slots[i][j]`` is
        the ``(block, offset)`` that token ``j`` of sequence ``i`` went to and
        ``cow`` lists ``(src, dst, n_slots_copied)`` in the order taken.
        """
        seqs = [int(s) for s in seqs]
        if n_tok < 0:
            raise ArgError("negative token count")
        if len(set(seqs)) != len(seqs):
            raise ArgError("a sequence appears twice in one append")
        for s in seqs:
            self._check(s)
        if k_bits is not None:
            want = (self.L, len(seqs), n_tok, self.Hkv, self.D)
            if k_bits.shape != want or v_bits is None or v_bits.shape != want:
                raise ArgError(f"K/V must be shaped {want}")

        # dry run on copies: the call is all-or-nothing
        rc = list(self.rc)
        fifo = deque(self.fifo)
        tables = {s: list(self.tables[s]) for s in seqs}
        lens = {s: self.lens[s] for s in seqs}
        slots = []
        cow = []
        for s in seqs:
            t = tables[s]
            mine = []
            for _ in range(n_tok):
                n = lens[s]
                if n % self.B == 0:
                    if not fifo:
                        raise OOMError("pool exhausted")
                    b = fifo.popleft()
                    rc[b] = 1
                    t.append(b)
                elif rc[t[-1]] > 1:
                    if not fifo:
                        raise OOMError("pool exhausted")
                    src = t[-1]
                    dst = fifo.popleft()
                    rc[dst] = 1
                    rc[src] -= 1
                    t[-1] = dst
                    cow.append((src, dst, n % self.B))
                mine.append((t[n // self.B], n % self.B))
                lens[s] = n + 1
            slots.append(mine)

        # commit
        self.rc = rc
        self.fifo = fifo
        for s in seqs:
            self.tables[s] = tables[s]
            self.lens[s] = lens[s]
        for src, dst, n in cow:
            if self.store_data:
                self.kbits[dst, :n] = self.kbits[src, :n]
                self.vbits[dst, :n] = self.vbits[src, :n]
            self.filled[dst] = n
        for i, mine in enumerate(slots):
            for j, (b, off) in enumerate(mine):
                if self.store_data and k_bits is not None:
                    self.kbits[b, off] = k_bits[:, i, j]
                    self.vbits[b, off] = v_bits[:, i, j]
                self.filled[b] = max(self.filled[b], off + 1)
        return slots, cow

    def tree_commit(self, seqs, n_nodes, parents, paths):
        """Keep the accepted path of each sequence's draft tree, drop the rest.

        The target model checks a draft tree in one pass and keeps the tokens
        it accepts (CAST page: lay summary part 2, the target approves the
        draft's guesses and the tree keeps other branches alive; technical
        summary, the accept length).  Reading: the tree is the last
        ``n_nodes`` tokens of the sequence in node order (as in verify);
        ``paths[i]`` lists the accepted nodes root first, each the parent of
        the next (possibly empty).  Afterwards the sequence is its context
        followed by the accepted nodes' tokens, in path order, and blocks
        past the new length are released in table order.

        Per sequence in call order: (1) release the blocks past the new
        length; (2) each block that receives a moved token (position
        ``ctx + k`` with ``path[k] != k``) and is shared is copied first
        (copy-on-write of its slots below the new length, fresh block from
        the free-list head, the old block loses a reference), in table
        order; copies take only blocks that were free before the call,
        since a block this call releases may still hold a kept token.
        All-or-nothing.  Returns the copies ``(src, dst, n_slots)``.
        """
        seqs = [int(s) for s in seqs]
        if len(set(seqs)) != len(seqs):
            raise ArgError("a sequence appears twice in one commit")
        if len(parents) != len(seqs) or len(paths) != len(seqs):
            raise ArgError("one tree and one path per sequence")
        for s, par, path in zip(seqs, parents, paths):
            self._check(s)
            if not 1 <= n_nodes <= self.lens[s]:
                raise ArgError("tree larger than the sequence")
            par = [int(x) for x in par]
            if len(par) != n_nodes or par[0] != -1 or any(not 0 <= par[i] < i for i in range(1, n_nodes)):
                raise ArgError("parents must form a tree in node order")
            path = [int(x) for x in path]
            if path and (path[0] != 0 or any(par[path[k]] != path[k - 1] for k in range(1, len(path)))
                         or any(not 0 <= x < n_nodes for x in path)):
                raise ArgError("path must run from the root along parent links")
        rc = list(self.rc)
        fifo = deque(self.fifo)
        free_before = len(self.fifo)    # copies take only blocks free before the call
        taken = 0
        tables = {s: list(self.tables[s]) for s in seqs}
        lens = {s: self.lens[s] for s in seqs}
        cow = []
        for s, path in zip(seqs, paths):
            t = tables[s]
            ctx = lens[s] - n_nodes
            new_len = ctx + len(path)
            keep = -(-new_len // self.B)
            for b in t[keep:]:
                rc[b] -= 1
                if rc[b] == 0:
                    fifo.append(b)
            del t[keep:]
            written = sorted({(ctx + k) // self.B for k in range(len(path)) if path[k] != k})
            for i in written:
                if rc[t[i]] > 1:
                    if taken >= free_before:
                        raise OOMError("pool exhausted")
                    src = t[i]
                    dst = fifo.popleft()
                    taken += 1
                    rc[dst] = 1
                    rc[src] -= 1
                    t[i] = dst
                    cow.append((s, src, dst, min(self.B, new_len - i * self.B)))
            lens[s] = new_len
        # data: every kept token's bits are read from the old layout first
        moves = []
        if self.store_data:
            for s, path in zip(seqs, paths):
                ctx = self.lens[s] - n_nodes
                old = self.tables[s]
                for k in range(len(path)):
                    if path[k] != k:
                        p = ctx + path[k]
                        b, off = old[p // self.B], p % self.B
                        moves.append((s, ctx + k, self.kbits[b, off].copy(), self.vbits[b, off].copy()))
        self.rc = rc
        self.fifo = fifo
        for s in seqs:
            self.tables[s] = tables[s]
            self.lens[s] = lens[s]
        for _, src, dst, n in cow:
            if self.store_data:
                self.kbits[dst, :n] = self.kbits[src, :n]
                self.vbits[dst, :n] = self.vbits[src, :n]
            self.filled[dst] = n
        for s, pos, kb, vb in moves:
            b, off = self.tables[s][pos // self.B], pos % self.B
            self.kbits[b, off] = kb
            self.vbits[b, off] = vb
        for b in range(self.N):
            if self.rc[b] == 0:
                self.filled[b] = 0
        return [(src, dst, n) for _, src, dst, n in cow]

    # --------------------------------------------------------- inspection
    def table(self, sid):
        self._check(sid)
        return list(self.tables[sid])

    def length(self, sid):
        self._check(sid)
        return self.lens[sid]

    def free_list(self):
        return list(self.fifo)

    def snapshot(self):
        return {
            "tables": {s: list(t) for s, t in self.tables.items()},
            "lens": dict(self.lens),
            "rc": list(self.rc),
            "fifo": list(self.fifo),
        }

    def gather_bits(self, sid, layer):
        """The sequence's K and V bits in logical token order, ``[len][Hkv][D]``.

        Token ``t`` is read from block ``table[t // B]`` at slot ``t % B``.
        """
        self._check(sid)
        if not self.store_data:
            raise ArgError("this model keeps no K/V data")
        n = self.lens[sid]
        tok = np.arange(n)
        blocks = np.asarray(self.tables[sid], dtype=np.int64)[tok // self.B]
        offs = tok % self.B
        return (self.kbits[blocks, offs, layer].copy(),
                self.vbits[blocks, offs, layer].copy())
