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
