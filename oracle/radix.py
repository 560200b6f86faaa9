"""Block-paged radix-tree prefix cache, as a plain Python model (test infrastructure).

What it follows:

* SGLang RadixAttention page, "Node and edge structure": a node is a branch
  point holding a dictionary of children and a ``ref_counter`` of the active
  requests that use it; an edge holds a slice of token ids plus the
  physical pages storing them; the root is the empty sequence.
* Same page, the three core operations: prefix matching walks the edges
  from the root for the longest common prefix and acquires the pages of the
  matched tokens; inserting a prompt whose tokens leave an edge part-way
  splits that edge into a new parent holding the common part with the two
  remainders below it, by slicing the page list (no page is copied); the new
  tokens become a new node.
* Same page, reference counting and LRU eviction: a node with
  ``ref_counter > 0`` is never evicted; finished requests decrement it and
  the pages stay cached; when memory is short, the leaf with
  ``ref_counter == 0`` and the oldest access time goes first, its pages
  return to the free pool and its edge is cut, and a parent left with no
  children and no references becomes a candidate in turn.
* "Introducing RadixAttention into Trellis", "RadixAttention in Trellis":
  the cache is block-paged -- a session sharing a prefix acquires the
  existing blocks (refcount + 1) -- and the benchmark section rounds the
  shared region to whole 32-token blocks, so the best possible hit rate is
  (L/32 - 1)/(L/32) when a probe differs in the warm prompt's last block.

Readings where the pages leave a step open:

* Granularity: edges hold whole blocks, children are keyed by the tokens of
  their first block, and a match only counts whole blocks (the Trellis
  page's block quantisation).  With ``block_size == 1`` this is the SGLang
  sketch's token-level tree.
* The cache keeps one pool reference on each block it stores; "returning
  pages to the free pool" is dropping that reference (a block still used by
  a live sequence stays allocated until that sequence lets it go).
* A match locks every node whose pages it used, including an edge it
  entered only part-way; a split gives the new parent the child's lock
  count and access time (every match through the child ran through the
  common part), and a live match that ended before the cut stops locking
  the remainder.
* Access time is a counter bumped for every node a match or insert touches
  (root first), which makes runs reproducible and ties impossible.
* Insert caches the whole blocks of a sequence's tokens; for tokens already
  in the tree the tree keeps its own blocks.
"""

from __future__ import annotations

from .pool import ArgError, SeqError


class _Node:
    def __init__(self, parent=None):
        self.parent = parent
        self.children = {}      # tuple of the first block's tokens -> _Node
        self.tokens = []        # the edge into this node
        self.pages = []         # one pool block per block_size tokens of the edge
        self.ref_counter = 0
        self.last_access = 0


class RadixModel:
    """Prefix cache over a :class:`oracle.pool.PoolModel`."""

    def __init__(self, pool):
        self.pool = pool
        self.B = pool.B
        self.root = _Node()
        self.clock = 0
        self.paths = {}         # sequence id -> nodes its match locked (root side first)
        self.reach = {}         # sequence id -> tokens it matched of its last node's edge

    # ---- helpers -------------------------------------------------------
    def _stamp(self, node):
        self.clock += 1
        node.last_access = self.clock

    def _nodes(self):
        out = []
        todo = [self.root]
        while todo:
            n = todo.pop()
            if n is not self.root:
                out.append(n)
            todo.extend(n.children.values())
        return out

    def _common_blocks(self, tokens, pos, node, limit_blocks):
        """Whole blocks that tokens[pos:] shares with node's edge (at most limit_blocks)."""
        B = self.B
        m = 0
        while (m < len(node.pages) and m < limit_blocks
               and list(tokens[pos + m * B:pos + (m + 1) * B]) == node.tokens[m * B:(m + 1) * B]):
            m += 1
        return m

    def _split(self, child, keep):
        """Cut child's edge after `keep` blocks; the common part becomes its new parent."""
        B = self.B
        parent = child.parent
        mid = _Node(parent)
        mid.tokens = child.tokens[:keep * B]
        mid.pages = child.pages[:keep]
        child.tokens = child.tokens[keep * B:]
        child.pages = child.pages[keep:]
        mid.ref_counter = child.ref_counter
        mid.last_access = child.last_access
        parent.children[tuple(mid.tokens[:B])] = mid
        mid.children[tuple(child.tokens[:B])] = child
        child.parent = mid
        for sid, path in self.paths.items():
            if child not in path:
                continue
            if path[-1] is child and self.reach[sid] <= keep * B:
                # the match ended before the cut: it holds the common part only
                path[-1] = mid
                child.ref_counter -= 1
            else:
                path.insert(path.index(child), mid)
                if path[-1] is child:
                    self.reach[sid] -= keep * B
        return mid

    # ---- the operations -----------------------------------------------
    def match(self, tokens):
        """Longest cached whole-block prefix -> (new sequence id, matched tokens)."""
        B = self.B
        tokens = [int(t) for t in tokens]
        cur = self.root
        pos = 0
        pages = []
        path = []
        reach = 0
        while len(tokens) - pos >= B:
            child = cur.children.get(tuple(tokens[pos:pos + B]))
            if child is None:
                break
            m = self._common_blocks(tokens, pos, child, (len(tokens) - pos) // B)
            pages += child.pages[:m]
            path.append(child)
            reach = m * B
            pos += m * B
            if m < len(child.pages):
                break
            cur = child
        sid = self.pool.adopt(pages, pos)
        for node in path:
            node.ref_counter += 1
            self._stamp(node)
        self.paths[sid] = path
        self.reach[sid] = reach
        return sid, pos

    def insert(self, sid, tokens):
        """Cache the whole blocks of sequence ``sid`` under ``tokens``."""
        B = self.B
        tokens = [int(t) for t in tokens]
        table = self.pool.table(sid)
        if len(tokens) > self.pool.length(sid):
            raise ArgError("more tokens than the sequence holds")
        nb = len(tokens) // B
        cur = self.root
        i = 0
        while i < nb:
            key = tuple(tokens[i * B:(i + 1) * B])
            child = cur.children.get(key)
            if child is None:
                leaf = _Node(cur)
                leaf.tokens = tokens[i * B:nb * B]
                leaf.pages = table[i:nb]
                for b in leaf.pages:
                    self.pool.hold(b)
                self._stamp(leaf)
                cur.children[key] = leaf
                break
            self._stamp(child)
            m = self._common_blocks(tokens, i * B, child, nb - i)
            if m < len(child.pages):
                if i + m == nb:
                    break
                child = self._split(child, m)
            i += m
            cur = child

    def release(self, sid):
        """The matching request finished: its nodes lose one reference."""
        if sid not in self.paths:
            raise SeqError("sequence holds no match of this cache")
        for node in self.paths.pop(sid):
            node.ref_counter -= 1
        del self.reach[sid]

    def evict(self, want_free):
        """Leaf-first LRU eviction until the free list holds want_free blocks."""
        while len(self.pool.fifo) < want_free:
            leaves = [n for n in self._nodes() if not n.children and n.ref_counter == 0]
            if not leaves:
                return False
            victim = min(leaves, key=lambda n: n.last_access)
            for b in victim.pages:
                self.pool.unhold(b)
            del victim.parent.children[tuple(victim.tokens[:self.B])]
        return True

    def close(self):
        """Drop every cached reference: nodes in preorder (children by key),
        each edge's pages in order."""
        for _, _, _, pages in self.dump():
            for b in pages:
                self.pool.unhold(b)
        self.root = _Node()
        self.paths = {}

    # ---- views -------------------------------------------------------
    def dump(self):
        """Preorder list of (depth, tokens, ref_counter, pages), children by key."""
        out = []

        def walk(node, depth):
            for key in sorted(node.children):
                c = node.children[key]
                out.append((depth, list(c.tokens), c.ref_counter, list(c.pages)))
                walk(c, depth + 1)

        walk(self.root, 1)
        return out

    def cached_pages(self):
        return sum(len(n.pages) for n in self._nodes())
