"""Workload shapes and op programs for paged KV attention.

A program is a list of ops.  Sequences are named by small integer handles;
each side maps handles to the sequence ids its own pool hands out.

Ops (tuples):

* ``("alloc", h)``                          new empty sequence ``h``
* ``("fork", parent, child)``               child shares parent's blocks
* ``("free", h)``                           drop sequence ``h``
* ``("append", hs, n_tok, key)``            append ``n_tok`` tokens to every
  sequence in ``hs``; K/V come from :meth:`Workload.append_data` (``key``)
* ``("decode", hs, layer, key)``            one query per sequence in ``hs``;
  Q from :meth:`Workload.decode_query`
* ``("verify", hs, layer, n_nodes, key)``   draft-tree verify: the last
  ``n_nodes`` tokens of every sequence in ``hs`` are the tree's nodes (in node
  order); parents from :meth:`Workload.tree_parents`, Q from
  :meth:`Workload.verify_query`
* ``("commit", hs, n_nodes, tree_key, path_key)``  keep the accepted path of
  each sequence's draft tree (parents from :meth:`Workload.tree_parents`
  with ``tree_key``, paths from :meth:`Workload.accept_paths`) and drop the
  other nodes
* ``("prefill", hs, layer, n_new, key)``    causal attention of the newest
  ``n_new[i]`` tokens of sequence ``hs[i]`` (already appended) over its whole
  cache; Q from :meth:`Workload.prefill_query`

Random draws use ``numpy.random.default_rng([cfg_id, stream, key])`` so every
tensor depends on the logical op that consumes it, never on where a pool puts
it.  K/V/Q values are fp32 N(0,1) draws (K optionally multiplied by
``k_scale`` in fp32) rounded to bf16.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from .bf16 import f32_to_bf16_bits

STREAM_K = 1
STREAM_V = 2
STREAM_Q = 3
STREAM_PERM = 4
STREAM_TREE = 5
STREAM_SIGNS = 7


@dataclass(frozen=True)
class Shape:
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_layers: int
    num_blocks: int


@dataclass
class Workload:
    name: str
    cfg_id: int
    shape: Shape
    ops: list
    sm_scale: float
    k_scale: float = 1.0
    permute_free_list: bool = False
    tree_depth: int = 0
    description: str = ""
    meta: dict = field(default_factory=dict)

    # ---- inputs -----------------------------------------------------------
    def _rng(self, stream: int, key: int) -> np.random.Generator:
        return np.random.default_rng([self.cfg_id, stream, key])

    def free_order(self):
        """Initial free-list order: ``None`` (identity) or an int32 permutation."""
        if not self.permute_free_list:
            return None
        rng = self._rng(STREAM_PERM, 0)
        return rng.permutation(self.shape.num_blocks).astype(np.int32)

    def append_data(self, key: int, n_seqs: int, n_tok: int):
        """bf16 bits of K and V, each ``[L][n_seqs][n_tok][Hkv][D]`` (uint16)."""
        s = self.shape
        size = (s.num_layers, n_seqs, n_tok, s.num_kv_heads, s.head_dim)
        k = self._rng(STREAM_K, key).standard_normal(size, dtype=np.float32)
        if self.k_scale != 1.0:
            k = k * np.float32(self.k_scale)
        v = self._rng(STREAM_V, key).standard_normal(size, dtype=np.float32)
        return f32_to_bf16_bits(k), f32_to_bf16_bits(v)

    def rotation_signs(self):
        """int8 [head_dim] of +-1: the random signs of a 4-bit pool's rotation."""
        rng = self._rng(STREAM_SIGNS, 0)
        return np.where(rng.random(self.shape.head_dim) < 0.5, -1, 1).astype(np.int8)

    def decode_query(self, key: int, n_seqs: int):
        """bf16 bits of Q, ``[n_seqs][Hq][D]`` (uint16)."""
        s = self.shape
        q = self._rng(STREAM_Q, key).standard_normal(
            (n_seqs, s.num_q_heads, s.head_dim), dtype=np.float32)
        return f32_to_bf16_bits(q)

    def verify_query(self, key: int, n_seqs: int, n_nodes: int):
        """bf16 bits of Q, ``[n_seqs][n_nodes][Hq][D]`` (uint16)."""
        s = self.shape
        q = self._rng(STREAM_Q, key).standard_normal(
            (n_seqs, n_nodes, s.num_q_heads, s.head_dim), dtype=np.float32)
        return f32_to_bf16_bits(q)

    def prefill_query(self, key: int, n_queries: int):
        """bf16 bits of Q, ``[n_queries][Hq][D]`` (uint16), sequence after sequence."""
        s = self.shape
        q = self._rng(STREAM_Q, key).standard_normal(
            (n_queries, s.num_q_heads, s.head_dim), dtype=np.float32)
        return f32_to_bf16_bits(q)

    def accept_paths(self, key: int, parents):
        """One accepted path per tree (root first along parent links): from
        the root, step to a uniformly drawn child with probability 0.8, else
        stop; with probability 0.1 nothing is accepted."""
        rng = self._rng(STREAM_TREE + 1, key)
        out = []
        for par in np.asarray(parents):
            kids = {}
            for i in range(1, len(par)):
                kids.setdefault(int(par[i]), []).append(i)
            if rng.random() < 0.1:
                out.append([])
                continue
            path = [0]
            while kids.get(path[-1]) and rng.random() < 0.8:
                ch = kids[path[-1]]
                path.append(ch[int(rng.integers(len(ch)))])
            out.append(path)
        return out

    def tree_parents(self, key: int, n_seqs: int, n_nodes: int):
        """int32 ``[n_seqs][n_nodes]`` parent pointers, one draft tree per sequence."""
        rng = self._rng(STREAM_TREE, key)
        depth = self.tree_depth if self.tree_depth > 0 else n_nodes
        return np.stack([draw_tree(rng, n_nodes, depth) for _ in range(n_seqs)])

    # ---- bookkeeping used by reports (no pool rules) ----------------------
    def count(self, kind: str) -> int:
        return sum(1 for op in self.ops if op[0] == kind)


def draw_tree(rng: np.random.Generator, n_nodes: int, max_depth: int) -> np.ndarray:
    """Random draft tree in node order (``parent[0] = -1``, ``parent[i] < i``).

    Node 0 is the root at depth 1.  Each later node picks its parent uniformly
    among the earlier nodes whose depth is below ``max_depth``.  The whole tree
    is redrawn until its deepest node sits exactly at ``max_depth``.
    """
    if n_nodes < 1:
        raise ValueError("a tree needs at least one node")
    max_depth = min(max_depth, n_nodes)
    for _ in range(10000):
        parent = np.full(n_nodes, -1, dtype=np.int32)
        depth = [1]
        for i in range(1, n_nodes):
            cands = [j for j in range(i) if depth[j] < max_depth]
            p = cands[int(rng.integers(len(cands)))]
            parent[i] = p
            depth.append(depth[p] + 1)
        if max(depth) == max_depth:
            return parent
    raise RuntimeError("could not draw a tree of the requested depth")


# ---------------------------------------------------------------------------
# program builders
# ---------------------------------------------------------------------------

def _default_scale(shape: Shape) -> float:
    return 1.0 / math.sqrt(shape.head_dim)


def fork_workload(name, cfg_id, shape, prefix_len, n_branches, branch_len,
                  decode_steps=0, sm_scale=None, permute=False, description=""):
    """One prefix forked into branches (the Dendrite-style fork scenario).

    parent = alloc + append ``prefix_len``; ``n_branches`` forks of it (the
    parent stays alive and issues no queries); all branches append
    ``branch_len`` tokens in one call.  Then, if ``decode_steps == 0``, one
    decode per layer over the branches; otherwise ``decode_steps`` rounds of
    [append 1 token to every branch, decode every layer].
    """
    ops = [("alloc", 0)]
    if prefix_len:
        ops.append(("append", (0,), prefix_len, len(ops)))
    kids = tuple(range(1, n_branches + 1))
    for c in kids:
        ops.append(("fork", 0, c))
    if branch_len:
        ops.append(("append", kids, branch_len, len(ops)))
    if decode_steps == 0:
        for layer in range(shape.num_layers):
            ops.append(("decode", kids, layer, len(ops)))
    else:
        for _ in range(decode_steps):
            ops.append(("append", kids, 1, len(ops)))
            for layer in range(shape.num_layers):
                ops.append(("decode", kids, layer, len(ops)))
    return Workload(name, cfg_id, shape, ops,
                    _default_scale(shape) if sm_scale is None else sm_scale,
                    permute_free_list=permute, description=description,
                    meta=dict(prefix_len=prefix_len, n_branches=n_branches,
                              branch_len=branch_len, decode_steps=decode_steps))


def shared_prompt_workload(name, cfg_id, shape, prompt_len, n_sessions,
                           shared_blocks, decode_steps, sm_scale=None,
                           description=""):
    """A warmed shared system prompt plus per-session suffixes.

    sys = alloc + append ``shared_blocks * block_size`` tokens; each session
    forks sys and appends the rest of its ``prompt_len``-token prompt; then
    ``decode_steps`` rounds of [append 1 token to every session, decode every
    layer].  The sys sequence stays alive and issues no queries.
    """
    shared_len = shared_blocks * shape.block_size
    ops = [("alloc", 0), ("append", (0,), shared_len, 1)]
    sessions = tuple(range(1, n_sessions + 1))
    for h in sessions:
        ops.append(("fork", 0, h))
        if prompt_len > shared_len:
            ops.append(("append", (h,), prompt_len - shared_len, len(ops)))
    for _ in range(decode_steps):
        ops.append(("append", sessions, 1, len(ops)))
        for layer in range(shape.num_layers):
            ops.append(("decode", sessions, layer, len(ops)))
    return Workload(name, cfg_id, shape, ops,
                    _default_scale(shape) if sm_scale is None else sm_scale,
                    description=description,
                    meta=dict(prompt_len=prompt_len, n_sessions=n_sessions,
                              shared_blocks=shared_blocks,
                              decode_steps=decode_steps))


def mcts_workload(name, cfg_id, shape, root_len, depth, fanout, edge_len,
                  sm_scale=None, k_scale=1.0, description=""):
    """A search tree of sequences: root prefix, then ``depth`` levels of forks.

    Built breadth first: every node of a level forks ``fanout`` children, and
    all children of the level append ``edge_len`` tokens in one call.  Every
    node stays alive; one decode query per leaf (per layer).
    """
    ops = [("alloc", 0)]
    if root_len:
        ops.append(("append", (0,), root_len, len(ops)))
    level = [0]
    nxt = 1
    for _ in range(depth):
        kids = []
        for p in level:
            for _ in range(fanout):
                ops.append(("fork", p, nxt))
                kids.append(nxt)
                nxt += 1
        if edge_len:
            ops.append(("append", tuple(kids), edge_len, len(ops)))
        level = kids
    for layer in range(shape.num_layers):
        ops.append(("decode", tuple(level), layer, len(ops)))
    return Workload(name, cfg_id, shape, ops,
                    _default_scale(shape) if sm_scale is None else sm_scale,
                    k_scale=k_scale, description=description,
                    meta=dict(root_len=root_len, depth=depth, fanout=fanout,
                              edge_len=edge_len, leaves=len(level)))


def verify_workload(name, cfg_id, shape, n_seqs, ctx_len, n_nodes, tree_depth,
                    sm_scale=None, permute=False, description=""):
    """Batched draft-tree verification.

    Every sequence = alloc + append ``ctx_len`` context tokens, then the
    ``n_nodes`` draft-tree tokens are appended in node order and one verify
    call per layer runs every node of every tree.
    """
    hs = tuple(range(n_seqs))
    ops = [("alloc", h) for h in hs]
    if ctx_len:
        ops.append(("append", hs, ctx_len, len(ops)))
    ops.append(("append", hs, n_nodes, len(ops)))
    for layer in range(shape.num_layers):
        ops.append(("verify", hs, layer, n_nodes, len(ops)))
    return Workload(name, cfg_id, shape, ops,
                    _default_scale(shape) if sm_scale is None else sm_scale,
                    permute_free_list=permute, tree_depth=tree_depth,
                    description=description,
                    meta=dict(n_seqs=n_seqs, ctx_len=ctx_len, n_nodes=n_nodes,
                              tree_depth=tree_depth))


def verify_commit_workload(name, cfg_id, shape, n_seqs, ctx_len, n_nodes, tree_depth, rounds=1,
                           fork_after=False, sm_scale=None, permute=False, description=""):
    """Speculative rounds: every sequence appends a draft tree, every layer
    verifies it, the accepted paths are committed, then one more token is
    appended and decoded.  ``fork_after``: each sequence is forked after its
    first tree is appended (the fork shares the tree blocks and issues no
    queries), so commits copy the shared blocks they write.
    """
    hs = tuple(range(n_seqs))
    ops = [("alloc", h) for h in hs]
    if ctx_len:
        ops.append(("append", hs, ctx_len, len(ops)))
    nxt = n_seqs
    for r in range(rounds):
        ops.append(("append", hs, n_nodes, len(ops)))
        tree_key = len(ops)
        if fork_after and r == 0:
            for h in hs:
                ops.append(("fork", h, nxt))
                nxt += 1
        for layer in range(shape.num_layers):
            ops.append(("verify", hs, layer, n_nodes, tree_key))
        ops.append(("commit", hs, n_nodes, tree_key, len(ops)))
        ops.append(("append", hs, 1, len(ops)))
        for layer in range(shape.num_layers):
            ops.append(("decode", hs, layer, len(ops)))
    return Workload(name, cfg_id, shape, ops,
                    _default_scale(shape) if sm_scale is None else sm_scale,
                    permute_free_list=permute, tree_depth=tree_depth,
                    description=description,
                    meta=dict(n_seqs=n_seqs, ctx_len=ctx_len, n_nodes=n_nodes,
                              tree_depth=tree_depth, rounds=rounds))


def prefill_workload(name, cfg_id, shape, shared_len, own_lens, sm_scale=None,
                     description=""):
    """Prompts whose first ``shared_len`` tokens hit a cached prefix.

    sys = alloc + append ``shared_len`` tokens (the cached prefix, kept
    alive); session ``i`` forks sys, appends its ``own_lens[i]`` unmatched
    prompt tokens, and one prefill call per layer computes causal attention
    of all sessions' new tokens over their whole caches.
    """
    ops = [("alloc", 0)]
    if shared_len:
        ops.append(("append", (0,), shared_len, len(ops)))
    sessions = tuple(range(1, len(own_lens) + 1))
    for h in sessions:
        ops.append(("fork", 0, h))
    by_len = {}
    for h, n in zip(sessions, own_lens):
        by_len.setdefault(n, []).append(h)
    for n, hs in sorted(by_len.items()):
        if n:
            ops.append(("append", tuple(hs), n, len(ops)))
    for layer in range(shape.num_layers):
        ops.append(("prefill", sessions, layer, tuple(own_lens), len(ops)))
    return Workload(name, cfg_id, shape, ops,
                    _default_scale(shape) if sm_scale is None else sm_scale,
                    description=description,
                    meta=dict(shared_len=shared_len, own_lens=tuple(own_lens)))


# ---------------------------------------------------------------------------
# the five named workloads
# ---------------------------------------------------------------------------

def _c1():
    shape = Shape(8, 2, 64, 16, 1, 64)
    return fork_workload(
        "c1_tiny_fork", 1, shape, prefix_len=128, n_branches=4, branch_len=16,
        permute=True,
        description="8 q / 2 kv heads, D 64, B 16; 128-token prefix forked "
                    "into 4 branches of +16 tokens; one decode per branch; "
                    "free list a seeded permutation of 64 blocks")


def _c2():
    # TinyLlama attention: 32 q heads, 4 kv heads, D 64, 22 layers; B = 32.
    # L = 512, phi = 0.5 -> round(0.5 * 512 / 32) = 8 shared blocks.
    shape = Shape(32, 4, 64, 32, 22, 256)
    return shared_prompt_workload(
        "c2_trellis", 2, shape, prompt_len=512, n_sessions=16,
        shared_blocks=round(0.5 * 512 / 32), decode_steps=64,
        description="32 q / 4 kv heads, D 64, B 32, 22 layers; 16 sessions "
                    "over a 256-token shared prompt + 256 own tokens; 64 "
                    "steps of [append 1, decode 22 layers]")


def _c3(prefix_len=4104):
    shape = Shape(32, 4, 64, 16, 1, 512)
    return fork_workload(
        "c3_dendrite" if prefix_len == 4104 else "c3_dendrite_aligned", 3,
        shape, prefix_len=prefix_len, n_branches=6, branch_len=256,
        decode_steps=128,
        description=f"32 q / 4 kv heads, D 64, B 16; {prefix_len}-token "
                    "prefix forked into 6 branches of +256 tokens; 128 steps "
                    "of [append 1, decode]")


def _c4(folded=False):
    shape = Shape(32, 8, 128, 16, 1, 2048)
    inv = 1.0 / math.sqrt(128)
    return mcts_workload(
        "c4_mcts_folded" if folded else "c4_mcts", 4, shape, root_len=2048,
        depth=4, fanout=4, edge_len=64,
        sm_scale=1.0 if folded else inv, k_scale=inv,
        description="32 q / 8 kv heads, D 128, B 16; 2048-token root, depth "
                    "4 fan-out 4 tree with 64-token edges; one decode per "
                    "leaf (256); K drawn as N(0,1)/sqrt(128)")


def _c5():
    shape = Shape(32, 8, 128, 16, 1, 1536)
    return verify_workload(
        "c5_verify", 5, shape, n_seqs=8, ctx_len=2048, n_nodes=64,
        tree_depth=6,
        description="32 q / 8 kv heads, D 128, B 16; 8 sequences with "
                    "2048-token context and a 64-node depth-6 draft tree each")


def _c2_prefill():
    # The Trellis-shaped prompts' prefill: 256 of each 512-token prompt hit
    # the cached shared prefix, the other 256 are computed (one layer).
    shape = Shape(32, 4, 64, 32, 1, 256)
    return prefill_workload(
        "c2_trellis_prefill", 6, shape, shared_len=256, own_lens=[256] * 16,
        description="32 q / 4 kv heads, D 64, B 32; 16 prompts of 512 tokens "
                    "whose first 256 hit a cached shared prefix; causal prefill "
                    "of the other 256 tokens of every prompt (4096 queries)")


def _c5_commit():
    shape = Shape(32, 8, 128, 16, 1, 1536)
    return verify_commit_workload(
        "c5_verify_commit", 5, shape, n_seqs=8, ctx_len=2048, n_nodes=64, tree_depth=6,
        description="32 q / 8 kv heads, D 128, B 16; 8 sequences with 2048-token "
                    "context; append a 64-node depth-6 draft tree, verify, commit the "
                    "accepted paths, append and decode one token")


_NAMED = {
    "c1_tiny_fork": _c1,
    "c2_trellis": _c2,
    "c3_dendrite": _c3,
    "c3_dendrite_aligned": lambda: _c3(4096),
    "c4_mcts": _c4,
    "c4_mcts_folded": lambda: _c4(True),
    "c5_verify": _c5,
    "c2_trellis_prefill": _c2_prefill,
    "c5_verify_commit": _c5_commit,
}
NAMES = tuple(_NAMED)


def named(name: str) -> Workload:
    """One of the named workloads (see ``NAMES``)."""
    return _NAMED[name]()
