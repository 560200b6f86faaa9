"""Textbook softmax attention in float64 over paged sequences (test infrastructure).

Decode: the query of a sequence is its newest token, already appended, and
it attends to every cached token of the sequence, its own included -- making
token t+1 needs the keys and values of tokens 0..t ("Introducing
RadixAttention into Trellis", section *LLM prefill and KV cache*).

Query head ``h`` reads key/value head ``h // (Hq // Hkv)`` (contiguous head
groups; the pages do not name a grouping, this is the plain reading).

Tree verify: a draft model proposes a tree of tokens and the target model
checks all of them in one forward pass ("Inference-Cost-Aware Dynamic Tree
Construction ...", technical summary, *Problem*; draft trees keep
alternative branches, lay summary part 2).  The tree's tokens are the last
``n_nodes`` tokens of the sequence, in node order.  Node ``i`` attends to the
whole context before the tree, to its ancestors, and to itself -- the same
rule causal attention applies along one branch.

All arithmetic is float64 on exact bf16 -> float64 upcasts:
``z_t = scale * <q, k_t>``, ``m = max z``, ``p_t = exp(z_t - m) / sum exp(z - m)``,
``out = sum_t p_t v_t``, ``lse = m + ln(sum exp(z - m))`` (natural log).
"""

from __future__ import annotations

import numpy as np

from .pool import ArgError, EmptyError


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def attend(q, k, v, scale):
    """Softmax attention of query rows over one key set.

    ``q [R][D]``, ``k [n][D]``, ``v [n][D]`` (float64) -> ``out [R][D]``, ``lse [R]``.
    """
    if k.shape[0] == 0:
        raise EmptyError("attention over an empty key set")
    z = scale * (q @ k.T)                       # [R][n]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    s = e.sum(axis=1, keepdims=True)
    out = (e @ v) / s
    lse = (m + np.log(s))[:, 0]
    return out, lse


def _group(num_q_heads, num_kv_heads):
    if num_kv_heads <= 0 or num_q_heads % num_kv_heads:
        raise ArgError("query heads must be a multiple of kv heads")
    return num_q_heads // num_kv_heads


def decode(pool, layer, seqs, q_bits, sm_scale):
    """One query per sequence. ``q_bits`` uint16 ``[n][Hq][D]``.

    Returns float64 ``out [n][Hq][D]`` and ``lse [n][Hq]``.
    """
    q = bf16_bits_to_f64(q_bits)
    n, hq, d = q.shape
    g = _group(hq, pool.Hkv)
    out = np.empty((n, hq, d))
    lse = np.empty((n, hq))
    for i, sid in enumerate(seqs):
        kb, vb = pool.gather_bits(sid, layer)
        if kb.shape[0] == 0:
            raise EmptyError("decode on an empty sequence")
        k = bf16_bits_to_f64(kb)
        v = bf16_bits_to_f64(vb)
        for kvh in range(pool.Hkv):
            rows = slice(kvh * g, (kvh + 1) * g)
            out[i, rows], lse[i, rows] = attend(q[i, rows], k[:, kvh], v[:, kvh], sm_scale)
    return out, lse


def _check_parents(parent):
    parent = np.asarray(parent)
    if parent.ndim != 1 or parent.size == 0 or parent[0] != -1:
        raise ArgError("node 0 must be the root (parent -1)")
    for i in range(1, parent.size):
        if not 0 <= parent[i] < i:
            raise ArgError("parent[i] must be an earlier node")
    return parent


def tree_key_positions(parent, node, ctx_len):
    """Positions node ``node`` attends to: ``0..ctx_len-1`` plus its path.

    The path is the node and all its ancestors, found by following parent
    pointers to the root; tree node ``j`` sits at position ``ctx_len + j``.
    """
    parent = _check_parents(parent)
    path = []
    j = node
    while j != -1:
        path.append(int(j))
        j = int(parent[j])
    return list(range(ctx_len)) + [ctx_len + j for j in sorted(path)]


def tree_verify(pool, layer, seqs, parents, q_bits, sm_scale):
    """Every draft-tree node of every sequence.

    ``parents`` int ``[n][T]``; ``q_bits`` uint16 ``[n][T][Hq][D]``.
    Returns float64 ``out [n][T][Hq][D]`` and ``lse [n][T][Hq]``.
    """
    q = bf16_bits_to_f64(q_bits)
    n, t_nodes, hq, d = q.shape
    parents = np.asarray(parents)
    if parents.shape != (n, t_nodes):
        raise ArgError("parents must be [n_seqs][n_nodes]")
    g = _group(hq, pool.Hkv)
    out = np.empty((n, t_nodes, hq, d))
    lse = np.empty((n, t_nodes, hq))
    for i, sid in enumerate(seqs):
        kb, vb = pool.gather_bits(sid, layer)
        ctx = kb.shape[0] - t_nodes
        if ctx < 0:
            raise ArgError("sequence shorter than its tree")
        k = bf16_bits_to_f64(kb)
        v = bf16_bits_to_f64(vb)
        for j in range(t_nodes):
            pos = tree_key_positions(parents[i], j, ctx)
            for kvh in range(pool.Hkv):
                rows = slice(kvh * g, (kvh + 1) * g)
                out[i, j, rows], lse[i, j, rows] = attend(
                    q[i, j, rows], k[pos, kvh], v[pos, kvh], sm_scale)
    return out, lse


def prefill(pool, layer, seqs, n_new, q_bits, sm_scale):
    """Causal attention of each sequence's newest tokens over its whole cache.

    After a prefix match only the unmatched part of a prompt is computed
    (SGLang RadixAttention page, "Three core operations", prefix matching:
    the forward pass runs over the n - k tokens that missed); those tokens
    are appended first, and token ``t`` attends to tokens ``0..t`` -- the
    causal rule of the Trellis page's section "LLM prefill and KV cache".

    ``n_new[i]`` tokens of sequence ``i`` are new: they are its last
    ``n_new[i]`` tokens, at positions ``len - n_new[i] .. len - 1``.  ``q_bits``
    uint16 ``[sum(n_new)][Hq][D]`` holds their queries, sequence after
    sequence.  Query ``j`` of sequence ``i`` attends to positions
    ``0 .. len - n_new[i] + j``.
    Returns float64 ``out [sum(n_new)][Hq][D]`` and ``lse [sum(n_new)][Hq]``.
    """
    q = bf16_bits_to_f64(q_bits)
    n_new = [int(x) for x in n_new]
    if len(n_new) != len(seqs):
        raise ArgError("one new-token count per sequence")
    total = sum(n_new)
    if q.shape[0] != total:
        raise ArgError("q must hold sum(n_new) query vectors")
    _, hq, d = q.shape
    g = _group(hq, pool.Hkv)
    out = np.empty((total, hq, d))
    lse = np.empty((total, hq))
    row = 0
    for sid, n in zip(seqs, n_new):
        kb, vb = pool.gather_bits(sid, layer)
        length = kb.shape[0]
        if n < 0 or n > length:
            raise ArgError("more new tokens than the sequence holds")
        k = bf16_bits_to_f64(kb)
        v = bf16_bits_to_f64(vb)
        ctx = length - n
        for j in range(n):
            visible = ctx + j + 1            # keys 0 .. ctx + j
            for kvh in range(pool.Hkv):
                rows = slice(kvh * g, (kvh + 1) * g)
                out[row, rows], lse[row, rows] = attend(
                    q[row, rows], k[:visible, kvh], v[:visible, kvh], sm_scale)
            row += 1
    return out, lse
