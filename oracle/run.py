"""Run a ``synth`` op program through the oracle (test infrastructure)."""

from __future__ import annotations

from .attention import decode, prefill, tree_verify
from .pool import PoolModel


_DEFAULT = object()


def run_program(workload, store_data=True, want=None, free_order=_DEFAULT):
    """Execute ``workload.ops`` on a fresh :class:`PoolModel`.

    Yields ``(index, op, pool, handles, result)`` after every op, where
    ``result`` is ``(out, lse)`` for decode/verify/prefill ops whose index is in
    ``want`` (all of them when ``want`` is None) and None otherwise.
    ``free_order`` overrides the workload's initial free-list order.
    """
    s = workload.shape
    order = workload.free_order() if free_order is _DEFAULT else free_order
    pool = PoolModel(s.num_blocks, s.block_size, s.num_layers, s.num_kv_heads,
                     s.head_dim, free_order=order, store_data=store_data)
    handles = {}
    for idx, op in enumerate(workload.ops):
        kind = op[0]
        result = None
        if kind == "alloc":
            handles[op[1]] = pool.allocate()
        elif kind == "fork":
            handles[op[2]] = pool.fork(handles[op[1]])
        elif kind == "free":
            pool.free(handles.pop(op[1]))
        elif kind == "append":
            hs, n_tok, key = op[1], op[2], op[3]
            if store_data:
                k, v = workload.append_data(key, len(hs), n_tok)
            else:
                k = v = None
            pool.append([handles[h] for h in hs], n_tok, k, v)
        elif kind == "decode":
            hs, layer, key = op[1], op[2], op[3]
            if store_data and (want is None or idx in want):
                q = workload.decode_query(key, len(hs))
                result = decode(pool, layer, [handles[h] for h in hs], q,
                                workload.sm_scale)
        elif kind == "verify":
            hs, layer, n_nodes, key = op[1], op[2], op[3], op[4]
            if store_data and (want is None or idx in want):
                parents = workload.tree_parents(key, len(hs), n_nodes)
                q = workload.verify_query(key, len(hs), n_nodes)
                result = tree_verify(pool, layer, [handles[h] for h in hs],
                                     parents, q, workload.sm_scale)
        elif kind == "commit":
            hs, n_nodes, tree_key, path_key = op[1], op[2], op[3], op[4]
            parents = workload.tree_parents(tree_key, len(hs), n_nodes)
            paths = workload.accept_paths(path_key, parents)
            pool.tree_commit([handles[h] for h in hs], n_nodes, parents, paths)
        elif kind == "prefill":
            hs, layer, n_new, key = op[1], op[2], op[3], op[4]
            if store_data and (want is None or idx in want):
                q = workload.prefill_query(key, sum(n_new))
                result = prefill(pool, layer, [handles[h] for h in hs], n_new, q,
                                 workload.sm_scale)
        else:
            raise ValueError(f"unknown op {kind}")
        yield idx, op, pool, handles, result
