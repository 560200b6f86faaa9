"""Run a ``synth`` op program through the C ABI on the GPU.

Device memory comes from torch (pools, new K/V, Q, outputs); every step of
the path runs in libpkv.so.  Nothing here imports the oracle.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

import paged_kv_cache_204_amd as pkv


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda")


class GpuPool:
    def __init__(self, shape, free_order=None, ws_limits=None, ws_bytes=None):
        self.shape = shape
        desc = dict(num_blocks=shape.num_blocks, block_size=shape.block_size,
                    num_layers=shape.num_layers, num_q_heads=shape.num_q_heads,
                    num_kv_heads=shape.num_kv_heads, head_dim=shape.head_dim)
        n = pkv.kv_pool_bytes(desc) // 2
        assert n > 0
        # poison unwritten slots with bf16 NaN so a stray read shows up
        self.k = torch.full((n,), 0x7FC0, dtype=torch.int16, device="cuda")
        self.v = torch.full((n,), 0x7FC0, dtype=torch.int16, device="cuda")
        # ws_limits = (max_seqs, max_tree_nodes): a caller workspace of
        # kv_workspace_bytes (or ws_bytes) bytes, from torch
        self.ws = None
        if ws_limits is not None:
            nbytes = ws_bytes or pkv.kv_workspace_bytes(desc, *ws_limits)
            self.ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
            assert self.ws.data_ptr() % 256 == 0
            self.pool = pkv.kv_pool_create(desc, self.k, self.v, free_order=free_order, workspace=self.ws,
                                           max_seqs=ws_limits[0], max_tree_nodes=ws_limits[1])
        else:
            self.pool = pkv.kv_pool_create(desc, self.k, self.v, free_order=free_order)
        self.stream = torch.cuda.current_stream().cuda_stream

    def close(self):
        if self.pool is not None:
            pkv.kv_pool_destroy(self.pool)
            self.pool = None

    def pool_bits(self):
        s = self.shape
        shp = (s.num_layers, s.num_blocks, s.num_kv_heads, s.block_size, s.head_dim)
        k = self.k.cpu().numpy().view(np.uint16).reshape(shp)
        v = self.v.cpu().numpy().view(np.uint16).reshape(shp)
        return k, v


def run_gpu(workload, want=None, free_order="default", on_result=None, pool_cb=None, ws_limits=None,
            ws_bytes=None):
    """Execute the program; return {op index: (out, lse)} as numpy float32.

    ``want``: op indices whose outputs are copied back (None = all).
    ``pool_cb(gpu_pool, handles)`` runs at the end, before the pool closes.
    """
    s = workload.shape
    order = workload.free_order() if isinstance(free_order, str) else free_order
    gp = GpuPool(s, order, ws_limits=ws_limits, ws_bytes=ws_bytes)
    handles = {}
    results = {}
    try:
        for idx, op in enumerate(workload.ops):
            kind = op[0]
            if kind == "alloc":
                handles[op[1]] = pkv.seq_allocate(gp.pool)
            elif kind == "fork":
                handles[op[2]] = pkv.seq_fork(gp.pool, handles[op[1]])
            elif kind == "free":
                pkv.seq_free(gp.pool, handles.pop(op[1]))
            elif kind == "append":
                hs, n_tok, key = op[1], op[2], op[3]
                k, v = workload.append_data(key, len(hs), n_tok)
                kd, vd = to_dev(k), to_dev(v)
                pkv.kv_append(gp.pool, [handles[h] for h in hs], n_tok, kd, vd, gp.stream)
            elif kind == "decode":
                hs, layer, key = op[1], op[2], op[3]
                q = to_dev(workload.decode_query(key, len(hs)))
                out = torch.empty((len(hs), s.num_q_heads, s.head_dim), dtype=torch.float32, device="cuda")
                lse = torch.empty((len(hs), s.num_q_heads), dtype=torch.float32, device="cuda")
                pkv.paged_attn_decode(gp.pool, layer, [handles[h] for h in hs], q,
                                      workload.sm_scale, out, lse, gp.stream)
                if want is None or idx in want:
                    results[idx] = (out.cpu().numpy(), lse.cpu().numpy())
            elif kind == "verify":
                hs, layer, n_nodes, key = op[1], op[2], op[3], op[4]
                parents = workload.tree_parents(key, len(hs), n_nodes)
                q = to_dev(workload.verify_query(key, len(hs), n_nodes))
                out = torch.empty((len(hs), n_nodes, s.num_q_heads, s.head_dim),
                                  dtype=torch.float32, device="cuda")
                lse = torch.empty((len(hs), n_nodes, s.num_q_heads), dtype=torch.float32, device="cuda")
                pkv.paged_attn_tree_verify(gp.pool, layer, [handles[h] for h in hs], n_nodes,
                                           parents, q, workload.sm_scale, out, lse, gp.stream)
                if want is None or idx in want:
                    results[idx] = (out.cpu().numpy(), lse.cpu().numpy())
            elif kind == "commit":
                hs, n_nodes, tree_key, path_key = op[1], op[2], op[3], op[4]
                parents = workload.tree_parents(tree_key, len(hs), n_nodes)
                paths = workload.accept_paths(path_key, parents)
                pkv.kv_tree_commit(gp.pool, [handles[h] for h in hs], n_nodes, parents, paths,
                                   gp.stream)
            elif kind == "prefill":
                hs, layer, n_new, key = op[1], op[2], op[3], op[4]
                total = sum(n_new)
                q = to_dev(workload.prefill_query(key, total))
                out = torch.empty((total, s.num_q_heads, s.head_dim), dtype=torch.float32, device="cuda")
                lse = torch.empty((total, s.num_q_heads), dtype=torch.float32, device="cuda")
                pkv.paged_attn_prefill(gp.pool, layer, [handles[h] for h in hs], n_new, q,
                                       workload.sm_scale, out, lse, gp.stream)
                if want is None or idx in want:
                    results[idx] = (out.cpu().numpy(), lse.cpu().numpy())
        torch.cuda.synchronize()
        if pool_cb is not None:
            pool_cb(gp, handles)
    finally:
        gp.close()
    return results
