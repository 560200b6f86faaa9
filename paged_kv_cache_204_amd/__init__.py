"""Python binding of libpkv.so: paged, prefix-sharing KV attention for gfx950.

Argument marshalling only -- every step of the path runs in the C++ host core
and the HIP kernels behind the C ABI declared in ``include/pkv.h``.  The
functions keep the C names.  Device arguments are raw addresses: an ``int``,
``None`` for NULL, or any object with ``data_ptr()`` (a torch tensor, which
must then be contiguous).  ``stream`` is a ``hipStream_t`` address (for torch:
``torch.cuda.current_stream().cuda_stream``); None means the null stream.

Errors raise :class:`PkvError` carrying the C status and message; the pool
is unchanged when that happens.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

__all__ = [
    "PkvError", "PkvDesc", "load", "library_path",
    "kv_pool_bytes", "kv_workspace_bytes", "kv_workspace_layout", "kv_pool_create", "kv_pool_destroy", "kv_pool_q4_bytes", "kv_pool_create_q4",
    "seq_allocate", "seq_fork", "seq_free", "kv_append",
    "paged_attn_decode", "paged_attn_decode_layers", "paged_attn_decode_scratch", "paged_attn_tree_verify", "paged_attn_prefill", "kv_tree_commit",
    "seq_block_table", "block_refcount", "free_list", "kv_last_append",
    "paged_attn_decode_plan_stats", "paged_attn_verify_plan_stats", "paged_attn_prefill_plan_stats",
    "pkv_timing_enable", "pkv_timing_read", "pkv_last_error",
    "pkv_hbm_read_probe",
    "seq_ids",
    "radix_create", "radix_destroy", "radix_match", "radix_insert", "radix_release",
    "radix_evict", "radix_stats", "radix_dump",
    "PKV_OK", "PKV_ERR_ARG", "PKV_ERR_OOM", "PKV_ERR_SEQ", "PKV_ERR_HIP",
    "PKV_ERR_EMPTY", "PKV_ERR_UNSUPPORTED",
]

PKV_OK = 0
PKV_ERR_ARG = -1
PKV_ERR_OOM = -2
PKV_ERR_SEQ = -3
PKV_ERR_HIP = -4
PKV_ERR_EMPTY = -5
PKV_ERR_UNSUPPORTED = -6

_NAMES = {0: "PKV_OK", -1: "PKV_ERR_ARG", -2: "PKV_ERR_OOM", -3: "PKV_ERR_SEQ",
          -4: "PKV_ERR_HIP", -5: "PKV_ERR_EMPTY", -6: "PKV_ERR_UNSUPPORTED"}

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_HERE, "libpkv.so")


class PkvError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"{_NAMES.get(code, code)}: {message}")
        self.code = code
        self.message = message


class PkvDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_layers", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32)]


class PkvPlanStats(ctypes.Structure):
    _fields_ = [("unique_tokens", ctypes.c_int64), ("logical_tokens", ctypes.c_int64),
                ("unique_blocks", ctypes.c_int32), ("segments", ctypes.c_int32),
                ("work_items", ctypes.c_int32), ("merged_rows", ctypes.c_int32),
                ("direct", ctypes.c_int32), ("max_parts", ctypes.c_int32),
                ("plan_bytes", ctypes.c_int64), ("partial_bytes", ctypes.c_int64)]


class PkvWorkspace(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("bytes", ctypes.c_size_t),
                ("max_seqs", ctypes.c_int32), ("max_tree_nodes", ctypes.c_int32)]


_lib = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_PI32 = ctypes.POINTER(ctypes.c_int32)
_PI64 = ctypes.POINTER(ctypes.c_int64)


def load():
    """Load the built library (never builds; raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is not built; run __graft_entry__.build() or "
            "python paged_kv_cache_204_amd/build.py")
    lib = ctypes.CDLL(path)
    sig = {
        "kv_pool_bytes": (ctypes.c_size_t, [ctypes.POINTER(PkvDesc)]),
        "kv_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(PkvDesc), _I32, _I32]),
        "kv_workspace_layout": (_I32, [ctypes.POINTER(PkvDesc), _I32, _I32, ctypes.POINTER(ctypes.c_size_t)]),
        "kv_pool_create": (_I32, [ctypes.POINTER(PkvDesc), _P, _P, ctypes.POINTER(PkvWorkspace), _PI32,
                                  ctypes.POINTER(_P)]),
        "kv_pool_destroy": (None, [_P]),
        "kv_pool_q4_bytes": (ctypes.c_size_t, [ctypes.POINTER(PkvDesc), ctypes.POINTER(ctypes.c_size_t)]),
        "kv_pool_create_q4": (_I32, [ctypes.POINTER(PkvDesc), _P, _P, _P, _P,
                                     ctypes.POINTER(ctypes.c_int8), _PI32, ctypes.POINTER(_P)]),
        "seq_allocate": (_I32, [_P, _PI64]),
        "seq_fork": (_I32, [_P, _I64, _PI64]),
        "seq_free": (_I32, [_P, _I64]),
        "kv_append": (_I32, [_P, _PI64, _I32, _I32, _P, _P, _P]),
        "paged_attn_decode": (_I32, [_P, _I32, _PI64, _I32, _P, ctypes.c_float, _P, _P, _P]),
        "paged_attn_decode_scratch": (_I32, [_P, _I32, _PI64, _I32, _P, ctypes.c_float, _P, _P, _P]),
        "paged_attn_decode_layers": (_I32, [_P, _I32, _I32, _PI64, _I32, _P, ctypes.c_float, _P, _P, _P]),
        "paged_attn_tree_verify": (_I32, [_P, _I32, _PI64, _I32, _I32, _PI32, _P,
                                          ctypes.c_float, _P, _P, _P]),
        "paged_attn_prefill": (_I32, [_P, _I32, _PI64, _I32, _PI32, _P, ctypes.c_float, _P, _P,
                                      _P]),
        "kv_tree_commit": (_I32, [_P, _PI64, _I32, _I32, _PI32, _PI32, _PI32, _P]),
        "seq_block_table": (_I32, [_P, _I64, _PI32, _I32, _PI32, _PI32]),
        "block_refcount": (_I32, [_P, _I32, _PI32]),
        "free_list": (_I32, [_P, _PI32, _I32, _PI32]),
        "kv_last_append": (_I32, [_P, _PI32, _I32, _PI32, _PI32, _I32, _PI32]),
        "paged_attn_decode_plan_stats": (_I32, [_P, _PI64, _I32, ctypes.POINTER(PkvPlanStats)]),
        "paged_attn_verify_plan_stats": (_I32, [_P, _PI64, _I32, _I32, _PI32, ctypes.POINTER(PkvPlanStats)]),
        "paged_attn_prefill_plan_stats": (_I32, [_P, _PI64, _I32, _PI32, ctypes.POINTER(PkvPlanStats)]),
        "pkv_timing_enable": (_I32, [_P, _I32]),
        "pkv_timing_read": (_I32, [_P, ctypes.POINTER(ctypes.c_double), _PI64, _I32]),
        "pkv_last_error": (ctypes.c_char_p, []),
        "pkv_hbm_read_probe": (_I32, [_P, ctypes.c_size_t, _P, _I32, _P]),
        "radix_create": (_I32, [_P, ctypes.POINTER(_P)]),
        "radix_destroy": (None, [_P]),
        "radix_match": (_I32, [_P, _PI32, _I32, _PI64, _PI32]),
        "radix_insert": (_I32, [_P, _I64, _PI32, _I32]),
        "radix_release": (_I32, [_P, _I64]),
        "radix_evict": (_I32, [_P, _I32, _PI32]),
        "radix_stats": (_I32, [_P, _PI32, _PI32, _PI32]),
        "radix_dump": (_I32, [_P, _PI32, _I32, _PI32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(code):
    if code != PKV_OK:
        raise PkvError(code, load().pkv_last_error().decode())


def _addr(x):
    if x is None:
        return None
    if type(x) is int:
        return x or None
    dp = getattr(x, "data_ptr", None)
    if dp is not None:
        contiguous = getattr(x, "is_contiguous", None)
        if contiguous is not None and not contiguous():
            raise ValueError("device arguments must be contiguous")
        return dp()
    if isinstance(x, int):
        return x or None
    raise TypeError(f"cannot take a device address from {type(x).__name__}")


def _stream(s):
    if s is None:
        return None
    if isinstance(s, int):
        return s or None
    if hasattr(s, "cuda_stream"):
        return s.cuda_stream or None
    raise TypeError("stream must be an int address or have .cuda_stream")


_SEQ_TYPES = {}


def seq_ids(seqs):
    """A ctypes int64 array of sequence ids: pass it to the per-step calls in
    place of a list to skip the conversion on every call."""
    return (ctypes.c_int64 * len(seqs))(*seqs)


def _seq_array(seqs):
    """(pointer argument, length) for a sequence-id argument: ctypes int64
    arrays (see seq_ids) pass through, lists and tuples become one, anything
    else goes through numpy."""
    if isinstance(seqs, ctypes.Array):
        if seqs._type_ is not ctypes.c_int64:
            raise TypeError("sequence ids must be int64")
        return seqs, len(seqs)
    if type(seqs) is list or type(seqs) is tuple:
        n = len(seqs)
        t = _SEQ_TYPES.get(n)
        if t is None:
            t = _SEQ_TYPES[n] = ctypes.c_int64 * n
        return t(*seqs), n
    a = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64).reshape(-1))
    return a.ctypes.data_as(_PI64), a.size


def _desc(desc):
    if isinstance(desc, PkvDesc):
        return desc
    if isinstance(desc, dict):
        return PkvDesc(**desc)
    return PkvDesc(desc.num_blocks, desc.block_size, desc.num_layers,
                   desc.num_q_heads, desc.num_kv_heads, desc.head_dim)


# ------------------------------------------------------------------- calls

def kv_pool_bytes(desc) -> int:
    d = _desc(desc)
    return load().kv_pool_bytes(ctypes.byref(d))


def kv_workspace_bytes(desc, max_seqs, max_tree_nodes) -> int:
    """Device bytes of workspace for calls of at most max_seqs sequences and
    max_tree_nodes query tokens per sequence (0 for invalid arguments)."""
    return int(load().kv_workspace_bytes(ctypes.byref(_desc(desc)), int(max_seqs), int(max_tree_nodes)))


def kv_workspace_layout(desc, max_seqs, max_tree_nodes) -> dict:
    """Bytes of each workspace region: decode, verify, prefill work lists and partial states."""
    r = (ctypes.c_size_t * 4)()
    _check(load().kv_workspace_layout(ctypes.byref(_desc(desc)), int(max_seqs), int(max_tree_nodes), r))
    return dict(zip(("decode", "verify", "prefill", "partials"), (int(x) for x in r)))


def kv_pool_create(desc, k_pool=None, v_pool=None, free_order=None, workspace=None, workspace_bytes=None,
                   max_seqs=0, max_tree_nodes=0):
    """workspace: a device buffer (tensor or address) the pool carves its
    work lists and partial states from, of workspace_bytes bytes (default:
    the tensor's size); None: the pool manages its own."""
    d = _desc(desc)
    fo = None
    keep = None
    if free_order is not None:
        keep = np.ascontiguousarray(np.asarray(free_order, dtype=np.int32))
        fo = keep.ctypes.data_as(_PI32)
    ws = None
    if workspace is not None or max_seqs or max_tree_nodes:
        nbytes = workspace_bytes
        if nbytes is None and workspace is not None:
            nbytes = workspace.numel() * workspace.element_size()
        ws = PkvWorkspace(_addr(workspace), int(nbytes or 0), int(max_seqs), int(max_tree_nodes))
    out = _P()
    _check(load().kv_pool_create(ctypes.byref(d), _addr(k_pool), _addr(v_pool),
                                 ctypes.byref(ws) if ws is not None else None, fo, ctypes.byref(out)))
    return out


def kv_pool_q4_bytes(desc):
    """(bytes of one codes array, bytes of one norms array) of a 4-bit pool."""
    nb = ctypes.c_size_t()
    codes = load().kv_pool_q4_bytes(ctypes.byref(_desc(desc)), ctypes.byref(nb))
    return codes, nb.value


def kv_pool_create_q4(desc, k_codes, v_codes, k_norms, v_norms, signs, free_order=None):
    d = _desc(desc)
    sg = np.ascontiguousarray(np.asarray(signs, dtype=np.int8).reshape(-1))
    if sg.size != d.head_dim:
        raise ValueError("one sign per head dimension")
    fo = None
    keep = None
    if free_order is not None:
        keep = np.ascontiguousarray(np.asarray(free_order, dtype=np.int32))
        fo = keep.ctypes.data_as(_PI32)
    out = _P()
    _check(load().kv_pool_create_q4(ctypes.byref(d), _addr(k_codes), _addr(v_codes), _addr(k_norms),
                                    _addr(v_norms), sg.ctypes.data_as(ctypes.POINTER(ctypes.c_int8)),
                                    fo, ctypes.byref(out)))
    return out


def kv_pool_destroy(pool):
    load().kv_pool_destroy(pool)


def seq_allocate(pool) -> int:
    out = _I64()
    _check(load().seq_allocate(pool, ctypes.byref(out)))
    return out.value


def seq_fork(pool, parent) -> int:
    out = _I64()
    _check(load().seq_fork(pool, int(parent), ctypes.byref(out)))
    return out.value


def seq_free(pool, seq):
    _check(load().seq_free(pool, int(seq)))


def kv_append(pool, seqs, n_tok, k_new=None, v_new=None, stream=None):
    p, n = _seq_array(seqs)
    _check(load().kv_append(pool, p, n, int(n_tok), _addr(k_new), _addr(v_new),
                            _stream(stream)))


def paged_attn_decode(pool, layer, seqs, q, sm_scale, out, lse=None, stream=None):
    p, n = _seq_array(seqs)
    code = (_lib or load()).paged_attn_decode(pool, int(layer), p, n, _addr(q), float(sm_scale),
                                              _addr(out), _addr(lse), _stream(stream))
    if code != PKV_OK:
        _check(code)


def paged_attn_decode_layers(pool, layer0, n_layers, seqs, q, sm_scale, out, lse=None, stream=None):
    """Decode over layers layer0 .. layer0 + n_layers - 1 in one call: q
    [n_layers][n][Hq][D] bf16, out [n_layers][n][Hq][D], lse [n_layers][n][Hq]."""
    p, n = _seq_array(seqs)
    _check(load().paged_attn_decode_layers(pool, int(layer0), int(n_layers), p, n, _addr(q), float(sm_scale),
                                           _addr(out), _addr(lse), _stream(stream)))


def paged_attn_decode_scratch(pool, layer, seqs, q, sm_scale, out, lse=None, stream=None):
    """paged_attn_decode with its work lists and partial states in the
    library's static device array (no device allocation)."""
    p, n = _seq_array(seqs)
    _check(load().paged_attn_decode_scratch(pool, int(layer), p, n, _addr(q), float(sm_scale),
                                            _addr(out), _addr(lse), _stream(stream)))


def paged_attn_tree_verify(pool, layer, seqs, n_nodes, parent, q, sm_scale, out, lse=None,
                           stream=None):
    p, n = _seq_array(seqs)
    par = np.ascontiguousarray(np.asarray(parent, dtype=np.int32))
    if par.size != n * int(n_nodes):
        raise ValueError("parent must hold n_seqs * n_nodes entries")
    _check(load().paged_attn_tree_verify(pool, int(layer), p, n, int(n_nodes),
                                         par.ctypes.data_as(_PI32), _addr(q), float(sm_scale),
                                         _addr(out), _addr(lse), _stream(stream)))


def paged_attn_prefill(pool, layer, seqs, n_new, q, sm_scale, out, lse=None, stream=None):
    p, n = _seq_array(seqs)
    nn = np.ascontiguousarray(np.asarray(n_new, dtype=np.int32).reshape(-1))
    if nn.size != n:
        raise ValueError("n_new must hold one count per sequence")
    _check(load().paged_attn_prefill(pool, int(layer), p, n, nn.ctypes.data_as(_PI32), _addr(q),
                                     float(sm_scale), _addr(out), _addr(lse), _stream(stream)))


def kv_tree_commit(pool, seqs, n_nodes, parent, paths, stream=None):
    """paths: one list of accepted nodes (root first) per sequence."""
    p, n = _seq_array(seqs)
    par = np.ascontiguousarray(np.asarray(parent, dtype=np.int32).reshape(-1))
    if par.size != n * int(n_nodes):
        raise ValueError("parent must hold n_seqs * n_nodes entries")
    if len(paths) != n:
        raise ValueError("one path per sequence")
    plen = np.asarray([len(x) for x in paths], dtype=np.int32)
    pad = np.zeros((max(n, 1), int(n_nodes)), dtype=np.int32)
    for i, x in enumerate(paths):
        if len(x) > n_nodes:
            raise ValueError("a path longer than the tree")
        pad[i, :len(x)] = x
    _check(load().kv_tree_commit(pool, p, n, int(n_nodes), par.ctypes.data_as(_PI32),
                                 plen.ctypes.data_as(_PI32), pad.ctypes.data_as(_PI32),
                                 _stream(stream)))


def seq_block_table(pool, seq):
    n = _I32()
    ln = _I32()
    _check(load().seq_block_table(pool, int(seq), None, 0, ctypes.byref(n), ctypes.byref(ln)))
    buf = (ctypes.c_int32 * max(1, n.value))()
    _check(load().seq_block_table(pool, int(seq), buf, n.value, ctypes.byref(n), ctypes.byref(ln)))
    return list(buf[:n.value]), ln.value


def block_refcount(pool, block) -> int:
    rc = _I32()
    _check(load().block_refcount(pool, int(block), ctypes.byref(rc)))
    return rc.value


def free_list(pool):
    n = _I32()
    _check(load().free_list(pool, None, 0, ctypes.byref(n)))
    buf = (ctypes.c_int32 * max(1, n.value))()
    _check(load().free_list(pool, buf, n.value, ctypes.byref(n)))
    return list(buf[:n.value])


def kv_last_append(pool):
    ns = _I32()
    nc = _I32()
    _check(load().kv_last_append(pool, None, 0, ctypes.byref(ns), None, 0, ctypes.byref(nc)))
    sb = (ctypes.c_int32 * max(1, ns.value))()
    cb = (ctypes.c_int32 * max(1, 3 * nc.value))()
    _check(load().kv_last_append(pool, sb, ns.value, ctypes.byref(ns), cb, 3 * nc.value,
                                 ctypes.byref(nc)))
    cow = [tuple(cb[3 * i:3 * i + 3]) for i in range(nc.value)]
    return list(sb[:ns.value]), cow


def paged_attn_decode_plan_stats(pool, seqs) -> dict:
    p, n = _seq_array(seqs)
    st = PkvPlanStats()
    _check(load().paged_attn_decode_plan_stats(pool, p, n, ctypes.byref(st)))
    return {f: getattr(st, f) for f, _ in PkvPlanStats._fields_}


def paged_attn_verify_plan_stats(pool, seqs, n_nodes, parents) -> dict:
    p, n = _seq_array(seqs)
    par = np.ascontiguousarray(np.asarray(parents, dtype=np.int32).reshape(-1))
    st = PkvPlanStats()
    _check(load().paged_attn_verify_plan_stats(pool, p, n, int(n_nodes), par.ctypes.data_as(_PI32),
                                               ctypes.byref(st)))
    return {f: getattr(st, f) for f, _ in PkvPlanStats._fields_}


def paged_attn_prefill_plan_stats(pool, seqs, n_new) -> dict:
    p, n = _seq_array(seqs)
    nn = np.ascontiguousarray(np.asarray(n_new, dtype=np.int32).reshape(-1))
    st = PkvPlanStats()
    _check(load().paged_attn_prefill_plan_stats(pool, p, n, nn.ctypes.data_as(_PI32), ctypes.byref(st)))
    return {f: getattr(st, f) for f, _ in PkvPlanStats._fields_}


def pkv_timing_enable(pool, enable=True):
    """enable: True (every call), False (off) or a sampling period n > 0."""
    if enable is True or enable is False:
        enable = 1 if enable else 0
    _check(load().pkv_timing_enable(pool, int(enable)))


def pkv_timing_read(pool, reset=True):
    """(summed attention-kernel milliseconds, bracketed calls)."""
    ms = ctypes.c_double()
    n = _I64()
    _check(load().pkv_timing_read(pool, ctypes.byref(ms), ctypes.byref(n), 1 if reset else 0))
    return ms.value, n.value


def pkv_last_error() -> str:
    return load().pkv_last_error().decode()


def pkv_hbm_read_probe(src, nbytes, sink, blocks, stream=None):
    _check(load().pkv_hbm_read_probe(_addr(src), int(nbytes), _addr(sink), int(blocks), _stream(stream)))


# ---- radix prefix cache ---------------------------------------------------

def _tokens(tokens):
    t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32).reshape(-1))
    return t, t.ctypes.data_as(_PI32), t.size


def radix_create(pool):
    out = _P()
    _check(load().radix_create(pool, ctypes.byref(out)))
    return out.value


def radix_destroy(cache):
    if cache:
        load().radix_destroy(cache)


def radix_match(cache, tokens):
    """(new sequence id, matched token count)."""
    t, p, n = _tokens(tokens)
    seq = _I64()
    m = _I32()
    _check(load().radix_match(cache, p, n, ctypes.byref(seq), ctypes.byref(m)))
    return seq.value, m.value


def radix_insert(cache, seq, tokens):
    t, p, n = _tokens(tokens)
    _check(load().radix_insert(cache, int(seq), p, n))


def radix_release(cache, seq):
    _check(load().radix_release(cache, int(seq)))


def radix_evict(cache, want_free):
    """Free-list length afterwards; raises PkvError (PKV_ERR_OOM) when the
    target cannot be reached."""
    n = _I32()
    _check(load().radix_evict(cache, int(want_free), ctypes.byref(n)))
    return n.value


def radix_stats(cache):
    a, b, c = _I32(), _I32(), _I32()
    _check(load().radix_stats(cache, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    return {"nodes": a.value, "cached_blocks": b.value, "locked_nodes": c.value}


def radix_dump(cache, block_size):
    """The tree as a list of (depth, tokens, lock, blocks) in preorder."""
    n = _I32()
    _check(load().radix_dump(cache, None, 0, ctypes.byref(n)))
    buf = (ctypes.c_int32 * max(1, n.value))()
    _check(load().radix_dump(cache, buf, n.value, ctypes.byref(n)))
    flat = list(buf[:n.value])
    out = []
    i = 0
    while i < len(flat):
        depth, t, lock = flat[i], flat[i + 1], flat[i + 2]
        toks = flat[i + 3:i + 3 + t]
        blocks = flat[i + 3 + t:i + 3 + t + t // block_size]
        out.append((depth, toks, lock, blocks))
        i += 3 + t + t // block_size
    return out
