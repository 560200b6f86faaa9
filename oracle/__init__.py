"""CPU oracle for paged, prefix-sharing KV attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import or run anything here.  The
product path (the C ABI library and its Python binding) never does, and this
package imports nothing from the product.  It shares no code with the HIP
path; the only common input is the seeded generator package ``synth``.

Contents:

* :mod:`oracle.pool` -- a plain Python model of the refcounted block pool:
  free list, per-sequence block tables, fork, append with copy-on-write,
  free.  It also keeps its own copy of every block's K/V bits.
* :mod:`oracle.attention` -- textbook softmax attention in float64 over each
  sequence's keys, gathered token by token through its block table; decode
  (one query per sequence), draft-tree verify (context plus tree
  ancestors and the node itself) and causal prefill of a sequence's newest
  tokens over its whole cache.
* :mod:`oracle.quant` -- 4-bit K/V codes (rotation, Lloyd-Max levels, fp16
  norm) and decode attention over them.
* :mod:`oracle.radix` -- a block-paged radix-tree prefix cache over the pool
  model: match, split-on-insert, release, leaf-first LRU eviction.
* :mod:`oracle.run` -- runs a ``synth`` op program through the two.

Every function here is pinned by the ``-m "not gpu"`` tests against facts the
pages or plain mathematics fix (hand-derived pool trace, closed forms,
invariants, a library attention routine, numbers the pages print); none is
"parity unpinned".
"""

from .pool import PoolModel, PoolError, OOMError, SeqError, ArgError, EmptyError
from .attention import bf16_bits_to_f64, attend, decode, prefill, tree_verify, tree_key_positions
from .radix import RadixModel
from .run import run_program

__all__ = [
    "PoolModel",
    "PoolError",
    "OOMError",
    "SeqError",
    "ArgError",
    "EmptyError",
    "bf16_bits_to_f64",
    "attend",
    "decode",
    "prefill",
    "tree_verify",
    "tree_key_positions",
    "run_program",
    "RadixModel",
]
