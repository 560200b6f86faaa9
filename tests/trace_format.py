"""Parser for the hand-derived pool trace fixtures under ``tests/golden``."""

import os
import re

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def parse_trace(name):
    """Return ``[(op_tokens, [expect_lines])]`` from a trace fixture."""
    steps = []
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            if line.startswith("op "):
                steps.append((line.split()[1:], []))
            else:
                steps[-1][1].append(line)
    return steps


def parse_table(text):
    return [int(x) for x in re.findall(r"-?\d+", text)]


def check_expectations(lines, *, table, length, live, rc_all, fifo, slots=None,
                       cow=None, label=""):
    """Check one step's expectation lines against an observed pool state.

    ``table(name)``/``length(name)`` read a sequence by its trace name,
    ``live`` is the set of live trace names, ``rc_all`` the full refcount
    list, ``fifo`` the free list, ``slots`` the ``(block, off)`` list of the
    step's append and ``cow`` its ``(src, dst, n)`` list (None when the
    implementation under test does not report them).
    """
    for e in lines:
        kind, _, rest = e.partition(" ")
        if kind == "seq":
            m = re.match(r"(\S+)\s+\[([^\]]*)\]\s+(\d+)", rest)
            name, tbl, ln = m.group(1), parse_table(m.group(2)), int(m.group(3))
            assert table(name) == tbl, f"{label}: table of {name}"
            assert length(name) == ln, f"{label}: len of {name}"
        elif kind == "live":
            assert set(live) == set(rest.split()), f"{label}: live set"
        elif kind == "rc":
            want = {}
            for tok in rest.split():
                b, c = tok.split(":")
                want[int(b)] = int(c)
            got = {b: c for b, c in enumerate(rc_all) if c}
            assert got == want, f"{label}: refcounts {got} != {want}"
        elif kind == "fifo":
            assert list(fifo) == [int(x) for x in rest.split()], f"{label}: free list"
        elif kind == "slots":
            if slots is None:
                continue
            toks = rest.split()[1:]
            want = [tuple(int(x) for x in t.split(":")) for t in toks]
            assert [tuple(s) for s in slots] == want, f"{label}: slots"
        elif kind == "cow":
            if cow is None:
                continue
            want = []
            for t in rest.split():
                src, tail = t.split(">")
                dst, n = tail.split(":")
                want.append((int(src), int(dst), int(n)))
            assert [tuple(c) for c in cow] == want, f"{label}: copy-on-write"
        else:
            raise ValueError(f"unknown trace line {e!r}")
