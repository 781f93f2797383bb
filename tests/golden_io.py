"""Readers for the text fixtures under tests/golden/ (no arithmetic of the method)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield [p.strip() for p in line.split(":", 2)]


def shard_cases(name="shard_lists.txt"):
    """(q_heads, kv_heads, sp, expected list or None for a rejection, source)."""
    out = []
    for key, val, src in _rows(name):
        q, kv, sp = (int(v) for v in key.split())
        exp = None if val == "REJECT" else [int(v) for v in val.split()]
        out.append((q, kv, sp, exp, src))
    return out


def head_id_cases():
    out = []
    for key, val, src in _rows("shard_head_ids.txt"):
        q, kv, sp = (int(v) for v in key.split())
        ids = [[int(v) for v in grp.split()] for grp in val.split("|")]
        out.append((q, kv, sp, ids, src))
    return out


def exchange_shape_cases():
    out = []
    for key, val, src in _rows("exchange_shapes.txt"):
        heads, sp, batch, tokens, dim = (int(v) for v in key.split())
        shapes = [tuple(int(v) for v in grp.split()) for grp in val.split("|")]
        out.append((heads, sp, batch, tokens, dim, shapes, src))
    return out
