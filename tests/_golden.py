"""Reader of the hand-written golden plan fixtures in tests/golden/."""

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _expand(tok):
    if "*" in tok:
        v, n = tok.split("*")
        return [_num(v)] * int(n)
    if ".." in tok:
        a, b = tok.split("..")
        return list(range(_num(a), _num(b) + 1))
    return [_num(tok)]


def _num(t):
    return int(t, 16) if t.lower().startswith("0x") else int(t)


def read_plan_fixture(name):
    """Return dict(lens, qseq, qpos, table, page_size, pages, words)."""
    fields, cur = {}, None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].rstrip()
            if not line.strip():
                continue
            if not line[0].isspace() and ":" in line:
                cur, rest = line.split(":", 1)
                fields[cur] = rest
            else:
                fields[cur] += " " + line
    out = {}
    for key in ("lens", "qseq", "qpos", "words"):
        out[key] = [x for tok in fields[key].split() for x in _expand(tok)]
    rows = [[x for tok in r.split() for x in _expand(tok)] for r in fields["table"].split("/")]
    out["table"] = np.array(rows, dtype=np.int64)
    out["page_size"] = _num(fields["page_size"].strip())
    out["pages"] = _num(fields["pages"].strip())
    out["words"] = np.array(out["words"], dtype=np.uint32)
    return out


FIXTURES = sorted(f for f in os.listdir(GOLDEN) if f.startswith("plan_"))


def read_append_fixture(name):
    """Return dict(lens, qseq, qpos, table, page_size, pages, targets)."""
    fields, cur = {}, None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].rstrip()
            if not line.strip():
                continue
            cur, rest = line.split(":", 1)
            fields[cur] = rest
    out = {key: [x for tok in fields[key].split() for x in _expand(tok)]
           for key in ("lens", "qseq", "qpos")}
    out["table"] = np.array([[x for tok in r.split() for x in _expand(tok)]
                             for r in fields["table"].split("/")], dtype=np.int64)
    out["page_size"] = int(fields["page_size"])
    out["pages"] = int(fields["pages"])
    out["targets"] = [tuple(int(x) for x in t.split(":")) for t in fields["targets"].split()]
    return out
