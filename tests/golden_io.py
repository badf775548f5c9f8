"""Readers for the cited text fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for ln in f:
            ln = ln.strip()
            if ln and not ln.startswith("#"):
                yield ln


def params(name):
    out = {}
    for ln in lines(name):
        k, v = ln.split(None, 1)
        out[k] = v
    return out


def e2m1_table():
    """[(code 0..7, value, kind)] from the page's E2M1 table."""
    rows = []
    for ln in lines("e2m1_table.txt"):
        s, ee, m, val, kind = ln.split()
        code = int(s + ee + m, 2)
        rows.append((code, float(val), kind))
    return rows
