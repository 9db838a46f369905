"""Readers for the text fixtures under tests/golden (comments start with '#')."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rows(name):
    out = []
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                out.append(line.split())
    return out


def keyed(name):
    return {r[0]: r[1:] for r in rows(name)}
