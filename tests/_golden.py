"""Reader for the hand-worked fixtures in tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def lines(name):
    """Non-comment lines of a fixture, split into whitespace fields."""
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for ln in f:
            ln = ln.split("#", 1)[0].strip()
            if ln:
                out.append(ln.split())
    return out


def table(name):
    """Fixture as {key: [fields...]} (first field is the key)."""
    return {f[0]: f[1:] for f in lines(name)}
