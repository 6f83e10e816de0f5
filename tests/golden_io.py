"""Reader for the text fixtures under tests/golden/ (one record per line,
'#' starts a comment)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def records(name):
    out = []
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                out.append(line.split())
    return out


def keyed(name):
    """First token -> list of remaining tokens (last occurrence wins for
    scalar keys; use records() for repeated keys)."""
    return {r[0]: r[1:] for r in records(name)}
