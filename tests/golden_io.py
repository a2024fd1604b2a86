"""Reader for the hand-worked fixtures under tests/golden/.

A fixture is plain text: '#' lines are comments (they carry the citation
and the hand working), 'case NAME' starts a new case, and every other line
is 'key value value ...'.  Hex tokens (0x..) are read as integers.
"""

import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _tok(s):
    if s.lower().startswith(("0x", "-0x")):
        return int(s, 16)
    try:
        return int(s)
    except ValueError:
        pass
    try:
        return float(s)
    except ValueError:
        return s


def read_cases(name):
    cases, cur = [], None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            if key == "case":
                cur = {"name": vals[0]}
                cases.append(cur)
                continue
            if cur is None:
                cur = {"name": name}
                cases.append(cur)
            cur[key] = [_tok(v) for v in vals]
    return cases
