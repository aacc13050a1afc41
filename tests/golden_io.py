"""Reader for the hand-derived fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _num(tok):
    tok = tok.strip()
    if tok.lower().startswith("0x") or tok.lower().startswith("-0x"):
        return int(tok, 16)
    if tok == "nan":
        return float("nan")
    return float(tok)


def rows(name):
    """Non-comment lines of a fixture, split into tokens."""
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                out.append(line.split())
    return out


def tagged(name):
    """{tag: {index: [values]}} for fixtures written as 'tag index v0 v1 ...'."""
    d = {}
    for toks in rows(name):
        tag = toks[0]
        if len(toks) == 2:
            d[tag] = _num(toks[1])
            continue
        d.setdefault(tag, {})[int(toks[1])] = [_num(t) for t in toks[2:]]
    return d


def table(name):
    return [[_num(t) for t in toks] for toks in rows(name)]
