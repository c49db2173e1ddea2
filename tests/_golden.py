"""Reader for the hand-derived fixtures in ``tests/golden`` (records separated by ``name:``)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(fname):
    records, cur = [], None
    with open(os.path.join(GOLDEN, fname)) as f:
        for raw in f:
            line = raw.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            key, val = key.strip(), val.strip()
            if key == "name":
                cur = {"name": val}
                records.append(cur)
            else:
                cur[key] = val
    return records


def hexbytes(s):
    return bytes(int(t, 16) for t in s.split())


def pairs(s, conv=float):
    out = {}
    for tok in s.split():
        k, v = tok.split(":")
        out[int(k)] = conv(v)
    return out
