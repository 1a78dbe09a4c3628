"""Reader for the hand-derived text fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_fixture(name):
    """Return (header dict of key -> list of tokens, list of blocks) for a fixture.

    Lines starting with '#' are comments.  'key v1 v2 ...' lines become header
    entries; a bare word line (e.g. 'W', 'q') opens a block collecting the
    following rows of tokens until the next bare word.
    """
    head, blocks, cur = {}, {}, None
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.strip()
            if not line or line.startswith("#"):
                continue
            toks = line.split()
            if len(toks) == 1 and not _is_number(toks[0]):
                cur = toks[0]
                blocks[cur] = []
            elif cur is not None and _is_number(toks[0]):
                blocks[cur].append(toks)
            else:
                head[toks[0]] = toks[1:]
                cur = None
    return head, blocks


def _is_number(t):
    try:
        float(t)
        return True
    except ValueError:
        return t.lower().startswith("0x")


def num(t):
    return int(t, 16) if t.lower().startswith("0x") else float(t)
