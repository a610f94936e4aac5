"""Reader for the small text fixtures in this folder."""
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def read_mask_fixture(name):
    """Return (parent list, list of (label, 0/1 row)) from a mask fixture."""
    parent = None
    rows = []
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            label, _, rest = line.partition(":")
            vals = [int(x) for x in rest.split()]
            if label == "parent":
                parent = vals
            else:
                rows.append((label, vals))
    return parent, rows
