"""Reader for the hand-worked block fixtures in tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _assignments(field):
    out = {}
    field = field.strip()
    if not field:
        return out
    for item in field.split(","):
        pos, val = item.split("=")
        out[pos.strip()] = int(val.strip(), 16)
    return out


def _expand(assign):
    vals = [assign["*"]] * 32 if "*" in assign else [0] * 32
    for k, v in assign.items():
        if k != "*":
            vals[int(k)] = v
    return vals


def hand_blocks():
    """[(name, bf16 bits[32], scale byte, codes[32])] from hand_blocks.txt."""
    rows = []
    with open(os.path.join(GOLDEN, "hand_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, inputs, scale, codes = [p.strip() for p in line.split(";")]
            rows.append((name, _expand(_assignments(inputs)), int(scale, 16), _expand(_assignments(codes))))
    return rows
