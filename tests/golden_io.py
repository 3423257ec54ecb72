"""Reader for the worked-example fixtures under tests/golden/ (``key: v1 v2 ...``)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, vals = line.split(":", 1)
            nums = [int(v, 16) if v.startswith("0x") else float(v) for v in vals.split()]
            out[key.strip()] = nums[0] if len(nums) == 1 else nums
    return out
