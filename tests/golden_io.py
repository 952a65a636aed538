"""Reader for the hand-built fixtures under tests/golden/ (see the file header there)."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _expand(tokens):
    out = []
    for t in tokens:
        if "*" in t:
            v, c = t.split("*")
            out.extend([v] * int(c))
        else:
            out.append(t)
    return out


def load_handbuilt(name="q8_0_handbuilt.txt", block_bytes=34):
    """Yield dicts: name, M, K, N, blocks uint8 [M][K/32][block_bytes], x fp16 [N][K],
    y float64 [N][M]. block_bytes is 34 for Q8_0 and 18 for Q4_0."""
    cases, cur = [], None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            if key == "case":
                f_ = rest.split()
                cur = dict(name=f_[0], M=int(f_[2]), K=int(f_[4]), N=int(f_[6]))
                cases.append(cur)
            elif key == "blocks":
                b = np.array([int(t, 16) for t in _expand(rest.split())], np.uint8)
                cur["blocks"] = b.reshape(cur["M"], cur["K"] // 32, block_bytes)
            elif key == "x":
                v = np.array([int(t, 16) for t in _expand(rest.split())], np.uint16)
                cur["x"] = v.view(np.float16).reshape(cur["N"], cur["K"])
            elif key == "y":
                cur["y"] = np.array([float(t) for t in rest.split()], np.float64).reshape(cur["N"], cur["M"])
            elif key == "why":
                cur["why"] = rest
    return cases
