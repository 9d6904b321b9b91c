"""Reader for the hand-worked fixtures in tests/golden/hand_examples.txt."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_examples.txt")


def load_cases(path=GOLDEN):
    cases, cur = [], None
    with open(path) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            if line.startswith("case "):
                cur = {"name": line[5:].strip()}
                cases.append(cur)
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            cur[key] = [float(v) for v in val.split()]
    out = []
    for c in cases:
        T, Cp, Dp, N = (int(v) for v in c["shape"])
        case = {"name": c["name"], "T": T, "Cp": Cp, "Dp": Dp, "N": N,
                "x": np.array(c["x"]).reshape(N, Cp * T),
                "w": np.array(c["w"]).reshape(Dp, Cp, T),
                "y": np.array(c["y"]).reshape(N, Dp * T)}
        if "dy" in c:
            case["dy"] = np.array(c["dy"]).reshape(N, Dp * T)
        if "dx" in c:
            case["dx"] = np.array(c["dx"]).reshape(N, Cp * T)
        if "dw" in c:
            case["dw"] = np.array(c["dw"]).reshape(Dp, Cp, T)
        out.append(case)
    return out
