"""Parser for the hand-worked fixtures under tests/golden/."""
import os

import numpy as np

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rows(lines, n):
    out = []
    for _ in range(n):
        out.append([float(v) for v in lines.pop(0).split()])
    return np.array(out, dtype=np.float32)


def load_cases(fname):
    with open(os.path.join(GOLDEN_DIR, fname)) as f:
        lines = [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]
    cases = []
    while lines:
        head = lines.pop(0)
        assert head.startswith("case "), head
        name = head.split(None, 1)[1]
        M, N, K = (int(v) for v in lines.pop(0).split(":")[1].split())
        alpha, beta = (float(v) for v in lines.pop(0).split(":")[1].split())
        ta = tb = 0
        if lines[0].startswith("trans:"):
            ta, tb = (int(v) for v in lines.pop(0).split(":")[1].split())
        assert lines.pop(0) == "A:"
        A = _rows(lines, K if ta else M)
        assert lines.pop(0) == "B:"
        B = _rows(lines, N if tb else K)
        c0h = lines.pop(0)
        C0 = None
        if c0h != "C0: none":
            assert c0h == "C0:"
            C0 = _rows(lines, M)
        assert lines.pop(0) == "C:"
        C = _rows(lines, M).astype(np.float64)
        assert lines.pop(0) == "end"
        cases.append(dict(name=name, M=M, N=N, K=K, alpha=alpha, beta=beta,
                          A=A, B=B, C0=C0, C=C, trans_a=bool(ta), trans_b=bool(tb)))
    return cases
