"""Readers for the hand-derived fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rows(fname):
    with open(os.path.join(GOLDEN, fname)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            yield [c.strip() for c in line.split("|")]


def quantize_worked():
    out = []
    for name, qtype, qmax, xs, scale, codes in _rows("quantize_worked.txt"):
        out.append(dict(name=name, qtype=qtype, qmax=float(qmax),
                        x=[float(v) for v in xs.split()], scale=float(scale),
                        codes=[int(c, 16) for c in codes.split()]))
    return out


def gemm_worked():
    out = []
    for (name, qtype, xs, ws, sx, sw, xc, wc, dot, y, ybits) in _rows("gemm_worked.txt"):
        out.append(dict(name=name, qtype=qtype, x=[float(v) for v in xs.split()],
                        w=[float(v) for v in ws.split()], sx=float(sx), sw=float(sw),
                        xcodes=[int(c, 16) for c in xc.split()],
                        wcodes=[int(c, 16) for c in wc.split()], dot=float(dot), y=float(y),
                        ybits=int(ybits, 16)))
    return out
