"""Write p1_relu1.json: the three-token fixture of the datawhalechina chapter "Linear
Attention and Recurrent State" (Step 4, p1_fixture.json) run under that chapter's
positive feature map max(x, 0) + 1 with eps = 0, causal and non-causal, in exact
rational arithmetic through oracle/exact.py.  The chapter prints no outputs for this
fixture, so the values are computed; they are also checked against a derivation by
hand (HAND below) before anything is written.

Run from the repository root:  python tests/golden/make_p1_relu1.py [--check]
(--check compares with the committed file instead of writing it)."""
from __future__ import annotations

import json
import os
import sys
from fractions import Fraction

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from oracle.exact import noncausal_exact, recurrence_exact, relu1_exact  # noqa: E402

OUT = os.path.join(HERE, "p1_relu1.json")

# By hand: q~ = [[2,1],[1.5,3],[4,1]], k~ = [[1,2],[3,1],[2.5,2.5]].  Causal: after t1
# S = [1,2]^T, z = [1,2], y1 = 4/4; after t2 S = [7,4]^T, z = [4,3], y2 = 22.5/15; after t3
# S = [17,14]^T, z = [6.5,5.5], y3 = 82/31.5.  Non-causal (every query reads the final
# state): y = 48/18.5, 67.5/26.25, 82/31.5.
HAND = {"causal_y": ["1", "3/2", "164/63"], "noncausal_y": ["96/37", "18/7", "164/63"],
        "S": ["17", "14"], "z": ["13/2", "11/2"]}


def build() -> dict:
    with open(os.path.join(HERE, "p1_fixture.json"), encoding="utf-8") as f:
        inp = json.load(f)["inputs"]
    qf = [[relu1_exact(Fraction(x)) for x in row] for row in inp["q"]]
    kf = [[relu1_exact(Fraction(x)) for x in row] for row in inp["k"]]
    v = [[Fraction(x) for x in row] for row in inp["v"]]
    ys, Ss, zs, _, _ = recurrence_exact(qf, kf, v, None, 0)
    yn, Sn, zn = noncausal_exact(qf, kf, v, 0)
    S, z = Ss[-1], zs[-1]
    assert [str(y[0]) for y in ys] == HAND["causal_y"] and [str(y[0]) for y in yn] == HAND["noncausal_y"]
    assert [str(row[0]) for row in S] == HAND["S"] and [str(x) for x in z] == HAND["z"]
    assert Sn == S and zn == z
    st = lambda m: [[str(x) for x in row] for row in m]
    return {
        "source": "datawhalechina llm-algo-leetcode ch. 45 \"Linear Attention and Recurrent State\", Step 4: the "
                  "three-token fixture of its tests under its positive feature map max(x,0)+1, state += phi(k) v^T, "
                  "normalizer += phi(k), output = phi(q)^T state / phi(q)^T normalizer, no epsilon",
        "note": "The page prints no outputs for this fixture. Written by tests/golden/make_p1_relu1.py with the exact "
                "rational recurrence of oracle/exact.py, and checked there against a derivation by hand.",
        "phi": "relu1",
        "eps": "0",
        "inputs": inp,
        "causal": {"y": st(ys), "S": st(S), "z": [str(x) for x in z]},
        "noncausal": {"y": st(yn), "S": st(Sn), "z": [str(x) for x in zn]},
    }


if __name__ == "__main__":
    fx = build()
    if "--check" in sys.argv:
        with open(OUT, encoding="utf-8") as f:
            assert json.load(f) == fx, "p1_relu1.json differs from what make_p1_relu1.py computes"
        print("p1_relu1.json matches")
    else:
        with open(OUT, "w", encoding="utf-8") as f:
            json.dump(fx, f, indent=1)
            f.write("\n")
        print("wrote", OUT)
