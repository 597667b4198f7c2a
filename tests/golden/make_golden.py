"""Writes the stored expected values under tests/golden/.

It calls only the oracle package (its 50-digit mpmath brute force), never the
HIP library. Run from the repository root:  python tests/golden/make_golden.py

The pages print no numeric value of the WKV output anywhere, so every fixture
here is a small worked case of the defining equation (page "Linear attention
without writing a CUDA kernel", section "The recurrence", the wkv_t equation),
evaluated term by term at 50 digits. The tests also re-derive each one by a
hand-written closed form, so a fixture and the brute force check each other.
"""

from __future__ import annotations

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle.wkv_brute import wkv_brute  # noqa: E402

CITATION = ('page "Linear attention without writing a CUDA kernel", section '
            '"The recurrence", the wkv_t equation (evaluated at 50 digits by '
            'oracle/wkv_brute.py; the pages print no worked numbers)')


def case(name, w, u, k, v, state_in=None, note=""):
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, T, C = k.shape
    out, st = wkv_brute(np.asarray(w, float), np.asarray(u, float), k, v, state_in)
    return {
        "name": name,
        "source": CITATION,
        "note": note,
        "w": list(map(float, w)), "u": list(map(float, u)),
        "k": k.tolist(), "v": v.tolist(),
        "state_in": None if state_in is None else np.asarray(state_in, float).tolist(),
        "out": out.tolist(),
        "state_out": st.tolist(),
    }


def main():
    cases = [
        case("t3_worked", [0.7], [0.3],
             [[[0.5], [-1.0], [2.0]]], [[[1.0], [-2.0], [3.0]]],
             note="T=3: the first position where w matters; out_1 = v_1, "
                  "out_2 does not depend on w"),
        case("t5_two_channels", [0.05, 3.0], [-0.4, 1.1],
             [[[0.3, -2.0], [1.7, 0.4], [-0.6, 2.2], [0.0, -1.3], [2.5, 0.9]]],
             [[[1.0, -1.0], [0.5, 2.0], [-3.0, 0.25], [2.0, -0.5], [-1.5, 1.5]]],
             note="slow and fast decay side by side"),
        case("t4_with_state", [0.4], [0.2],
             [[[1.0], [-0.5], [0.25], [3.0]]], [[[2.0], [-1.0], [0.5], [-2.0]]],
             state_in=[[[1.5]], [[0.75]], [[2.0]]],
             note="non-empty initial state (n0, d0, m0) = (1.5, 0.75, 2.0)"),
    ]
    path = os.path.join(HERE, "worked_cases.json")
    with open(path, "w") as f:
        json.dump({"generated_by": "tests/golden/make_golden.py", "cases": cases}, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
