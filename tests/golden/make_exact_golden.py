"""Writes exact_unrolled.json: tiny dyadic cases evaluated by the oracle's
exact-rational unrolled closed form (oracle/exact.py) and nothing else.

Run from the repository root:  python tests/golden/make_exact_golden.py
"""
import json
import os
import random
import sys

sys.path.insert(0, os.path.abspath(os.path.join(os.path.dirname(__file__), "..", "..")))
from oracle import exact  # noqa: E402


def dyadic(rng, lo=-8, hi=8, den=4):
    return f"{rng.randint(lo, hi)}/{den}"


def case(rng, T, S, D, with_state):
    mk = lambda: [[[dyadic(rng) for _ in range(D)] for _ in range(S)] for _ in range(T)]
    q, k, v = mk(), mk(), mk()
    gamma = [f"{rng.randint(2, 4)}/4" for _ in range(T)]
    beta = [f"{rng.randint(0, 4)}/4" for _ in range(T)]
    state = [[dyadic(rng) for _ in range(D)] for _ in range(D)] if with_state else None
    O, M = exact.unrolled(q, k, v, gamma, beta, state)
    return {"T": T, "S": S, "D": D, "q": q, "k": k, "v": v, "gamma": gamma, "beta": beta,
            "state": state,
            "O": [[[str(x) for x in row] for row in Ot] for Ot in O],
            "M_T": [[str(x) for x in row] for row in M]}


def main():
    rng = random.Random(20261203)
    cases = [case(rng, 3, 3, 2, False), case(rng, 3, 2, 3, True), case(rng, 4, 4, 2, True),
             case(rng, 2, 1, 3, True)]
    out = {
        "what": "Frame-wise GDN on tiny dyadic inputs, evaluated exactly (fractions) by the "
                "unrolled closed form M_t = M_0 A_1..A_t + sum_u b_u A_{u+1}..A_t, O_t = Q_t M_t^T.",
        "written_by": "tests/golden/make_exact_golden.py (calls oracle/exact.py only)",
        "cases": cases,
    }
    path = os.path.join(os.path.dirname(__file__), "exact_unrolled.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
