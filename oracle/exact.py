"""Exact-rational brute force of the frame-wise GDN forward.

TEST INFRASTRUCTURE (see the header of gdn_ref.py for who may use it).

Instead of stepping the recurrence, this evaluates the unrolled closed form

    M_t = M_0 A_1 A_2 ... A_t + sum_{u<=t} b_u A_{u+1} ... A_t,
    A_u = gamma_u (I - beta_u K_u^T K_u),   b_u = beta_u V_u^T K_u,
    O_t = Q_t M_t^T,

with every entry a fractions.Fraction and hand-written list-of-lists matrix
helpers (no NumPy).  It is meant for tiny inputs (D <= 3, S <= 4, T <= 4) and
is the brute-force pin for the fp64 oracle: on dyadic inputs with few bits
every fp64 operation of the oracle is exact, so both must agree bit for bit.
"""
from __future__ import annotations

from fractions import Fraction
from typing import List, Optional, Sequence

Mat = List[List[Fraction]]


def frac(x) -> Fraction:
    return Fraction(x)


def zeros(r: int, c: int) -> Mat:
    return [[Fraction(0)] * c for _ in range(r)]


def eye(n: int) -> Mat:
    m = zeros(n, n)
    for i in range(n):
        m[i][i] = Fraction(1)
    return m


def transpose(a: Mat) -> Mat:
    return [list(col) for col in zip(*a)]


def matmul(a: Mat, b: Mat) -> Mat:
    n, k, m = len(a), len(b), len(b[0])
    assert len(a[0]) == k
    out = zeros(n, m)
    for i in range(n):
        for j in range(m):
            s = Fraction(0)
            for p in range(k):
                s += a[i][p] * b[p][j]
            out[i][j] = s
    return out


def add(a: Mat, b: Mat) -> Mat:
    return [[x + y for x, y in zip(ra, rb)] for ra, rb in zip(a, b)]


def scale(c: Fraction, a: Mat) -> Mat:
    return [[c * x for x in r] for r in a]


def to_mat(x) -> Mat:
    return [[frac(e) for e in row] for row in x]


def unrolled(q: Sequence, k: Sequence, v: Sequence, gamma: Sequence, beta: Sequence,
             state: Optional[Sequence] = None):
    """q, k, v: T nested lists of S x D numbers; gamma, beta: T numbers.
    Returns (O as T lists of S x D Fractions, M_T as D x D Fractions)."""
    T = len(q)
    D = len(q[0][0])
    M0 = zeros(D, D) if state is None else to_mat(state)
    A = []
    b = []
    for t in range(T):
        Kt, Vt = to_mat(k[t]), to_mat(v[t])
        g, be = frac(gamma[t]), frac(beta[t])
        A.append(scale(g, add(eye(D), scale(-be, matmul(transpose(Kt), Kt)))))
        b.append(scale(be, matmul(transpose(Vt), Kt)))

    def prod(lo: int, hi: int) -> Mat:
        """A_lo A_{lo+1} ... A_{hi-1} (identity when empty)."""
        p = eye(D)
        for u in range(lo, hi):
            p = matmul(p, A[u])
        return p

    O = []
    Mt = M0
    for t in range(T):
        Mt = matmul(M0, prod(0, t + 1))
        for u in range(t + 1):
            Mt = add(Mt, matmul(b[u], prod(u + 1, t + 1)))
        O.append(matmul(to_mat(q[t]), transpose(Mt)))
    return O, Mt
