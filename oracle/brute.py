"""Exact rational brute force for tiny gated-delta-rule cases -- TEST INFRASTRUCTURE ONLY.

The rule (Gated DeltaNet, cited by the "open-jev-fast" README, "Phase 3",
reference [5]) unrolled into its sum-of-products closed form instead of being
stepped:

    A_s   = alpha_s (I - beta_s k_s k_s^T)                       (dk x dk)
    S_t   = S_0 A_1 A_2 ... A_t + sum_{s<=t} beta_s v_s k_s^T A_{s+1} ... A_t
    o_t   = S_t q_t

with alpha_s = exp(g_s) given directly as a rational number, so every value is
an exact ``fractions.Fraction``.  Used only for T <= 8 and small dk, dv.
"""
from __future__ import annotations

from fractions import Fraction


def _matmul(a, b):
    n, m, p = len(a), len(b), len(b[0])
    return [[sum((a[i][l] * b[l][j] for l in range(m)), Fraction(0)) for j in range(p)] for i in range(n)]


def _eye(n):
    return [[Fraction(int(i == j)) for j in range(n)] for i in range(n)]


def transition(alpha, beta, kvec):
    """A = alpha (I - beta k k^T)."""
    d = len(kvec)
    return [[alpha * (Fraction(int(i == j)) - beta * kvec[i] * kvec[j]) for j in range(d)] for i in range(d)]


def state_at(t, alpha, beta, k, v, S0):
    """S_t (dv x dk) from the closed form; inputs are lists of Fractions, t in 0..T."""
    dk = len(k[0])
    dv = len(v[0])
    prod = _eye(dk)  # A_1 ... A_t
    for s in range(t):
        prod = _matmul(prod, transition(alpha[s], beta[s], k[s]))
    S = _matmul(S0, prod) if S0 is not None else [[Fraction(0)] * dk for _ in range(dv)]
    for s in range(t):
        tail = _eye(dk)
        for r in range(s + 1, t):
            tail = _matmul(tail, transition(alpha[r], beta[r], k[r]))
        outer = [[beta[s] * v[s][i] * k[s][j] for j in range(dk)] for i in range(dv)]
        term = _matmul(outer, tail)
        S = [[S[i][j] + term[i][j] for j in range(dk)] for i in range(dv)]
    return S


def run(alpha, beta, q, k, v, S0=None):
    """All outputs o_1..o_T (T x dv) and the final state S_T (dv x dk), exactly."""
    T = len(alpha)
    outs = []
    for t in range(1, T + 1):
        S = state_at(t, alpha, beta, k, v, S0)
        outs.append([sum((S[i][j] * q[t - 1][j] for j in range(len(q[0]))), Fraction(0)) for i in range(len(S))])
    S_T = state_at(T, alpha, beta, k, v, S0)
    return outs, S_T
