"""Exact rational brute force of the KDA recurrence forms (TEST INFRASTRUCTURE).

Pure-Python ``fractions.Fraction`` arithmetic on tiny shapes (K, V of a few
channels, up to 8 tokens). Decays and normalised keys are given directly as
rationals (this bypasses exp and the square root, which are irrational), so the
three forms of the method can be compared for *exact* equality:

* the stock recurrence, one token at a time,
* the closed-form RecoverSSM commit, and
* the chunked (WY) verify,

as stated on the vLLM page "vllm.models.kimi_k3.nvidia.specialized_decode.
cutedsl.kda.fused" (module docstring) and on the page "vllm.models.kimi_k3.
nvidia.recoverssm.cutedsl.commit" (module docstring). A mistake in any one form
(a dropped term, an off-by-one in a decay product, a transposed operand) breaks
the exact equality. Matrices are lists of rows: S[v][c].
"""
from fractions import Fraction


def zeros(rows, cols):
    return [[Fraction(0)] * cols for _ in range(rows)]


def copy(S):
    return [list(r) for r in S]


def seq_step(S, d, u, kn):
    """S <- S diag(d) + u kn^T."""
    V, K = len(S), len(S[0])
    return [[S[v][c] * d[c] + u[v] * kn[c] for c in range(K)] for v in range(V)]


def commit_seq(S0, u, kn, d, n):
    S = copy(S0)
    for t in range(n):
        S = seq_step(S, d[t], u[t], kn[t])
    return S


def commit_closed(S0, u, kn, d, n):
    V, K = len(S0), len(S0[0])
    D = [Fraction(1)] * K
    for s in range(n):
        D = [D[c] * d[s][c] for c in range(K)]
    S = [[S0[v][c] * D[c] for c in range(K)] for v in range(V)]
    for t in range(n):
        P = [Fraction(1)] * K
        for s in range(t + 1, n):
            P = [P[c] * d[s][c] for c in range(K)]
        for v in range(V):
            for c in range(K):
                S[v][c] += u[t][v] * kn[t][c] * P[c]
    return S


def verify_seq(S0, q, kn, v, d, beta):
    """The stock recurrence; returns (o, u, final state)."""
    S = copy(S0)
    V, K = len(S), len(S[0])
    T = len(q)
    o, u = [], []
    for t in range(T):
        S = [[S[r][c] * d[t][c] for c in range(K)] for r in range(V)]
        sk = [sum(S[r][c] * kn[t][c] for c in range(K)) for r in range(V)]
        ut = [beta[t] * (v[t][r] - sk[r]) for r in range(V)]
        S = [[S[r][c] + ut[r] * kn[t][c] for c in range(K)] for r in range(V)]
        o.append([sum(S[r][c] * q[t][c] for c in range(K)) for r in range(V)])
        u.append(ut)
    return o, u, S


def verify_wy(S, q, kn, v, d, beta):
    """The chunked form from an unmodified S; returns (o, u)."""
    V, K = len(S), len(S[0])
    T = len(q)
    gamma = []
    g = [Fraction(1)] * K
    for t in range(T):
        g = [g[c] * d[t][c] for c in range(K)]
        gamma.append(g)

    def pprod(s, t, c):
        p = Fraction(1)
        for r in range(s + 1, t + 1):
            p *= d[r][c]
        return p

    w = [[sum(S[r][c] * gamma[t][c] * kn[t][c] for c in range(K)) for r in range(V)]
         for t in range(T)]
    y = [[sum(S[r][c] * gamma[t][c] * q[t][c] for c in range(K)) for r in range(V)]
         for t in range(T)]
    A = [[sum(kn[s][c] * pprod(s, t, c) * kn[t][c] for c in range(K)) if s < t else None
          for s in range(T)] for t in range(T)]
    B = [[sum(kn[s][c] * pprod(s, t, c) * q[t][c] for c in range(K)) if s <= t else None
          for s in range(T)] for t in range(T)]
    u = [[None] * V for _ in range(T)]
    o = [[None] * V for _ in range(T)]
    for r in range(V):
        for t in range(T):
            acc = v[t][r] - w[t][r]
            for s in range(t):
                acc -= A[t][s] * u[s][r]
            u[t][r] = beta[t] * acc
            oo = y[t][r]
            for s in range(t + 1):
                oo += B[t][s] * u[s][r]
            o[t][r] = oo
    return o, u
