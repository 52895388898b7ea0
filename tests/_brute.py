"""Exact-rational brute force of the gated delta rule for tiny cases (T <= 8).

Independent of the oracle's rank-1 update: it writes the state after t tokens as
an explicit product of transition matrices,

    H_t = (Phi_t ... Phi_1) H_0 + sum_{s<=t} (Phi_t ... Phi_{s+1}) beta_s k_s v_s^T,
    Phi_t = alpha_t (I - beta_t k_t k_t^T)       ([d_k x d_k]),

which is the definition on the "Prizma seq/delta.py" page (module docstring)
rearranged: alpha H + k (beta (v - alpha H^T k))^T = alpha (I - beta k k^T) H + beta k v^T.
Everything is fractions.Fraction; nothing is rounded.
"""
from fractions import Fraction as F


def eye(n):
    return [[F(int(i == j)) for j in range(n)] for i in range(n)]


def matmul(A, B):
    return [[sum((A[i][k] * B[k][j] for k in range(len(B))), F(0)) for j in range(len(B[0]))]
            for i in range(len(A))]


def add(A, B):
    return [[a + b for a, b in zip(ra, rb)] for ra, rb in zip(A, B)]


def outer(x, y, s=F(1)):
    return [[s * a * b for b in y] for a in x]


def transpose(A):
    return [list(r) for r in zip(*A)]


def phi(alpha, beta, k):
    n = len(k)
    I = eye(n)
    kk = outer(k, k, beta)
    return [[alpha * (I[i][j] - kk[i][j]) for j in range(n)] for i in range(n)]


def state_after(order, k, v, alpha, beta, H0, upto):
    """State after the first `upto` tokens of `order` (a list of token indices)."""
    dk, dv = len(H0), len(H0[0])
    toks = order[:upto]
    prod = eye(dk)
    for t in toks:
        prod = matmul(phi(alpha[t], beta[t], k[t]), prod)
    H = matmul(prod, H0)
    for i, s in enumerate(toks):
        P = eye(dk)
        for t in toks[i + 1:]:
            P = matmul(phi(alpha[t], beta[t], k[t]), P)
        H = add(H, matmul(P, outer(k[s], v[s], beta[s])))
    return H


def read(H, qv):
    return [sum((H[r][c] * qv[r] for r in range(len(qv))), F(0)) for c in range(len(H[0]))]


def run(order, q, k, v, alpha, beta, H0, read_mode="post"):
    """Outputs o[t] for t in order (dict token -> vector) and the final state."""
    out = {}
    for i, t in enumerate(order):
        H = state_after(order, k, v, alpha, beta, H0, i + 1 if read_mode == "post" else i)
        out[t] = read(H, q[t])
    return out, state_after(order, k, v, alpha, beta, H0, len(order))
