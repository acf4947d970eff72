"""Independent fp64 forms of the KDA operator -- TEST INFRASTRUCTURE ONLY.

Used to pin the C recurrence (kda_oracle.c) against forms that share none of
its code.  All functions work on one sequence and one head:

    q, k : [T, dk]   v : [T, dv]   log_alpha : [T, dk]   beta : [T]
    S0   : [dk, dv]  (state rows are key channels)

returning (o [T, dv], S_T [dk, dv]) in fp64.
"""
from __future__ import annotations

import numpy as np


def transitions(k, log_alpha, beta):
    """Per-token dk x dk transitions A_t = (I - beta_t k_t k_t^T) Diag(alpha_t).

    This is the DPLR matrix Diag(alpha) - a b^T with a = beta k and
    b = alpha (.) k ("Kimi Linear" page, "The constrained DPLR form and the
    chunkwise algorithm").
    """
    T, dk = k.shape
    A = np.empty((T, dk, dk))
    eye = np.eye(dk)
    for t in range(T):
        A[t] = (eye - beta[t] * np.outer(k[t], k[t])) @ np.diag(np.exp(log_alpha[t]))
    return A


def brute(q, k, v, log_alpha, beta, S0):
    """S_t = A_t S_{t-1} + beta_t k_t v_t^T with explicit dense A_t; o_t = S_t^T q_t."""
    A = transitions(k, log_alpha, beta)
    S = np.array(S0, dtype=np.float64)
    o = np.empty((len(q), v.shape[1]))
    for t in range(len(q)):
        S = A[t] @ S + beta[t] * np.outer(k[t], v[t])
        o[t] = S.T @ q[t]
    return o, S


def attention_form(q, k, v, log_alpha, beta, S0):
    """Unrolled sum: o_t = sum_i beta_i (k_i^T M_{t,i}^T q_t) v_i + (M_{t,-1} S0)^T q_t,

    where M_{t,i} = A_t A_{t-1} ... A_{i+1} carries write i forward to read t
    (the expansion of the output over earlier keys that the "Kimi Linear" page
    describes in "Why channel-wise gating matters").  O(T^2 dk^3): tiny T only.
    """
    A = transitions(k, log_alpha, beta)
    T, dk = k.shape
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        M = np.eye(dk)  # M_{t,t}
        for i in range(t, -1, -1):
            # M = A_t ... A_{i+1}
            o[t] += beta[i] * (k[i] @ (M.T @ q[t])) * v[i]
            M = M @ A[i]
        # M = A_t ... A_0
        o[t] += (M @ S0).T @ q[t]
    S = np.array(S0, dtype=np.float64)
    for t in range(T):
        S = A[t] @ S + beta[t] * np.outer(k[t], v[t])
    return o, S


def forward_substitution(Atil):
    """T = (I + Atil)^{-1} for strictly lower-triangular Atil, row by row.

    T_{r,:r} = -Atil_{r,:r} T_{:r,:r}, T_{rr} = 1 (the UT transform of the
    "Kimi Linear" page, "The constrained DPLR form and the chunkwise algorithm").
    """
    n = Atil.shape[0]
    T = np.eye(n)
    for r in range(1, n):
        T[r, :r] = -Atil[r, :r] @ T[:r, :r]
    return T


def chunkwise(q, k, v, log_alpha, beta, S0, C=64, solve="substitution"):
    """Chunked WY/UT evaluation of the same recurrence (derived from it).

    Within a chunk of n tokens with start state S, with G_r = sum_{j<=r} g_j
    (chunk-local inclusive cumsum of log_alpha, per key channel):

      Atil[r,i] = beta_r sum_c k_rc k_ic exp(G_rc - G_ic)   (i < r)
      Tm        = (I + Atil)^{-1}
      W         = Tm diag(beta) (K * exp(G))       Util = Tm diag(beta) V
      U         = Util - W S
      P[r,i]    = sum_c q_rc k_ic exp(G_rc - G_ic)      (i <= r)
      O         = (Q * exp(G)) S + P U
      S_next    = Diag(exp(G_last)) S + (K * exp(G_last - G))^T U

    The products use exp(G_r - G_i) formed pairwise, so nothing overflows.
    """
    T, dk = k.shape
    dv = v.shape[1]
    S = np.array(S0, dtype=np.float64)
    o = np.empty((T, dv))
    for c0 in range(0, T, C):
        c1 = min(T, c0 + C)
        L = chunk_local(q[c0:c1], k[c0:c1], v[c0:c1], log_alpha[c0:c1], beta[c0:c1], solve)
        U = L["Ut"] - L["W"] @ S
        o[c0:c1] = L["Qg"] @ S + L["P"] @ U
        S = L["gamma"][:, None] * S + L["Kh"].T @ U
    return o, S


def chunk_local(Q, K, V, log_alpha, beta, solve="substitution"):
    """The quantities of one chunk that do not depend on the state entering it (the
    terms of ``chunkwise``'s docstring): G, Atil, Tm = (I + Atil)^-1, W, Util, P,
    Qg = Q exp(G), Kh = K exp(G_last - G) and gamma = exp(G_last); fp64 dict."""
    b = np.asarray(beta, np.float64)
    G = np.cumsum(log_alpha, axis=0)
    D = np.exp(G[:, None, :] - G[None, :, :])           # [r, i, c] = exp(G_rc - G_ic)
    kk = np.einsum("rc,ic,ric->ri", K, K, D)
    qk = np.einsum("rc,ic,ric->ri", Q, K, D)
    Atil = np.tril(b[:, None] * kk, -1)
    P = np.tril(qk)
    if solve == "substitution":
        Tm = forward_substitution(Atil)
    else:
        Tm = np.linalg.inv(np.eye(len(b)) + Atil)
    W = Tm @ (b[:, None] * (K * np.exp(G)))
    Ut = Tm @ (b[:, None] * V)
    return {"G": G, "Atil": Atil, "Tm": Tm, "W": W, "Ut": Ut, "P": P, "Qg": Q * np.exp(G),
            "Kh": K * np.exp(G[-1][None, :] - G), "gamma": np.exp(G[-1])}


# ---------------------------------------------------------------------------
# The general DPLR transition (independent a and b; "Kimi Linear" page, "The
# constrained DPLR form and the chunkwise algorithm"):
#     S_t = (Diag(alpha_t) - a_t b_t^T) S_{t-1} + k_t v_t^T,   o_t = S_t^T q_t.
# ---------------------------------------------------------------------------
def dplr_transitions(a, b, log_alpha):
    """Per-token dense dk x dk transitions Diag(alpha_t) - a_t b_t^T."""
    T, dk = a.shape
    return np.stack([np.diag(np.exp(log_alpha[t])) - np.outer(a[t], b[t]) for t in range(T)]) if T else \
        np.zeros((0, dk, dk))


def dplr_attention_form(q, k, v, a, b, log_alpha, S0):
    """o_t = sum_{i<=t} (q_t^T M_{t,i} k_i) v_i + (M_{t,-1} S0)^T q_t with M_{t,i} the
    product of the dense transitions of tokens i+1 .. t; O(T^2 dk^3), tiny T only."""
    A = dplr_transitions(a, b, log_alpha)
    T, dk = k.shape
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        M = np.eye(dk)
        for i in range(t, -1, -1):
            o[t] += (q[t] @ M @ k[i]) * v[i]
            M = M @ A[i]
        o[t] += (M @ S0).T @ q[t]
    M = np.eye(dk)
    for t in range(T):
        M = A[t] @ M
    S = M @ S0
    for i in range(T):
        P = np.eye(dk)
        for t in range(i + 1, T):
            P = A[t] @ P
        S = S + P @ np.outer(k[i], v[i])
    return o, S


def dplr_chunkwise(q, k, v, a, b, log_alpha, S0, C=64):
    """Chunked evaluation of the general DPLR recurrence (derived from it).

    With w_r = b_r^T S_{r-1} (what the rank-one term reads), G the chunk-local
    inclusive cumsum of log_alpha and Gx = G - log_alpha (exclusive):
      Mba[r,i] = sum_c b_rc a_ic e^{Gx_rc - G_ic},  Mbk likewise with k   (i < r)
      Mqa[r,i] = sum_c q_rc a_ic e^{G_rc - G_ic},   Mqk likewise with k   (i <= r)
      (I + Mba) w = (B e^{Gx}) S + Mbk V
      O      = (Q e^{G}) S + Mqk V - Mqa w
      S_next = e^{G_last} S + (K e^{G_last - G})^T V - (A e^{G_last - G})^T w
    b sees the state before its own token's decay (Gx), the other vectors after.
    """
    T, dk = k.shape
    dv = v.shape[1]
    S = np.array(S0, dtype=np.float64)
    o = np.empty((T, dv))
    for c0 in range(0, T, C):
        c1 = min(T, c0 + C)
        L = dplr_chunk_local(q[c0:c1], k[c0:c1], v[c0:c1], a[c0:c1], b[c0:c1], log_alpha[c0:c1])
        w = L["Z"] + L["Y"] @ S
        o[c0:c1] = L["Qg"] @ S + L["Mqk"] @ v[c0:c1] - L["Mqa"] @ w
        S = L["gamma"][:, None] * S + L["Kh"].T @ v[c0:c1] - L["Ah"].T @ w
    return o, S


def dplr_chunk_local(Q, K, V, A_, B_, log_alpha):
    """The state-free quantities of one chunk of ``dplr_chunkwise`` (fp64 dict): the four
    gated products, Y = (I + Mba)^-1 B e^{Gx} and Z = (I + Mba)^-1 Mbk V (so that
    w = Z + Y S), Qg = Q e^G, Kh = K e^{G_last - G}, Ah = A e^{G_last - G} and
    gamma = e^{G_last}."""
    G = np.cumsum(log_alpha, axis=0)
    Gx = G - log_alpha
    # [r, i, c]; only i < r (Dx) and i <= r (D) are used, where the exponent is <= 0
    Dx = np.exp(np.minimum(Gx[:, None, :] - G[None, :, :], 0.0))
    D = np.exp(np.minimum(G[:, None, :] - G[None, :, :], 0.0))
    Mba = np.tril(np.einsum("rc,ic,ric->ri", B_, A_, Dx), -1)
    Mbk = np.tril(np.einsum("rc,ic,ric->ri", B_, K, Dx), -1)
    Mqa = np.tril(np.einsum("rc,ic,ric->ri", Q, A_, D))
    Mqk = np.tril(np.einsum("rc,ic,ric->ri", Q, K, D))
    I_M = np.eye(len(G)) + Mba
    dec = np.exp(G[-1][None, :] - G)
    return {"Mba": Mba, "Mbk": Mbk, "Mqa": Mqa, "Mqk": Mqk,
            "Y": np.linalg.solve(I_M, B_ * np.exp(Gx)), "Z": np.linalg.solve(I_M, Mbk @ V),
            "Qg": Q * np.exp(G), "Kh": K * dec, "Ah": A_ * dec, "gamma": np.exp(G[-1])}
