"""Chunk-parallel fp64 form of the gated delta rule -- TEST INFRASTRUCTURE.

Exists only to pin the chunk algebra (the WY/UT-transform form) against the
token-by-token definition in ``gdn_oracle.c``; it never grades the GPU.

The form follows Yang, Kautz and Hatamizadeh, "Gated Delta Networks" (ICLR
2025), chunkwise algorithm, which extends the WY/UT representation of Yang et
al., "Parallelizing Linear Transformers with the Delta Rule over Sequence
Length" (NeurIPS 2024).  Derivation in this notation: write the step as
S_t = e^{g_t} S_{t-1} + u_t k_t^T with u_t = beta_t (v_t - e^{g_t} S_{t-1} k_t).
Inside a chunk with cumulative decay gamma_r = sum_{s<=r} g_s and entering
state S0, unrolling gives
    S_r = e^{gamma_r} S0 + sum_{s<=r} e^{gamma_r - gamma_s} u_s k_s^T,
so the u's satisfy the unit lower-triangular system
    (I + A) U = diag(beta) V - diag(beta e^{gamma}) K S0^T,
    A_rs = beta_r e^{gamma_r - gamma_s} (k_r . k_s)   for s < r.
With Tm = (I + A)^{-1}:  W = Tm diag(beta e^gamma) K,  U~ = Tm diag(beta) V,
    U = U~ - W S0^T
    O = diag(e^gamma) Q S0^T + tril_incl(Q K^T (.) D) U,  D_rs = e^{gamma_r-gamma_s}
    S_C = e^{gamma_last} S0 + U^T diag(e^{gamma_last - gamma}) K.
Only exponentials of non-positive differences are formed.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def delta_rule_chunked(q, k, v, g, beta, S0=None, C: int = 16):
    """Same contract as ``oracle.delta_rule``: q, k [T, dk], v [T, dv],
    g, beta [T], S0 [dv, dk].  Returns (o [T, dv], S [dv, dk])."""
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in
                        (q, k, v, g, beta))
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, dtype=np.float64)
    o = np.empty((T, dv))
    for c0 in range(0, T, C):
        c1 = min(T, c0 + C)
        Qc, Kc, Vc = q[c0:c1], k[c0:c1], v[c0:c1]
        gc, bc = g[c0:c1], beta[c0:c1]
        L = c1 - c0
        gam = np.cumsum(gc)
        diff = gam[:, None] - gam[None, :]                 # gamma_r - gamma_s
        lower = np.tril(np.ones((L, L), dtype=bool), -1)
        D = np.where(np.tril(np.ones((L, L), dtype=bool)),
                     np.exp(np.where(lower | np.eye(L, dtype=bool), diff, 0.0)),
                     0.0)
        A = np.where(lower, bc[:, None] * D * (Kc @ Kc.T), 0.0)
        IA = np.eye(L) + A
        W = solve_triangular(IA, (bc * np.exp(gam))[:, None] * Kc, lower=True,
                             unit_diagonal=True)
        Ut = solve_triangular(IA, bc[:, None] * Vc, lower=True,
                              unit_diagonal=True)
        U = Ut - W @ S.T
        M = np.tril((Qc @ Kc.T) * D)
        o[c0:c1] = np.exp(gam)[:, None] * (Qc @ S.T) + M @ U
        last = gam[-1]
        S = np.exp(last) * S + U.T @ (np.exp(last - gam)[:, None] * Kc)
    return o, S


def chunk_affine_map(k, v, g, beta):
    """The affine map a whole chunk applies to the entering state:
    S_C = S0 P^T + R  with P = e^{gamma_last} I - K^T diag(e^{gamma_last -
    gamma}) W  (dk x dk) and R = U~^T diag(e^{gamma_last - gamma}) K
    (dv x dk).  Returned as (P, R); used to pin the chunk algebra."""
    k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (k, v, g, beta))
    L, dk = k.shape
    gam = np.cumsum(g)
    lower = np.tril(np.ones((L, L), dtype=bool), -1)
    diff = gam[:, None] - gam[None, :]
    D = np.exp(np.where(lower, diff, 0.0))
    A = np.where(lower, beta[:, None] * D * (k @ k.T), 0.0)
    IA = np.eye(L) + A
    W = solve_triangular(IA, (beta * np.exp(gam))[:, None] * k, lower=True,
                         unit_diagonal=True)
    Ut = solve_triangular(IA, beta[:, None] * v, lower=True,
                          unit_diagonal=True)
    Kd = np.exp(gam[-1] - gam)[:, None] * k
    P = np.exp(gam[-1]) * np.eye(dk) - Kd.T @ W
    R = Ut.T @ Kd
    return P, R
