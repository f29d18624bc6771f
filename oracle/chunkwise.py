"""fp64 chunkwise-parallel form of the KDA forward -- TEST INFRASTRUCTURE ONLY.

Kimi K3 technical report summary ("Method", section 2.1) states that KDA has a
chunkwise-parallel form.  This module writes that form out plainly, as an
independent check of the sequential oracle (it shares no code with it):

Per (b, h) and per chunk of L <= C rows with state S entering the chunk,
Gamma = inclusive cumulative sum of g over the chunk's rows:

  1. A[r,s] = beta_r * sum_c k[r,c] k[s,c] exp(Gamma[r,c]-Gamma[s,c])   (s < r)
  2. M[r,s] = sum_c q[r,c] k[s,c] exp(Gamma[r,c]-Gamma[s,c])            (s <= r)
  3. Tm     = (I + A)^{-1} Diag(beta)
  4. W      = Tm (exp(Gamma) * K),   Ut = Tm V
  5. U      = Ut - W S
  6. O      = scale * ((exp(Gamma) * Q) S + M U)
  7. S     <- exp(Gamma_L) * S (row-wise) + (exp(Gamma_L - Gamma) * K)^T U

Derivation: with u_r = beta_r (v_r - (Diag(exp g_r) S_{r-1})^T k_r) the
recurrence is S_r = Diag(exp g_r) S_{r-1} + k_r u_r^T; unrolled inside the
chunk, S_r = Diag(exp Gamma_r) S + sum_{s<=r} Diag(exp(Gamma_r-Gamma_s)) k_s u_s^T,
which gives (I + A) U = Diag(beta) (V - (exp(Gamma)*K) S).

Pinned by tests/test_oracle_pins.py::test_chunkwise_matches_seq (C in
{1, 16, 64}; C = 1 is the recurrence itself) and the invariants there.
"""
from __future__ import annotations

import numpy as np


def kda_chunkwise(q, k, v, g, beta, h0=None, scale=None, chunk: int = 64):
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(dk)
    o = np.zeros((B, T, H, dv))
    ht = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if h0 is None else np.array(h0[b, h], dtype=np.float64)
            for t0 in range(0, T, chunk):
                sl = slice(t0, min(t0 + chunk, T))
                Q, K, V, G = q[b, sl, h], k[b, sl, h], v[b, sl, h], g[b, sl, h]
                bt = beta[b, sl, h]
                L = Q.shape[0]
                Gam = np.cumsum(G, axis=0)                       # [L, dk]
                diff = Gam[:, None, :] - Gam[None, :, :]         # [r, s, c]
                lower_strict = np.tril(np.ones((L, L), bool), -1)
                lower = np.tril(np.ones((L, L), bool), 0)
                E = np.where(lower[:, :, None], np.exp(np.where(lower[:, :, None], diff, 0.0)), 0.0)
                A = bt[:, None] * np.einsum("rc,sc,rsc->rs", K, K, E)
                A = np.where(lower_strict, A, 0.0)
                M = np.where(lower, np.einsum("rc,sc,rsc->rs", Q, K, E), 0.0)
                Tm = np.linalg.solve(np.eye(L) + A, np.diag(bt))
                W = Tm @ (np.exp(Gam) * K)
                Ut = Tm @ V
                U = Ut - W @ S
                o[b, sl, h] = scale * ((np.exp(Gam) * Q) @ S + M @ U)
                GL = Gam[-1]
                S = np.exp(GL)[:, None] * S + (np.exp(GL[None, :] - Gam) * K).T @ U
            ht[b, h] = S
    return o, ht


def kda_chunkwise_bwd(q, k, v, g, beta, h0, do, dht=None, scale=None, chunk: int = 64):
    """Gradient of the chunkwise form above, chunk by chunk from the last one.

    Per chunk, with S entering, N = dL/dS leaving (dht for the last chunk),
    dO the chunk's output gradient, L = I + A, Kb = exp(Gamma) * K,
    Qb = exp(Gamma) * Q, Kh = exp(Gamma_L - Gamma) * K, R = V - Kb S,
    U = L^{-1} Diag(beta) R (steps 1-7 above), the reverse-mode chain rule gives

      dU  = scale M^T dO + Kh N                dS = exp(Gamma_L) * N + scale Qb^T dO - Kb^T (beta * Z)
      Z   = L^{-T} dU                          dV = beta * Z,   dbeta = rowsum(Z * R) + rowsum(dA * A) / beta
      dA  = -strict_lower(Z U^T)               dM = scale lower(dO U^T)
      dQb = scale dO S^T,  dKb = -(beta * Z) S^T,  dKh = U N^T

    then through the decay factors to q, k and Gamma (Gamma_L also through
    the state's decay), and dg = reverse cumulative sum of dGamma.  Written
    with the full pairwise factors exp(Gamma_r - Gamma_s) (fp64), as an
    independent check of kda_seq_bwd (tests/test_oracle_pins.py)."""
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    do = np.asarray(do, dtype=np.float64)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(dk)
    out = {"dq": np.zeros((B, T, H, dk)), "dk": np.zeros((B, T, H, dk)), "dv": np.zeros((B, T, H, dv)),
           "dg": np.zeros((B, T, H, dk)), "dbeta": np.zeros((B, T, H)), "dh0": np.zeros((B, H, dk, dv))}
    starts = list(range(0, T, chunk))
    for b in range(B):
        for h in range(H):
            # states entering each chunk (forward)
            S = np.zeros((dk, dv)) if h0 is None else np.array(h0[b, h], dtype=np.float64)
            entering = []
            for t0 in starts:
                entering.append(S)
                _, S = kda_chunkwise(q[b:b + 1, t0:t0 + chunk, h:h + 1], k[b:b + 1, t0:t0 + chunk, h:h + 1],
                                     v[b:b + 1, t0:t0 + chunk, h:h + 1], g[b:b + 1, t0:t0 + chunk, h:h + 1],
                                     beta[b:b + 1, t0:t0 + chunk, h:h + 1], S[None, None], scale, chunk)
                S = S[0, 0]
            N = np.zeros((dk, dv)) if dht is None else np.array(dht[b, h], dtype=np.float64)
            for ci in range(len(starts) - 1, -1, -1):
                t0 = starts[ci]
                sl = slice(t0, min(t0 + chunk, T))
                Q, K, V, G, dO = q[b, sl, h], k[b, sl, h], v[b, sl, h], g[b, sl, h], do[b, sl, h]
                bt = beta[b, sl, h]
                S = entering[ci]
                Lr = Q.shape[0]
                Gam = np.cumsum(G, axis=0)
                GL = Gam[-1]
                lower_strict = np.tril(np.ones((Lr, Lr), bool), -1)
                lower = np.tril(np.ones((Lr, Lr), bool), 0)
                diff = Gam[:, None, :] - Gam[None, :, :]
                E = np.where(lower[:, :, None], np.exp(np.where(lower[:, :, None], diff, 0.0)), 0.0)
                Graw = np.where(lower_strict, np.einsum("rc,sc,rsc->rs", K, K, E), 0.0)
                A = bt[:, None] * Graw
                M = np.where(lower, np.einsum("rc,sc,rsc->rs", Q, K, E), 0.0)
                Lm = np.eye(Lr) + A
                Kb, Qb, Kh = np.exp(Gam) * K, np.exp(Gam) * Q, np.exp(GL[None, :] - Gam) * K
                R = V - Kb @ S
                U = np.linalg.solve(Lm, bt[:, None] * R)
                # reverse
                dU = scale * M.T @ dO + Kh @ N
                Z = np.linalg.solve(Lm.T, dU)
                dS_in = np.exp(GL)[:, None] * N + scale * Qb.T @ dO - Kb.T @ (bt[:, None] * Z)
                out["dv"][b, sl, h] = bt[:, None] * Z
                dA = -np.where(lower_strict, Z @ U.T, 0.0)
                dM = scale * np.where(lower, dO @ U.T, 0.0)
                out["dbeta"][b, sl, h] = np.sum(Z * R, axis=1) + np.sum(dA * Graw, axis=1)
                dGr = bt[:, None] * dA                             # gradient of the unscaled Gram
                dQb, dKb, dKh = scale * dO @ S.T, -(bt[:, None] * Z) @ S.T, U @ N.T
                # pairwise-decayed terms: row side (r) and column side (s)
                dk_grow = np.einsum("rs,sc,rsc->rc", dGr, K, E)
                dk_gcol = np.einsum("rs,rc,rsc->sc", dGr, K, E)
                dq_m = np.einsum("rs,sc,rsc->rc", dM, K, E)
                dk_mcol = np.einsum("rs,rc,rsc->sc", dM, Q, E)
                dq = np.exp(Gam) * dQb + dq_m
                dk_plus = np.exp(Gam) * dKb + dk_grow
                dk_minus = dk_gcol + dk_mcol + np.exp(GL[None, :] - Gam) * dKh
                out["dq"][b, sl, h] = dq
                out["dk"][b, sl, h] = dk_plus + dk_minus
                dGam = Q * dq + K * (dk_plus - dk_minus)
                dGL = np.sum(K * np.exp(GL[None, :] - Gam) * dKh, axis=0) + np.exp(GL) * np.sum(N * S, axis=1)
                out["dg"][b, sl, h] = np.cumsum(dGam[::-1], axis=0)[::-1] + dGL[None, :]
                N = dS_in
            out["dh0"][b, h] = N
    return out
