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
