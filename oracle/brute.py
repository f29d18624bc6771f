"""Brute-force KDA forward on tiny inputs (mpmath, 50 digits) -- TEST INFRASTRUCTURE ONLY.

Follows the definition of the recurrence directly (Kimi K3 technical report
summary, "Key claims"/"Method", section 2.1: delta-rule state update after a
channel-wise decay), but in its unrolled product-of-transitions form rather
than step by step: with Phi_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)),

    S_t = Phi_t ... Phi_1 S_0 + sum_{s<=t} Phi_t ... Phi_{s+1} beta_s k_s v_s^T
    o_t = scale * S_t^T q_t

and every S_t is rebuilt from scratch (no reuse of S_{t-1}).  Meant for
T <= 6 and dk, dv <= 4.
"""
from __future__ import annotations

import mpmath as mp


def _mat(rows, cols, f):
    return mp.matrix([[f(i, j) for j in range(cols)] for i in range(rows)])


def kda_brute(q, k, v, g, beta, h0=None, scale=None, dps: int = 50):
    """Inputs are nested numeric arrays indexable [b][t][h][c]; returns
    (o [B][T][H][dv], ht [B][H][dk][dv]) as nested lists of mpf."""
    with mp.workdps(dps):
        B, T, H = len(q), len(q[0]), len(q[0][0])
        dk, dv = len(q[0][0][0]), len(v[0][0][0])
        sc = mp.mpf(1) / mp.sqrt(dk) if scale is None else mp.mpf(scale)
        o = [[[None] * H for _ in range(T)] for _ in range(B)]
        ht = [[None] * H for _ in range(B)]
        for b in range(B):
            for h in range(H):
                S0 = _mat(dk, dv, lambda i, j: mp.mpf(0) if h0 is None else mp.mpf(float(h0[b][h][i][j])))
                ks = [mp.matrix([mp.mpf(float(x)) for x in k[b][t][h]]) for t in range(T)]
                vs = [mp.matrix([mp.mpf(float(x)) for x in v[b][t][h]]) for t in range(T)]
                qs = [mp.matrix([mp.mpf(float(x)) for x in q[b][t][h]]) for t in range(T)]
                bs = [mp.mpf(float(beta[b][t][h])) for t in range(T)]
                Phi = []
                for t in range(T):
                    D = mp.diag([mp.exp(mp.mpf(float(x))) for x in g[b][t][h]])
                    P = mp.eye(dk) - bs[t] * (ks[t] * ks[t].T)
                    Phi.append(P * D)
                for t in range(T):
                    prod = mp.eye(dk)
                    for s in range(t, -1, -1):
                        prod = prod * Phi[s]
                    St = prod * S0
                    for s in range(t + 1):
                        tail = mp.eye(dk)
                        for r in range(t, s, -1):
                            tail = tail * Phi[r]
                        St = St + tail * (bs[s] * (ks[s] * vs[s].T))
                    ot = sc * (St.T * qs[t])
                    o[b][t][h] = [ot[j] for j in range(dv)]
                    if t == T - 1:
                        ht[b][h] = [[St[i, j] for j in range(dv)] for i in range(dk)]
                if T == 0:
                    ht[b][h] = [[S0[i, j] for j in range(dv)] for i in range(dk)]
        return o, ht
