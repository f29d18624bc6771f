"""Pins for the backward oracle (no GPU).

The gradient of the recurrence (Kimi K3 technical report summary,
"Key claims"/"Method", section 2.1: delta-rule state update after a
channel-wise decay, output read from the updated state) is fixed by the
forward alone: it must equal central finite differences of the pinned
forward oracle.  A chunkwise form of the gradient (the algebra the GPU
kernels follow) must agree with the token-by-token one, and planted
mistakes in a numpy copy of the token-by-token gradient must fail the
finite-difference pin.
"""
import numpy as np
import pytest

from oracle import chunkwise, seq

NAMES = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "h0": "dh0"}


def _case(seed, B, T, H, dk, dv, g_low=-2.0):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, T, H, dk))
    X = {"q": rng.standard_normal((B, T, H, dk)), "k": k / np.linalg.norm(k, axis=-1, keepdims=True),
         "v": rng.standard_normal((B, T, H, dv)), "g": rng.uniform(g_low, -0.05, (B, T, H, dk)),
         "beta": rng.uniform(0.1, 0.95, (B, T, H))}
    X = {n: x.astype(np.float32) for n, x in X.items()}
    X["h0"] = rng.standard_normal((B, H, dk, dv))
    do = rng.standard_normal((B, T, H, dv))
    dht = rng.standard_normal((B, H, dk, dv))
    return X, do, dht


def _loss(X, do, dht):
    o, ht = seq.kda_seq(X["q"], X["k"], X["v"], X["g"], X["beta"], X["h0"])
    return float(np.sum(o * do) + np.sum(ht * dht))


def _finite_differences(X, do, dht, eps=2.0 ** -12):
    """Central differences of the forward oracle; the step actually taken is
    the difference of the fp32-rounded perturbed inputs."""
    fd = {}
    for n, a in X.items():
        d = np.zeros(a.shape)
        for idx in np.ndindex(a.shape):
            ap, am = a.copy(), a.copy()
            ap[idx] = a[idx] + eps
            am[idx] = a[idx] - eps
            lp = _loss({**X, n: ap}, do, dht)
            lm = _loss({**X, n: am}, do, dht)
            d[idx] = (lp - lm) / (float(ap[idx]) - float(am[idx]))
        fd[NAMES[n]] = d
    return fd


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / np.max(np.abs(b)))


@pytest.mark.parametrize("B,T,H,dk,dv,seg", [(1, 9, 2, 4, 3, 4), (2, 5, 1, 3, 5, 64), (1, 1, 1, 2, 2, 1)])
def test_seq_bwd_matches_finite_differences(B, T, H, dk, dv, seg):
    X, do, dht = _case(3, B, T, H, dk, dv)
    gr = seq.kda_seq_bwd(X["q"], X["k"], X["v"], X["g"], X["beta"], X["h0"], do, dht, seg=seg)
    fd = _finite_differences(X, do, dht)
    for n in fd:
        assert _rel(gr[n], fd[n]) < 1e-6, n


def test_seq_bwd_does_not_depend_on_the_checkpoint_spacing():
    X, do, dht = _case(4, 1, 23, 2, 5, 4)
    a = seq.kda_seq_bwd(X["q"], X["k"], X["v"], X["g"], X["beta"], X["h0"], do, dht, seg=1)
    for seg in (5, 23, 64):
        b = seq.kda_seq_bwd(X["q"], X["k"], X["v"], X["g"], X["beta"], X["h0"], do, dht, seg=seg)
        assert all(np.array_equal(a[n], b[n]) for n in a)


def test_seq_bwd_zero_initial_state_and_no_state_gradient():
    # h0 = None is the zero state; dht = None adds no final-state term
    X, do, _ = _case(5, 1, 7, 1, 3, 2)
    a = seq.kda_seq_bwd(X["q"], X["k"], X["v"], X["g"], X["beta"], None, do, None)
    b = seq.kda_seq_bwd(X["q"], X["k"], X["v"], X["g"], X["beta"], np.zeros((1, 1, 3, 2)), do, np.zeros((1, 1, 3, 2)))
    assert all(np.array_equal(a[n], b[n]) for n in a)


def test_seq_bwd_single_token_closed_form():
    # T = 1, h0 = 0: S_1 = beta k v^T, o = scale beta (q.k) v.  With loss
    # do.o: dv = scale beta (q.k) do, dbeta = scale (q.k)(v.do),
    # dq = scale beta (v.do) k, dk = scale beta (v.do) q, dg = 0 (S_0 = 0).
    rng = np.random.default_rng(6)
    dk, dv = 4, 3
    q, k, v = (rng.standard_normal((1, 1, 1, n)).astype(np.float32) for n in (dk, dk, dv))
    g = rng.uniform(-1, 0, (1, 1, 1, dk)).astype(np.float32)
    beta = np.array([[[0.7]]], np.float32)
    do = rng.standard_normal((1, 1, 1, dv))
    gr = seq.kda_seq_bwd(q, k, v, g, beta, None, do)
    sc = 1 / np.sqrt(dk)
    q64, k64, v64 = (x.astype(np.float64)[0, 0, 0] for x in (q, k, v))
    qk, vdo = q64 @ k64, v64 @ do[0, 0, 0]
    b = float(np.float32(0.7))
    np.testing.assert_allclose(gr["dv"][0, 0, 0], sc * b * qk * do[0, 0, 0], rtol=1e-12)
    np.testing.assert_allclose(gr["dbeta"][0, 0, 0], sc * qk * vdo, rtol=1e-12)
    np.testing.assert_allclose(gr["dq"][0, 0, 0], sc * b * vdo * k64, rtol=1e-12)
    np.testing.assert_allclose(gr["dk"][0, 0, 0], sc * b * vdo * q64, rtol=1e-12)
    assert np.all(gr["dg"] == 0.0)


@pytest.mark.parametrize("chunk", [1, 16, 64])
def test_chunkwise_bwd_matches_seq_bwd(chunk):
    X, do, dht = _case(7, 2, 70, 2, 8, 6, g_low=-5.0)
    a = seq.kda_seq_bwd(X["q"], X["k"], X["v"], X["g"], X["beta"], X["h0"], do, dht)
    b = chunkwise.kda_chunkwise_bwd(X["q"], X["k"], X["v"], X["g"], X["beta"], X["h0"], do, dht, chunk=chunk)
    for n in a:
        rms = np.sqrt(np.mean(a[n] ** 2))
        assert np.max(np.abs(a[n] - b[n])) <= 1e-12 * rms, n


# ------------------------------------------------------------ planted mistakes
def _np_bwd(X, do, dht, kind=None):
    """Token-by-token gradient in numpy with one optional planted mistake."""
    q, k, v, g, beta = (X[n].astype(np.float64) for n in ("q", "k", "v", "g", "beta"))
    B, T, H, dk = q.shape
    sc = 1 / np.sqrt(dk)
    out = {n: np.zeros(X[m].shape) for m, n in NAMES.items()}
    for b in range(B):
        for h in range(H):
            S = [X["h0"][b, h].copy()]
            for t in range(T):
                Sp = np.exp(g[b, t, h])[:, None] * S[-1]
                u = beta[b, t, h] * (v[b, t, h] - Sp.T @ k[b, t, h])
                S.append(Sp + np.outer(k[b, t, h], u))
            dS = dht[b, h].copy()
            for t in range(T - 1, -1, -1):
                e = np.exp(g[b, t, h])
                Sp = e[:, None] * S[t]
                p = Sp.T @ k[b, t, h]
                u = beta[b, t, h] * (v[b, t, h] - p)
                read = S[t] if kind == "read_prev_state" else S[t + 1]
                out["dq"][b, t, h] = sc * read @ do[b, t, h]
                dS = dS + sc * np.outer(q[b, t, h], do[b, t, h])
                du = dS.T @ k[b, t, h]
                dkt = dS @ u
                out["dbeta"][b, t, h] = du @ (v[b, t, h] - p) * (-1 if kind == "dbeta_sign" else 1)
                out["dv"][b, t, h] = beta[b, t, h] * du
                dp = -beta[b, t, h] * du
                if kind != "no_erase_term":
                    dkt = dkt + Sp @ dp
                    dS = dS + np.outer(k[b, t, h], dp)
                out["dk"][b, t, h] = dkt
                out["dg"][b, t, h] = np.sum(dS * (S[t] if kind == "dg_undecayed" else Sp), axis=1)
                if kind != "no_decay_carry":
                    dS = e[:, None] * dS
            out["dh0"][b, h] = dS
    return out


MUTANTS = ["read_prev_state", "dbeta_sign", "no_erase_term", "dg_undecayed", "no_decay_carry"]


def test_planted_mistakes_fail_the_finite_difference_pin():
    X, do, dht = _case(8, 1, 6, 1, 3, 2)
    fd = _finite_differences(X, do, dht)
    good = _np_bwd(X, do, dht)
    assert max(_rel(good[n], fd[n]) for n in fd) < 1e-6
    for kind in MUTANTS:
        bad = _np_bwd(X, do, dht, kind)
        assert max(_rel(bad[n], fd[n]) for n in fd) > 1e-3, kind
