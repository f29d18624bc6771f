"""Sensitivity of the oracle pins (CPU only).

Plausible mistakes are planted in small numpy copies of the recurrence, never
in the GPU path: decay applied after the delta step, output read before the
update, decay on the value axis, beta dropped from the erase term, the erase
sign flipped, the scale dropped, and a gate without the exp on A.  Each
mutant must fail the same brute-force pin the real oracle passes, so a
mistake of that kind in the oracle could not hide.
"""
import numpy as np
import pytest

from oracle import brute, gate, seq


def _mutant(kind, q, k, v, g, beta, h0):
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    sc = 1 / np.sqrt(dk) if kind != "no_scale" else 1.0
    o = np.zeros((B, T, H, dv))
    for b in range(B):
        for h in range(H):
            S = np.array(h0[b, h], np.float64)
            for t in range(T):
                kt, vt, qt = (x[b, t, h].astype(np.float64) for x in (k, v, q))
                bt, e = float(beta[b, t, h]), np.exp(g[b, t, h].astype(np.float64))
                S_prev = S.copy()
                if kind == "decay_after_delta":
                    S = S + np.outer(kt, bt * (vt - S.T @ kt))
                    S = e[:, None] * S
                else:
                    if kind == "decay_on_values":
                        S = S * e[None, :dv] if dv <= dk else S
                    else:
                        S = e[:, None] * S
                    bb = 1.0 if kind == "no_beta_erase" else bt
                    sign = -1.0 if kind == "erase_sign" else 1.0
                    S = S + np.outer(kt, bt * vt) - sign * bb * np.outer(kt, S.T @ kt)
                read = S_prev if kind == "read_before_update" else S
                o[b, t, h] = sc * read.T @ qt
    return o


KINDS = ["decay_after_delta", "read_before_update", "decay_on_values",
         "no_beta_erase", "erase_sign", "no_scale"]


@pytest.mark.parametrize("kind", KINDS)
def test_brute_force_pin_rejects_mutant(kind):
    rng = np.random.default_rng(21)
    B, T, H, dk, dv = 1, 5, 1, 3, 2
    q = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    k = rng.standard_normal((B, T, H, dk))
    k = (k / np.linalg.norm(k, axis=-1, keepdims=True)).astype(np.float32)
    v = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    g = rng.uniform(-1.5, -0.1, (B, T, H, dk)).astype(np.float32)
    beta = rng.uniform(0.2, 0.9, (B, T, H)).astype(np.float32)
    h0 = rng.standard_normal((B, H, dk, dv))
    ob, _ = brute.kda_brute(q, k, v, g, beta, h0)
    ob = np.array([[[[float(x) for x in ob[b][t][h]] for h in range(H)] for t in range(T)] for b in range(B)])
    o_real, _ = seq.kda_seq(q, k, v, g, beta, h0)
    rms = np.sqrt(np.mean(ob ** 2))
    assert np.max(np.abs(o_real - ob)) <= 1e-12 * rms
    o_mut = _mutant(kind, q, k, v, g, beta, h0)
    assert np.max(np.abs(o_mut - ob)) > 1e-3 * rms, kind


def test_gate_pins_reject_mutants():
    A = np.array([0.7])
    z = np.full((1, 1, 1, 1), np.log(3.0) / np.exp(0.7))
    good = gate.gate(z, A)
    assert abs(good.item() + 3.75) < 1e-14
    no_exp = -5.0 / (1 + np.exp(-(A[None, None, :, None] * z)))          # exp(A) replaced by A
    flipped = -5.0 / (1 + np.exp(+(np.exp(A)[None, None, :, None] * z)))  # sign of the argument
    assert abs(no_exp.item() + 3.75) > 1e-3 and abs(flipped.item() + 3.75) > 1e-3


def test_softplus_gate_pins_reject_mutants():
    A = np.array([0.7])
    x = np.log(np.e - 1.0)
    z = np.full((1, 1, 1, 1), x / np.exp(0.7))
    assert abs(gate.gate_softplus(z, A).item() + 1.0) < 1e-14
    no_log1p = -(np.maximum(x, 0) + np.exp(-abs(x)))                  # log1p dropped
    no_max = -np.log1p(np.exp(-abs(x)))                                 # max(x, 0) dropped
    assert abs(no_log1p + 1.0) > 1e-3 and abs(no_max + 1.0) > 1e-3
