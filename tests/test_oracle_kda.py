"""Pins of the KDA oracle: the per-channel gate reduces to GDN when all
channels share a gate; replay equals the recurrence over exhaustive tiny
schedules; a zero gate channel erases that column; beta = 0 is pure decay."""

import numpy as np
import pytest

from oracle import gdn as OG
from oracle import kda as OK


def _inputs(rng, n, nb, HK, HV, K, V, scalar_gate=False):
    def unit(shape):
        a = rng.normal(size=shape)
        return a / np.linalg.norm(a, axis=-1, keepdims=True)
    out = []
    for _ in range(n):
        gs = np.exp(-np.log1p(np.exp(rng.normal(size=(nb, HV) if scalar_gate else (nb, HV, K)))))
        out.append(dict(q=unit((nb, HK, K)), k=unit((nb, HK, K)), v=rng.normal(size=(nb, HV, V)),
                        g=gs, beta=1 / (1 + np.exp(-rng.normal(size=(nb, HV))))))
    return out


def test_shared_gate_is_gdn():
    rng = np.random.default_rng(0)
    nb, HK, HV, K, V = 3, 2, 4, 5, 3
    S = rng.normal(0, 0.3, (nb, HV, V, K))
    a, b = S.copy(), S.copy()
    for x in _inputs(rng, 6, nb, HK, HV, K, V, scalar_gate=True):
        o1 = OG.gdn_standard_step(a, np.arange(nb), x["q"], x["k"], x["v"], x["g"], x["beta"])
        gk = np.repeat(x["g"][:, :, None], K, axis=2)
        o2 = OK.kda_standard_step(b, np.arange(nb), x["q"], x["k"], x["v"], gk, x["beta"])
        np.testing.assert_allclose(o2, o1, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(b, a, rtol=1e-13, atol=1e-15)


def test_zero_gate_channel_and_pure_decay():
    rng = np.random.default_rng(1)
    HK, HV, K, V = 1, 1, 4, 3
    S = rng.normal(size=(1, HV, V, K))
    x = _inputs(rng, 1, 1, HK, HV, K, V)[0]
    x["g"][0, 0, 2] = 0.0
    x["beta"][:] = 0.0
    b = S.copy()
    OK.kda_standard_step(b, np.array([0]), x["q"], x["k"], x["v"], x["g"], x["beta"])
    np.testing.assert_allclose(b[0, 0], S[0, 0] * x["g"][0, 0][None, :], rtol=1e-14)
    assert (b[0, 0][:, 2] == 0).all()


@pytest.mark.parametrize("L", [1, 2, 3, 5])
def test_replay_equals_recurrence_exhaustive(L):
    """Every row forced to flush at a different step; outputs, stored
    checkpoints and the state S0 + ring represent all equal the recurrence."""
    rng = np.random.default_rng(L)
    nb, HK, HV, K, V, T = 4, 1, 2, 3, 2, 3 * L + 2
    S_init = rng.normal(0, 0.3, (nb, HV, V, K))
    rec, rep = S_init.copy(), S_init.copy()
    dr = np.full((nb, HV, L, V), np.nan)
    kr = np.full((nb, HK, L, K), np.nan)
    gr = np.full((nb, HV, L, K), np.nan)
    wp = np.zeros(nb, np.int32)
    fl = np.full(nb, 1 if L == 1 else 0, np.uint8)
    for t, x in enumerate(_inputs(rng, T, nb, HK, HV, K, V)):
        force = ((np.arange(nb) + t) % (nb + 1) == 0).astype(np.uint8)
        fl = fl | force
        o_rec = OK.kda_standard_step(rec, np.arange(nb), x["q"], x["k"], x["v"], x["g"], x["beta"])
        o_rep, wp, fl, st = OK.kda_replay_step(rep, dr, kr, gr, np.arange(nb), wp, fl, x["q"],
                                               x["k"], x["v"], x["g"], x["beta"])
        assert st == 0
        np.testing.assert_allclose(o_rep, o_rec, rtol=1e-10, atol=1e-12)
        for b in range(nb):
            logical = OK.kda_replay_logical_state(rep, dr, kr, gr, b, wp[b])
            np.testing.assert_allclose(logical, rec[b], rtol=1e-10, atol=1e-12)
