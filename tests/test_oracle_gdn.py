"""Pins for oracle.gdn (CPU only).

The recurrence is pinned by the delta rule's defining property (with g = 1,
beta = 1 and a unit key, the value just written is recalled exactly; keys
that are orthonormal are all recalled), by pure decay when beta = 0 and by
NaN-poisoned key heads.  The replay is pinned to the recurrence over small
exhaustive schedules, with L = 1 equal to the recurrence and the stored
checkpoint after each flush equal to the recurrent state.
"""

import numpy as np
import pytest

from oracle import gdn as Gd
from oracle import mamba2 as M


def _unit(r, shape):
    a = r.standard_normal(shape)
    return a / np.linalg.norm(a, axis=-1, keepdims=True)


def test_delta_rule_recalls_the_written_value():
    r = np.random.default_rng(30)
    HV, HK, V, K = 2, 1, 3, 5
    S = r.standard_normal((1, HV, V, K))
    k = _unit(r, (1, HK, K))
    v = r.standard_normal((1, HV, V))
    o = Gd.gdn_standard_step(S, [0], k, k, v, np.ones((1, HV)), np.ones((1, HV)))
    for h in range(HV):
        np.testing.assert_allclose(S[0, h] @ k[0, 0], v[0, h], rtol=1e-13, atol=1e-13)
    # q = k reads the value back, scaled by 1/sqrt(K)
    np.testing.assert_allclose(o, v / np.sqrt(K), rtol=1e-13, atol=1e-13)


def test_orthonormal_keys_are_all_recalled():
    r = np.random.default_rng(31)
    HV, HK, V, K, m = 1, 1, 4, 6, 5
    Q, _ = np.linalg.qr(r.standard_normal((K, K)))
    S = r.standard_normal((1, HV, V, K))
    vals = r.standard_normal((m, V))
    for i in range(m):
        ki = Q[:, i][None, None, :]
        Gd.gdn_standard_step(S, [0], ki, ki, vals[i][None, None, :],
                             np.ones((1, HV)), np.ones((1, HV)))
    for i in range(m):
        np.testing.assert_allclose(S[0, 0] @ Q[:, i], vals[i], rtol=1e-12, atol=1e-12)


def test_zero_beta_is_pure_decay():
    r = np.random.default_rng(32)
    HV, HK, V, K, T = 2, 1, 3, 4, 5
    S0 = r.standard_normal((1, HV, V, K))
    S = S0.copy()
    gam = np.ones(HV)
    for _ in range(T):
        g = r.uniform(0.2, 1.0, (1, HV))
        q = _unit(r, (1, HK, K))
        o = Gd.gdn_standard_step(S, [0], q, _unit(r, (1, HK, K)),
                                 r.standard_normal((1, HV, V)), g,
                                 np.zeros((1, HV)), scale=0.5)
        gam = gam * g[0]
        for h in range(HV):
            np.testing.assert_allclose(S[0, h], gam[h] * S0[0, h], rtol=1e-13)
            np.testing.assert_allclose(o[0, h], 0.5 * gam[h] * (S0[0, h] @ q[0, 0]),
                                       rtol=1e-12, atol=1e-14)


def test_value_heads_read_their_key_head():
    r = np.random.default_rng(33)
    HV, HK, V, K = 4, 2, 2, 3
    S = r.standard_normal((1, HV, V, K))
    for bad in range(HK):
        k = _unit(r, (1, HK, K))
        q = _unit(r, (1, HK, K))
        k[:, bad] = np.nan
        o = Gd.gdn_standard_step(S.copy(), [0], q, k, r.standard_normal((1, HV, V)),
                                 np.full((1, HV), 0.9), np.full((1, HV), 0.5))
        heads_bad = np.arange(HV) // (HV // HK) == bad
        assert np.isnan(o[:, heads_bad]).all()
        assert np.isfinite(o[:, ~heads_bad]).all()


def _run_pair(r, HV, HK, V, K, L, T, nb, force=None, resets=None,
              state_dtype="f64"):
    slots = nb + 1
    pool = np.full((slots, HV, V, K), np.nan)
    slot_idx = np.arange(nb) + 1
    for s in slot_idx:
        pool[s] = r.standard_normal((HV, V, K)) * 0.1
    rec = pool.copy()
    dr = np.full((slots, HV, L, V), np.nan)
    kr = np.full((slots, HK, L, K), np.nan)
    gr = np.full((slots, HV, L), np.nan)
    wp = np.zeros(nb, np.int32)
    fl = np.full(nb, 1 if L == 1 else 0, np.uint8)
    for t in range(T):
        if resets and t in resets:
            for b in resets[t]:
                fresh = r.standard_normal((HV, V, K)) * 0.1
                pool[slot_idx[b]] = fresh
                rec[slot_idx[b]] = fresh
            wp, fl = M.ring_reset(wp, fl, resets[t], L)
        if force and t in force:
            fl = fl.copy()
            fl[force[t]] = 1
        q = _unit(r, (nb, HK, K))
        k = _unit(r, (nb, HK, K))
        v = r.standard_normal((nb, HV, V))
        g = r.uniform(0.3, 1.0, (nb, HV))
        beta = r.uniform(0.0, 1.0, (nb, HV))
        o_rec = Gd.gdn_standard_step(rec, slot_idx, q, k, v, g, beta,
                                     state_dtype=state_dtype)
        flushing = fl.astype(bool).copy()
        o, nwp, nfl, st = Gd.gdn_replay_step(pool, dr, kr, gr, slot_idx, wp, fl,
                                             q, k, v, g, beta,
                                             state_dtype=state_dtype)
        assert st == 0
        cw, cf = M.cursor_advance(wp, fl, L)
        assert np.array_equal(cw, nwp) and np.array_equal(cf, nfl)
        np.testing.assert_allclose(o, o_rec, rtol=1e-11, atol=1e-12)
        for b in range(nb):
            s = slot_idx[b]
            logical = Gd.gdn_replay_logical_state(pool, dr, kr, gr, s, nwp[b])
            np.testing.assert_allclose(logical, rec[s], rtol=1e-11, atol=1e-12)
            if flushing[b]:
                np.testing.assert_allclose(pool[s], rec[s], rtol=1e-11, atol=1e-12)
        wp, fl = nwp, nfl
    return pool, rec


@pytest.mark.parametrize("HV,HK", [(1, 1), (2, 1), (4, 2)])
@pytest.mark.parametrize("V,K", [(1, 2), (3, 2), (2, 4)])
@pytest.mark.parametrize("L", [1, 2, 3, 5])
def test_gdn_replay_equals_recurrence_exhaustive(HV, HK, V, K, L):
    r = np.random.default_rng(1000 + 100 * L + 10 * HV + V + K)
    T = 3 * L + 2
    nb = T + 1
    force = {t: [t] for t in range(T)}
    resets = {L + 1: [0, nb - 1], 2 * L: [1]}
    _run_pair(r, HV, HK, V, K, L, T, nb, force=force, resets=resets)


def test_gdn_L1_equals_recurrence_with_f32_pool():
    r = np.random.default_rng(40)
    pool, rec = _run_pair(r, 2, 1, 3, 4, 1, 6, 3, state_dtype="f32")
    assert np.array_equal(pool, rec, equal_nan=True)
