"""Pins of the GDN speculative-verify oracle: every verified draft output and
every exactly folded state equals the plain recurrence over the committed
tokens followed by the drafts; rejected drafts leave no trace."""

import numpy as np
import pytest

from oracle import gdn as OG
from oracle import gdn_spec as OS
from oracle.mamba2 import ST_RING_OVERFLOW


def _tokens(rng, n, HK, HV, K, V):
    def unit(shape):
        a = rng.normal(size=shape)
        return a / np.linalg.norm(a, axis=-1, keepdims=True)
    return dict(q=unit((n, HK, K)), k=unit((n, HK, K)), v=rng.normal(size=(n, HV, V)),
                g=np.exp(-np.log1p(np.exp(rng.normal(size=(n, HV))))),
                beta=1 / (1 + np.exp(-rng.normal(size=(n, HV)))))


def _recurrent_outputs(S, tok, idx):
    """Outputs and final state of the recurrence over tokens idx (one row)."""
    S = S.copy()[None]
    outs = []
    for i in idx:
        o = OG.gdn_standard_step(S, np.array([0]), tok["q"][i][None], tok["k"][i][None],
                                 tok["v"][i][None], tok["g"][i][None], tok["beta"][i][None])
        outs.append(o[0])
    return outs, S[0]


@pytest.mark.parametrize("L,T", [(8, 3), (6, 3), (16, 4), (4, 2), (2, 1)])
def test_spec_rounds_match_the_recurrence(L, T):
    """Many verify/commit rounds with random acceptance on one row: each
    draft output equals the recurrence over the committed history plus the
    drafts before it; each exact fold equals the recurrent state."""
    rng = np.random.default_rng(L * 10 + T)
    HK, HV, K, V = 2, 4, 3, 5
    S_init = rng.normal(0, 0.2, (HV, V, K))
    n_tok = 200
    tok = _tokens(rng, n_tok, HK, HV, K, V)
    state = S_init[None].copy()
    dr = np.full((1, HV, L, V), np.nan)
    kr = np.full((1, HK, L, K), np.nan)
    gr = np.full((1, HV, L), np.nan)
    vr = np.full((1, HV, L, V), np.nan)
    br = np.full((1, HV, L), np.nan)
    wp = np.zeros(1, np.int32)
    committed = []          # token indices in the committed history
    nxt = 0                 # next unused token (drafts are fresh tokens each round)
    flushes = 0
    while nxt + T <= n_tok:
        drafts = list(range(nxt, nxt + T))
        nxt += T
        o, st = OS.gdn_spec_verify(state, dr, kr, gr, vr, br, np.array([0]), wp,
                                   tok["q"][drafts][None], tok["k"][drafts][None],
                                   tok["v"][drafts][None], tok["g"][drafts][None],
                                   tok["beta"][drafts][None])
        assert st == 0
        ref, _ = _recurrent_outputs(S_init, tok, committed + drafts)
        for t in range(T):
            np.testing.assert_allclose(o[0, t], ref[len(committed) + t], rtol=1e-9, atol=1e-12)
        a = int(rng.integers(0, T + 1))
        committed += drafts[:a]
        wp, fl, st = OS.gdn_spec_commit(state, kr, gr, vr, br, np.array([0]), wp,
                                        np.array([a]), T)
        assert st == 0
        if fl[0]:
            flushes += 1
            _, S_ref = _recurrent_outputs(S_init, tok, committed)
            np.testing.assert_allclose(state[0], S_ref, rtol=1e-9, atol=1e-12)
            assert wp[0] == 0
        else:
            assert wp[0] + T <= L
    assert flushes > 0


def test_forced_flush_and_bad_cursors():
    rng = np.random.default_rng(1)
    HK, HV, K, V, L, T = 1, 2, 3, 3, 6, 2
    tok = _tokens(rng, 4, HK, HV, K, V)
    S_init = rng.normal(0, 0.2, (HV, V, K))
    state = S_init[None].copy()
    rings = [np.zeros((1, HV, L, V)), np.zeros((1, HK, L, K)), np.zeros((1, HV, L)),
             np.zeros((1, HV, L, V)), np.zeros((1, HV, L))]
    d = [0, 1]
    OS.gdn_spec_verify(state, *rings, np.array([0]), np.array([0], np.int32),
                       tok["q"][d][None], tok["k"][d][None], tok["v"][d][None],
                       tok["g"][d][None], tok["beta"][d][None])
    wp, fl, _ = OS.gdn_spec_commit(state, *rings[1:], np.array([0]), np.array([0], np.int32),
                                   np.array([1]), T, force_flush=np.array([1]))
    assert fl[0] == 1 and wp[0] == 0
    _, S_ref = _recurrent_outputs(S_init, tok, [0])
    np.testing.assert_allclose(state[0], S_ref, rtol=1e-12)
    # a verify that would run past the ring is refused
    o, st = OS.gdn_spec_verify(state, *rings, np.array([0]), np.array([5], np.int32),
                               tok["q"][d][None], tok["k"][d][None], tok["v"][d][None],
                               tok["g"][d][None], tok["beta"][d][None])
    assert st & ST_RING_OVERFLOW and np.isnan(o).all()


@pytest.mark.parametrize("L,T", [(8, 3), (16, 4), (2, 1)])
def test_deferred_fold_rounds_match_the_recurrence(L, T):
    """The deferred-fold rounds composed from the same oracle steps: the
    advance keeps w' = (folded ? 0 : w) + accepted and marks the row when
    w' + T > L (or forced); the next verify first folds entries 0..w'-1 by
    the exact recurrence and verifies at entry 0.  Every draft output equals
    the recurrence over the committed history plus the drafts before it, and
    every fold equals the recurrent state: the rule keeps each verify inside
    the ring and loses no committed token."""
    rng = np.random.default_rng(L * 100 + T)
    HK, HV, K, V = 2, 4, 3, 5
    S_init = rng.normal(0, 0.2, (HV, V, K))
    n_tok = 160
    tok = _tokens(rng, n_tok, HK, HV, K, V)
    state = S_init[None].copy()
    rings = [np.full((1, HV, L, V), np.nan), np.full((1, HK, L, K), np.nan),
             np.full((1, HV, L), np.nan), np.full((1, HV, L, V), np.nan),
             np.full((1, HV, L), np.nan)]
    kh = np.arange(HV) // (HV // HK)
    w, flag = 0, False
    committed, nxt, folds = [], 0, 0
    while nxt + T <= n_tok:
        if flag:
            state[0] = OS.exact_fold(state[0], rings[1], rings[2], rings[3], rings[4], 0, w, kh)
            _, S_ref = _recurrent_outputs(S_init, tok, committed)
            np.testing.assert_allclose(state[0], S_ref, rtol=1e-9, atol=1e-12)
            folds += 1
            w = 0
        assert w + T <= L
        drafts = list(range(nxt, nxt + T))
        nxt += T
        o, st = OS.gdn_spec_verify(state, *rings, np.array([0]), np.array([w], np.int32),
                                   tok["q"][drafts][None], tok["k"][drafts][None],
                                   tok["v"][drafts][None], tok["g"][drafts][None],
                                   tok["beta"][drafts][None])
        assert st == 0
        ref, _ = _recurrent_outputs(S_init, tok, committed + drafts)
        for t in range(T):
            np.testing.assert_allclose(o[0, t], ref[len(committed) + t], rtol=1e-9, atol=1e-12)
        a = int(rng.integers(0, T + 1))
        committed += drafts[:a]
        w += a
        flag = w + T > L or rng.random() < 0.1
    assert folds > 0
