"""Pins for oracle.mamba2 (CPU only).

The standard update is pinned to closed forms (geometric series under
constant inputs, a cumulative sum when A = 0, frozen state when dt = 0),
brute-force loops for the output contraction, the gate's known values and
NaN-poisoned groups and slots.  The replay is pinned to the standard update:
same outputs and same logical state at every step over small exhaustive
schedules (every write position, forced flushes, resets), L = 1 equal to the
standard update, and the stored checkpoint after each flush equal to the
recurrent state.
"""

import math

import numpy as np
import pytest

from oracle import mamba2 as M
from oracle.numerics import round_bf16


def _softplus_py(v):
    return math.log1p(math.exp(v))


def _rand_problem(r, nb, H, P, N, G, slots):
    return dict(
        x=r.standard_normal((nb, H, P)),
        dt_raw=r.standard_normal((nb, H)),
        B=r.standard_normal((nb, G, N)) * 0.25,
        C=r.standard_normal((nb, G, N)) * 0.25,
        z=r.standard_normal((nb, H, P)),
    )


def _params(r, H):
    A = -np.exp(r.uniform(0, math.log(16), H))
    dt_bias = np.log(np.expm1(r.uniform(1e-3, 1e-1, H)))
    D = r.standard_normal(H)
    return A, D, dt_bias


def test_standard_geometric_closed_form():
    """Constant inputs: S_T = a^T S0 + dt x B^T (1 - a^T) / (1 - a)."""
    r = np.random.default_rng(10)
    H, P, N, G, T = 3, 5, 4, 1, 7
    A, D, dt_bias = _params(r, H)
    S0 = r.standard_normal((1, H, P, N)) * 0.1
    x = r.standard_normal((1, H, P))
    dt_raw = r.standard_normal((1, H))
    B = r.standard_normal((1, G, N))
    C = r.standard_normal((1, G, N))
    state = S0.copy()
    for _ in range(T):
        y = M.ssu_standard_step(state, [0], x, dt_raw, A, B, C, D=D,
                                dt_bias=dt_bias)
    for h in range(H):
        dt = _softplus_py(dt_raw[0, h] + dt_bias[h])
        a = math.exp(dt * A[h])
        for p in range(P):
            for n in range(N):
                want = (a ** T * S0[0, h, p, n]
                        + dt * x[0, h, p] * B[0, 0, n] * (1 - a ** T) / (1 - a))
                assert state[0, h, p, n] == pytest.approx(want, rel=1e-12, abs=1e-14)
            # brute-force output contraction over dstate
            yp = sum(state[0, h, p, n] * C[0, 0, n] for n in range(N))
            yp += D[h] * x[0, h, p]
            assert y[0, h, p] == pytest.approx(yp, rel=1e-12, abs=1e-14)


def test_standard_zero_A_is_cumulative_sum_and_no_softplus():
    """A = 0: S_T = S0 + sum_t dt_t x_t B_t^T; dt_softplus=False uses dt_raw + bias."""
    r = np.random.default_rng(11)
    nb, H, P, N, G, T = 2, 2, 3, 5, 1, 6
    A = np.zeros(H)
    dt_bias = r.uniform(0.1, 0.5, H)
    S0 = r.standard_normal((nb, H, P, N))
    state = S0.copy()
    acc = S0.copy()
    for t in range(T):
        pr = _rand_problem(r, nb, H, P, N, G, nb)
        M.ssu_standard_step(state, [0, 1], pr["x"], pr["dt_raw"], A, pr["B"],
                            pr["C"], dt_bias=dt_bias, dt_softplus=False)
        for b in range(nb):
            for h in range(H):
                dt = pr["dt_raw"][b, h] + dt_bias[h]
                for p in range(P):
                    for n in range(N):
                        acc[b, h, p, n] += dt * pr["x"][b, h, p] * pr["B"][b, 0, n]
    assert np.allclose(state, acc, rtol=1e-13, atol=1e-13)


def test_standard_dt_zero_freezes_state_and_D_term():
    """dt -> 0 (huge negative bias, softplus -> 0): state unchanged; y = S0 C + D x."""
    r = np.random.default_rng(12)
    H, P, N = 2, 4, 3
    S0 = r.standard_normal((1, H, P, N))
    state = S0.copy()
    A = -np.ones(H)
    D = np.array([0.5, -2.0])
    x = r.standard_normal((1, H, P))
    C = r.standard_normal((1, 1, N))
    y = M.ssu_standard_step(state, [0], x, np.zeros((1, H)), A,
                            r.standard_normal((1, 1, N)), C, D=D,
                            dt_bias=np.full(H, -800.0))
    assert np.array_equal(state, S0)
    for h in range(H):
        for p in range(P):
            want = sum(S0[0, h, p, n] * C[0, 0, n] for n in range(N)) + D[h] * x[0, h, p]
            assert y[0, h, p] == pytest.approx(want, rel=1e-13)


def test_standard_gate_values():
    r = np.random.default_rng(13)
    H, P, N = 1, 3, 2
    args = dict(dt_raw=np.zeros((1, H)), A=-np.ones(H),
                B=r.standard_normal((1, 1, N)), C=r.standard_normal((1, 1, N)),
                D=np.ones(H))
    S0 = r.standard_normal((1, H, P, N))
    x = r.standard_normal((1, H, P))
    y_plain = M.ssu_standard_step(S0.copy(), [0], x, **args)
    for zv, factor in ((0.0, 0.0), (1.0, 1 / (1 + math.exp(-1))),
                       (-1.0, -1 / (1 + math.exp(1)))):
        z = np.full((1, H, P), zv)
        y = M.ssu_standard_step(S0.copy(), [0], x, z=z, **args)
        assert np.allclose(y, y_plain * factor, rtol=1e-14, atol=0)


def test_standard_groups_and_slots_are_indexed_correctly():
    """Heads read group h // (H/G); rows touch only their own slot."""
    r = np.random.default_rng(14)
    H, P, N, G = 4, 2, 3, 2
    A, D, dt_bias = _params(r, H)
    pool = np.full((6, H, P, N), np.nan)
    pool[4] = r.standard_normal((H, P, N))
    pool[1] = r.standard_normal((H, P, N))
    x = r.standard_normal((2, H, P))
    dt_raw = r.standard_normal((2, H))
    B = r.standard_normal((2, G, N))
    C = r.standard_normal((2, G, N))
    for bad in range(G):
        Bp, Cp = B.copy(), C.copy()
        Bp[:, bad] = np.nan
        Cp[:, bad] = np.nan
        st = pool.copy()
        y = M.ssu_standard_step(st, [4, 1], x, dt_raw, A, Bp, Cp, D=D,
                                dt_bias=dt_bias)
        heads_bad = np.arange(H) // (H // G) == bad
        assert np.isnan(y[:, heads_bad]).all()
        assert np.isfinite(y[:, ~heads_bad]).all()
    st = pool.copy()
    M.ssu_standard_step(st, [4, 1], x, dt_raw, A, B, C, D=D, dt_bias=dt_bias)
    for s in (0, 2, 3, 5):
        assert np.isnan(st[s]).all()
    assert np.isfinite(st[[1, 4]]).all()
    # row 0 -> slot 4 alone gives the same slot-4 state
    st1 = pool.copy()
    M.ssu_standard_step(st1, [4], x[:1], dt_raw[:1], A, B[:1], C[:1], D=D,
                        dt_bias=dt_bias)
    assert np.array_equal(st1[4], st[4])


def test_standard_bf16_storage_rounds_to_nearest():
    r = np.random.default_rng(15)
    H, P, N = 2, 8, 16
    A, D, dt_bias = _params(r, H)
    S0 = round_bf16(r.standard_normal((1, H, P, N)) * 0.1)
    pr = _rand_problem(r, 1, H, P, N, 1, 1)
    exact = S0.copy()
    M.ssu_standard_step(exact, [0], pr["x"], pr["dt_raw"], A, pr["B"], pr["C"],
                        dt_bias=dt_bias, state_dtype="f64")
    st = S0.copy()
    M.ssu_standard_step(st, [0], pr["x"], pr["dt_raw"], A, pr["B"], pr["C"],
                        dt_bias=dt_bias, state_dtype="bf16")
    bits = st.astype(np.float32).view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)                 # bf16 representable
    # nearest: within half a bf16 ulp (2^-8 relative) plus the fp32 step
    assert np.all(np.abs(st - exact) <= np.abs(exact) * (2.0**-8 + 2.0**-23) + 1e-45)
    assert not np.array_equal(st, exact)


# ---------------------------------------------------------------- replay pins

def _run_pair(r, H, G, P, N, L, T, nb, state_dtype="f64", force=None,
              resets=None):
    """Run replay and recurrence side by side; compare every step.

    force[t] / resets[t]: rows forced to flush / reset before step t.
    """
    A, D, dt_bias = _params(r, H)
    slots = nb + 2
    pool = np.full((slots, H, P, N), np.nan)
    slot_idx = np.arange(nb)[::-1] + 1
    for s in slot_idx:
        pool[s] = r.standard_normal((H, P, N)) * 0.1
    rec = pool.copy()
    xr = np.full((slots, H, L, P), np.nan)
    dr = np.full((slots, H, L), np.nan)
    br = np.full((slots, G, L, N), np.nan)
    wp = np.zeros(nb, np.int32)
    fl = np.full(nb, 1 if L == 1 else 0, np.uint8)
    for t in range(T):
        if resets and t in resets:
            for b in resets[t]:
                fresh = r.standard_normal((H, P, N)) * 0.1
                pool[slot_idx[b]] = fresh
                rec[slot_idx[b]] = fresh
            wp, fl = M.ring_reset(wp, fl, resets[t], L)
        if force and t in force:
            fl = fl.copy()
            fl[force[t]] = 1
        pr = _rand_problem(r, nb, H, P, N, G, slots)
        y_rec = M.ssu_standard_step(rec, slot_idx, pr["x"], pr["dt_raw"], A,
                                    pr["B"], pr["C"], D=D, z=pr["z"],
                                    dt_bias=dt_bias, state_dtype=state_dtype)
        flushing = fl.astype(bool).copy()
        y, nwp, nfl, status = M.replay_step(
            pool, xr, dr, br, slot_idx, wp, fl, pr["x"], pr["dt_raw"], A,
            pr["B"], pr["C"], D=D, z=pr["z"], dt_bias=dt_bias,
            state_dtype=state_dtype)
        assert status == 0
        cw, cf = M.cursor_advance(wp, fl, L)
        assert np.array_equal(cw, nwp) and np.array_equal(cf, nfl)
        assert np.isfinite(y).all()
        np.testing.assert_allclose(y, y_rec, rtol=1e-11, atol=1e-12)
        for b in range(nb):
            s = slot_idx[b]
            logical = M.replay_logical_state(pool, xr, dr, br, s, nwp[b], A)
            np.testing.assert_allclose(logical, rec[s], rtol=1e-11, atol=1e-12)
            if flushing[b]:
                # the stored checkpoint itself is the recurrent state
                np.testing.assert_allclose(pool[s], rec[s], rtol=1e-11, atol=1e-12)
        wp, fl = nwp, nfl
    return pool, rec


@pytest.mark.parametrize("H,G", [(1, 1), (2, 1), (2, 2), (4, 2)])
@pytest.mark.parametrize("P,N", [(1, 1), (2, 3), (3, 2)])
@pytest.mark.parametrize("L", [1, 2, 3, 4, 5])
def test_replay_equals_recurrence_exhaustive(H, G, P, N, L):
    """Every row is forced to flush at a different step, so rows pass through
    every write position and every flush position; resets hit mid-ring."""
    r = np.random.default_rng(100 * L + 10 * H + P + N)
    T = 3 * L + 2
    nb = T + 1
    force = {t: [t] for t in range(T)}          # row t forced at step t
    resets = {L + 1: [0, nb - 1], 2 * L: [1]}
    _run_pair(r, H, G, P, N, L, T, nb, force=force, resets=resets)


def test_replay_L1_equals_standard_update_bf16():
    """L = 1: every step is a flush, so replay is the standard update,
    including the bf16 rounding of the stored state on every step."""
    r = np.random.default_rng(21)
    pool, rec = _run_pair(r, 2, 1, 4, 8, 1, 6, 3, state_dtype="bf16")
    assert np.array_equal(pool, rec, equal_nan=True)


def test_replay_bf16_flush_rounds_once_per_period():
    """With a bf16 pool the replay stores, at each flush, the bf16 rounding of
    the exact recurrence restarted from the previous stored checkpoint, and
    writes nothing in between."""
    r = np.random.default_rng(22)
    H, G, P, N, L = 2, 1, 3, 4, 4
    A, D, dt_bias = _params(r, H)
    pool = round_bf16(r.standard_normal((1, H, P, N)) * 0.1)
    ck = pool.copy()
    xr = np.full((1, H, L, P), np.nan)
    dr = np.full((1, H, L), np.nan)
    br = np.full((1, G, L, N), np.nan)
    wp, fl = np.zeros(1, np.int32), np.zeros(1, np.uint8)
    flushes = 0
    for t in range(3 * L):
        pr = _rand_problem(r, 1, H, P, N, G, 1)
        M.ssu_standard_step(ck, [0], pr["x"], pr["dt_raw"], A, pr["B"],
                            pr["C"], dt_bias=dt_bias)
        before = pool.copy()
        _, wp, fl2, _ = M.replay_step(pool, xr, dr, br, [0], wp, fl, pr["x"],
                                      pr["dt_raw"], A, pr["B"], pr["C"],
                                      dt_bias=dt_bias, state_dtype="bf16")
        if fl[0]:
            flushes += 1
            assert np.array_equal(pool, round_bf16(ck))
            ck = pool.copy()
        else:
            assert np.array_equal(pool, before)
        fl = fl2
    assert flushes == 3


def test_cursor_closed_form():
    """w_t = (w0 + t) mod L; flush at t iff (w0 + t) mod L == L - 1;
    flushes in T steps = floor((w0 + T) / L)."""
    for L in range(1, 9):
        w0 = np.arange(L, dtype=np.int32)
        wp = w0.copy()
        fl = (wp == L - 1).astype(np.uint8)
        count = np.zeros(L, int)
        T = 5 * L + 3
        for t in range(T):
            assert np.array_equal(wp, (w0 + t) % L)
            assert np.array_equal(fl.astype(bool), (w0 + t) % L == L - 1)
            count += fl
            wp, fl = M.cursor_advance(wp, fl, L)
        assert np.array_equal(count, (w0 + T) // L)


def test_ring_reset():
    wp, fl = M.ring_reset([3, 2, 1], [1, 0, 0], [0, 2], 4)
    assert wp.tolist() == [0, 2, 0] and fl.tolist() == [0, 0, 0]
    wp, fl = M.ring_reset([0, 0], [1, 1], [1], 1)
    assert wp.tolist() == [0, 0] and fl.tolist() == [1, 1]


def test_replay_status_bits():
    r = np.random.default_rng(23)
    H, G, P, N, L = 2, 1, 2, 3, 4
    A, D, dt_bias = _params(r, H)
    pool = r.standard_normal((4, H, P, N))
    xr = np.zeros((4, H, L, P))
    dr = np.zeros((4, H, L))
    br = np.zeros((4, G, L, N))
    pr = _rand_problem(r, 4, H, P, N, G, 4)
    y, nwp, nfl, st = M.replay_step(
        pool, xr, dr, br, np.array([0, 9, 2, 3]), np.array([0, 0, 7, 3]),
        np.array([0, 0, 0, 0]), pr["x"], pr["dt_raw"], A, pr["B"], pr["C"],
        dt_bias=dt_bias)
    assert st == M.ST_BAD_SLOT | M.ST_BAD_WRITE_POS | M.ST_RING_OVERFLOW
    assert np.isnan(y[1]).all() and np.isfinite(y[[0, 2, 3]]).all()
    assert nwp.tolist() == [1, 0, 0, 0]
