"""Host metadata builder (replayssm_build_metadata, replayssm_check_copy_sources):
the oracle pinned against the device cursor rule, closed forms and the replay
method itself, then the C++ builder against the oracle, bit for bit."""

import numpy as np
import pytest

import linear_recurrence_amd as R
from oracle import mamba2 as OM
from oracle import metadata as OMD


def _steps(pos0, base0, L, T, force=None, align=0, anchors=None):
    """Drive the oracle builder for T steps, one token per step."""
    pos, base = list(pos0), list(base0)
    out = []
    for t in range(T):
        if anchors and t in anchors:
            for r, p in anchors[t].items():
                pos[r], base[r] = p, p
        fo = None if force is None else force[t]
        w, f, nb = OMD.build_metadata(pos, base, L, fo, align)
        out.append((w, f, list(base), list(pos)))
        base = nb
        pos = [p + 1 for p in pos]
    return out


# ---------------------------------------------------------------- oracle pins

@pytest.mark.parametrize("L", [1, 2, 5, 16])
def test_oracle_reproduces_the_device_cursor_rule(L):
    """One token per step from any start: w' = 0 after a flush else w + 1,
    flush iff w = L - 1 (the rule the decode kernel applies on the device)."""
    rng = np.random.default_rng(L)
    w0 = rng.integers(0, L, 40)
    n = rng.integers(1, 500, 40)
    seq = _steps(n + w0, n, L, 3 * L + 2)
    w, f = np.array(seq[0][0], np.int32), np.array(seq[0][1], np.uint8)
    np.testing.assert_array_equal(w, w0)
    for wt, ft, _, _ in seq[1:]:
        w, f = OM.cursor_advance(w, f, L)
        np.testing.assert_array_equal(w, wt)
        np.testing.assert_array_equal(f, ft)


@pytest.mark.parametrize("L,n", [(4, 7), (16, 1), (1, 3), (8, 0)])
def test_oracle_closed_form_for_a_fresh_request(L, n):
    """After a prefill of n tokens (the one-token prefill included): w_t = t mod L,
    flush iff t mod L = L - 1, and the base after T steps is n + L*floor(T/L)."""
    T = 5 * L + 3
    seq = _steps([n], [n], L, T)
    for t, (w, f, base, _) in enumerate(seq):
        assert w == [t % L]
        assert f == [1 if t % L == L - 1 else 0]
        assert base == [n + L * (t // L)]


@pytest.mark.parametrize("A,L", [(4, 16), (8, 8), (3, 5), (16, 16)])
def test_oracle_align_mode_puts_checkpoints_on_block_boundaries(A, L):
    """With block A <= L every flush after the first lands on a multiple of A,
    and a block-completing token always flushes."""
    for n in (0, 1, A - 1, A, 2 * A + 1, 37):
        seq = _steps([n], [n], L, 6 * A + 5, align=A)
        bases = [s[2][0] for s in seq]
        for (w, f, base, pos) in seq:
            assert 0 <= w[0] < L
            if (pos[0] + 1) % A == 0:
                assert f == [1]
        later = [b for b in bases if b != n]
        assert later and all(b % A == 0 for b in later)


def test_oracle_errors_and_copy_rule():
    with pytest.raises(ValueError):
        OMD.build_metadata([5], [6], 4)            # position before the checkpoint
    with pytest.raises(ValueError):
        OMD.build_metadata([10], [6], 4)           # ring would overflow
    assert OMD.copy_sources_flushed([0, 0, 0])
    assert not OMD.copy_sources_flushed([0, 2, 0])


def _recurrence(S, xs, dts, Bs, C, A, D):
    """Plain recurrence over a token sequence; returns (states, outputs)."""
    states, ys = [S.copy()], []
    for x, dt, B, c in zip(xs, dts, Bs, C):
        S = np.exp(dt * A)[:, None, None] * S + dt[:, None, None] * x[:, :, None] * B[None, None, :]
        ys.append(np.einsum("hpn,n->hp", S, c) + D[:, None] * x)
        states.append(S.copy())
    return states, ys


def test_oracle_metadata_drives_the_replay_to_the_recurrence():
    """The builder's cursors fed to the replay oracle give the recurrent
    outputs, and after every flush the checkpoint equals the recurrent state
    after decode_base tokens; a preempted request is re-prefilled and
    re-anchored mid-ring; align mode and forced flushes included."""
    rng = np.random.default_rng(7)
    H, P, N, L = 2, 3, 4, 5
    n_prefill, T = 6, 40
    total = n_prefill + T
    A = -np.exp(rng.uniform(0, np.log(16), H))
    D = rng.normal(size=H)
    xs = rng.normal(size=(total, H, P))
    dts = np.log1p(np.exp(rng.normal(size=(total, H))))
    Bs = rng.normal(size=(total, N)) / 2
    Cs = rng.normal(size=(total, N)) / 2
    S_init = rng.normal(0, 0.1, (H, P, N))
    states, ys = _recurrence(S_init, xs, dts, Bs, Cs, A, D)
    force = [[1 if rng.random() < 0.1 else 0] for _ in range(T)]
    resume_at = 17                                   # preemption: re-prefill, re-anchor
    pool = states[n_prefill][None].copy()            # checkpoint after the prefill
    xr = np.full((1, H, L, P), np.nan)
    dr = np.full((1, H, L), np.nan)
    br = np.full((1, 1, L, N), np.nan)
    pos, base = [n_prefill], [n_prefill]
    for t in range(T):
        if t == resume_at:
            pos, base = [pos[0]], [pos[0]]
            pool[0] = states[pos[0]]
        w, f, nb = OMD.build_metadata(pos, base, L, force[t], align_block=4)
        p = pos[0]
        y, _, _, _ = OM.replay_step(pool, xr, dr, br, np.array([0]), np.array(w, np.int32),
                                    np.array(f, np.uint8), xs[p][None], np.log(np.expm1(dts[p]))[None],
                                    A, Bs[p][None, None], Cs[p][None, None], D=D)
        np.testing.assert_allclose(y[0], ys[p], rtol=1e-10, atol=1e-12)
        if f[0]:
            np.testing.assert_allclose(pool[0], states[nb[0]], rtol=1e-10, atol=1e-13)
        base, pos = nb, [p + 1]


# ------------------------------------------------------ C++ builder vs oracle

@pytest.mark.parametrize("L", [1, 3, 16, 64])
@pytest.mark.parametrize("align", [0, 2, 8, 16])
def test_builder_matches_oracle(L, align):
    rng = np.random.default_rng(100 * L + align)
    n = 97
    w0 = rng.integers(0, L, n)
    base = rng.integers(0, 10_000, n).astype(np.int64)
    if align:
        # in align mode, start within one block of the checkpoint
        w0 = np.minimum(w0, min(L, align) - 1)
    pos = (base + w0).astype(np.int64)
    obase = base.tolist()
    for t in range(3 * L + 5):
        force = (rng.random(n) < 0.05).astype(np.uint8)
        if t % 7 == 3:                               # re-anchor a few rows (resume)
            for r in rng.choice(n, 5, replace=False):
                base[r] = pos[r]
                obase[r] = int(pos[r])
        ow, of, onb = OMD.build_metadata(pos.tolist(), obase, L, force.tolist(), align)
        w, f = R.build_metadata(pos, base, L, force, align)
        np.testing.assert_array_equal(w, np.array(ow, np.int32))
        np.testing.assert_array_equal(f, np.array(of, np.uint8))
        np.testing.assert_array_equal(base, np.array(onb, np.int64))
        obase = onb
        pos = pos + 1


def test_builder_rejects_out_of_range_rows_and_writes_nothing():
    pos = np.array([10, 11, 12], np.int64)
    base = np.array([10, 10, 13], np.int64)        # row 2: pos < base
    keep = base.copy()
    with pytest.raises(R.RssmError):
        R.build_metadata(pos, base, 4)
    np.testing.assert_array_equal(base, keep)
    base = np.array([10, 10, 6], np.int64)         # row 2: w = 6 >= L
    with pytest.raises(R.RssmError):
        R.build_metadata(pos, base, 4)
    with pytest.raises(R.RssmError):
        R.build_metadata(np.array([-1], np.int64), np.array([-1], np.int64), 4)
    with pytest.raises(R.RssmError):
        R.build_metadata(pos, np.array([10, 10, 10], np.int64), 0)
    w, f = R.build_metadata(np.zeros(0, np.int64), np.zeros(0, np.int64), 4)
    assert w.size == 0 and f.size == 0


def test_builder_L1_and_one_token_prefill():
    w, f = R.build_metadata(np.array([5, 1], np.int64), np.array([5, 1], np.int64), 1)
    np.testing.assert_array_equal(w, [0, 0])
    np.testing.assert_array_equal(f, [1, 1])
    base = np.array([1], np.int64)
    w, f = R.build_metadata(np.array([1], np.int64), base, 16)
    assert w[0] == 0 and f[0] == 0 and base[0] == 1


def test_copy_source_rule():
    R.check_copy_sources(np.zeros(4, np.int32))
    R.check_copy_sources(np.zeros(0, np.int32))
    with pytest.raises(R.RssmError):
        R.check_copy_sources(np.array([0, 0, 3], np.int32))


def test_oracle_flush_first_order_is_a_stable_partition():
    """Flush rows first, each class in increasing row index: the same as a
    stable sort on the key (flag == 0), and a permutation of the rows."""
    rng = np.random.default_rng(5)
    for n in (0, 1, 7, 64, 130):
        fl = rng.integers(0, 3, n).astype(np.uint8)  # any nonzero value flushes
        order = OMD.flush_first_order(fl)
        assert sorted(order) == list(range(n))
        assert order == np.argsort(fl == 0, kind="stable").tolist()
        nf = int((fl != 0).sum())
        assert all(fl[r] != 0 for r in order[:nf]) and all(fl[r] == 0 for r in order[nf:])


def test_flush_first_order_helper_matches_oracle():
    rng = np.random.default_rng(6)
    for n in (0, 1, 5, 64, 100, 512):
        for p in (0.0, 1.0 / 16, 0.5, 1.0):
            fl = (rng.random(n) < p).astype(np.uint8) * rng.integers(1, 4, n).astype(np.uint8)
            assert R.flush_first_order(fl).tolist() == OMD.flush_first_order(fl)
    with pytest.raises(TypeError):
        R.flush_first_order(np.zeros(4, np.int32))
