"""Pins of the stochastic-rounding oracle: Philox4x64-10 against numpy's
Philox bit generator (an independent implementation of the same published
generator), and the rounding rule against its defining properties
(exhaustively over the 2^16 random values)."""

import numpy as np
import pytest

from oracle import mamba2 as OM
from oracle import numerics as NU


@pytest.mark.parametrize("key", [(0, 0), (123, 456), (2**64 - 1, 2**63 + 5), (0xDEADBEEF, 7)])
@pytest.mark.parametrize("ctr", [(1, 0, 0, 0), (5, 0, 0, 0), (2**40 + 3, 0, 0, 0),
                                 (17, 9, 2**33, 1)])
def test_philox_matches_numpy(key, ctr):
    # numpy's generator advances its 256-bit counter before each block
    c = list(ctr)
    c_prev = ((c[0] + (c[1] << 64) + (c[2] << 128) + (c[3] << 192)) - 1)
    prev = [(c_prev >> (64 * i)) & (2**64 - 1) for i in range(4)]
    ref = np.random.Philox(counter=prev, key=list(key)).random_raw(4)
    got = NU.philox4x64_10(np.array([ctr], np.uint64), key)[0]
    np.testing.assert_array_equal(got, ref)


def test_philox_vectorised_blocks_match_numpy_stream():
    """Consecutive counters = numpy's consecutive output blocks."""
    key = (31337, 271828)
    n = 64
    ctr = np.zeros((n, 4), np.uint64)
    ctr[:, 0] = np.arange(1, n + 1, dtype=np.uint64)
    got = NU.philox4x64_10(ctr, key).reshape(-1)
    ref = np.random.Philox(counter=0, key=list(key)).random_raw(4 * n)
    np.testing.assert_array_equal(got, ref)


def _all_r(v):
    a = np.full(65536, v, np.float32)
    return NU.round_bf16_sr_from_f32(a, np.arange(65536, dtype=np.uint32))


@pytest.mark.parametrize("v", [1.0 + 2**-10, -3.3, 0.1, 123.456, -1e-30, 3.0e38, 2.0 - 2**-23,
                               1e-40])
def test_sr_is_exactly_unbiased_over_all_random_values(v):
    v32 = np.float32(v)
    out = _all_r(v32).astype(np.float64)
    down = NU.round_bf16_from_f32(np.array([v32]))[0]
    vals = np.unique(out)
    assert len(vals) <= 2
    # the two candidates bracket v and are adjacent bf16 values
    assert vals.min() <= float(v32) <= vals.max()
    # mean over every 16-bit draw equals the fp32 value exactly (unbiased),
    # unless rounding up overflows to infinity
    if np.isfinite(out).all():
        assert out.sum() / 65536 == pytest.approx(float(v32), rel=0, abs=0)
    assert down in vals or np.isinf(out).any()


def test_sr_keeps_representable_values_and_specials():
    for v in (0.0, -0.0, 1.0, -2.5, 0.15625, 3.0e38):
        v32 = NU.round_bf16_from_f32(np.array([np.float32(v)]))[0]
        assert (_all_r(v32) == v32).all()
    for v in (np.inf, -np.inf):
        assert (_all_r(np.float32(v)) == v).all()
    assert np.isnan(_all_r(np.float32(np.nan))).all()


def test_sr_is_sign_symmetric():
    rng = np.random.default_rng(3)
    a = rng.normal(size=4096).astype(np.float32)
    r = rng.integers(0, 65536, 4096).astype(np.uint32)
    np.testing.assert_array_equal(NU.round_bf16_sr_from_f32(-a, r), -NU.round_bf16_sr_from_f32(a, r))


def test_sr_probability_matches_the_dropped_bits():
    """P(round away from zero) = dropped 16 bits / 2^16, e.g. 1/4 here."""
    v = np.float32(1.0 + 2**-9)              # dropped bits 0x4000 of 0x10000
    out = _all_r(v)
    assert (out > 1.0).sum() == 0x4000


def test_sr_bits_layout():
    """Element e of a tile takes bits 16*(e%4) of word (e%16)//4 of the block
    with counter tile*n/16 + e//16."""
    tile, n, seed, off = 37, 256, 99, 12
    bits = NU.sr_bits(tile, n, seed, off)
    for e in (0, 3, 4, 15, 16, 100, 255):
        blk = NU.philox4x64_10(np.array([[tile * n // 16 + e // 16, 0, 0, 0]], np.uint64),
                               (seed, off))[0]
        w = int(blk[(e % 16) // 4])
        assert bits[e] == (w >> (16 * (e % 4))) & 0xFFFF


def test_sr_state_store_in_the_standard_step():
    """The standard step's SR store equals element-wise SR of the fp32 state
    with the tile's bits; a different offset gives different bits."""
    rng = np.random.default_rng(5)
    H, P, N, ns = 2, 4, 16, 3
    pool = NU.round_bf16(rng.normal(0, 0.1, (ns, H, P, N)))
    x = rng.normal(size=(1, H, P))
    dt = rng.normal(size=(1, H))
    A = -np.exp(rng.uniform(0, 2, H))
    B = rng.normal(size=(1, 1, N)) / 4
    C = rng.normal(size=(1, 1, N)) / 4
    p1, p2, p3 = pool.copy(), pool.copy(), pool.copy()
    OM.ssu_standard_step(p1, np.array([2]), x, dt, A, B, C, state_dtype="bf16",
                         rounding="stochastic", sr_seed=7, sr_offset=1)
    OM.ssu_standard_step(p2, np.array([2]), x, dt, A, B, C, state_dtype="f64")
    OM.ssu_standard_step(p3, np.array([2]), x, dt, A, B, C, state_dtype="bf16",
                         rounding="stochastic", sr_seed=7, sr_offset=2)
    for h in range(H):
        ref = NU.round_bf16_sr_from_f32(p2[2, h].reshape(-1).astype(np.float32),
                                        NU.sr_bits(2 * H + h, P * N, 7, 1))
        np.testing.assert_array_equal(p1[2, h].reshape(-1), ref.astype(np.float64))
    assert not np.array_equal(p1[2], p3[2])
    np.testing.assert_array_equal(p1[:2], pool[:2])
