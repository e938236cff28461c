"""Pins for oracle.numerics: bf16 rounding against torch, softplus closed forms."""

import math

import numpy as np
import pytest
import torch

from oracle.numerics import (round_bf16, round_bf16_from_f32, round_f32,
                             silu_gate, softplus, store)


def _torch_bf16(a32):
    return torch.from_numpy(a32).to(torch.bfloat16).to(torch.float32).numpy()


def test_bf16_matches_torch_on_random_values():
    r = np.random.default_rng(0)
    a = (r.standard_normal(200_000) * np.exp(r.uniform(-100, 80, 200_000))).astype(np.float32)
    got = round_bf16_from_f32(a)
    assert np.array_equal(got.view(np.uint32), _torch_bf16(a).view(np.uint32))


def test_bf16_matches_torch_on_ties_and_specials():
    r = np.random.default_rng(1)
    hi = r.integers(0, 0x7F80, 50_000, dtype=np.uint32)
    sign = r.integers(0, 2, 50_000, dtype=np.uint32) << np.uint32(31)
    ties = ((hi << np.uint32(16)) | np.uint32(0x8000) | sign).view(np.float32)
    near = ((hi << np.uint32(16)) | np.uint32(0x7FFF) | sign).view(np.float32)
    subn = (r.integers(1, 0x7FFFFF, 20_000, dtype=np.uint32)).view(np.float32)
    spec = np.array([0.0, -0.0, np.inf, -np.inf, 3.4028235e38, -3.4028235e38,
                     1e-45, 1.0], dtype=np.float32)
    for a in (ties, near, subn, spec):
        assert np.array_equal(round_bf16_from_f32(a).view(np.uint32),
                              _torch_bf16(a).view(np.uint32))
    nan = round_bf16_from_f32(np.array([np.nan], np.float32))
    assert np.isnan(nan).all()


def test_bf16_known_answers():
    # bf16 keeps 7 explicit mantissa bits: spacing near 1 is 2^-7.
    vals = np.array([1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-8 + 2**-20, 256 + 1],
                     dtype=np.float32)
    want = np.array([1.0, 1 + 2**-6, 1 + 2**-7, 256.0], dtype=np.float32)
    assert np.array_equal(round_bf16_from_f32(vals), want)
    assert round_bf16_from_f32(np.array([3.4028235e38], np.float32))[0] == np.inf


def test_round_f32_and_store():
    a = np.array([1 / 3, 2 / 3, 1e-40, 1e30], dtype=np.float64)
    assert np.array_equal(round_f32(a), a.astype(np.float32).astype(np.float64))
    assert np.array_equal(store(a, "f64"), a)
    # f64 -> f32 -> bf16: 1 + 2^-8 + 2^-30 rounds to 1 + 2^-8 in fp32 (a bf16
    # tie), which then rounds to even (1.0); a single rounding would give 1 + 2^-7.
    assert store(np.array([1 + 2**-8 + 2**-30]), "bf16")[0] == 1.0
    b = store(np.linspace(-3, 3, 1001), "bf16")
    assert np.all((b.astype(np.float32).view(np.uint32) & 0xFFFF) == 0)
    with pytest.raises(ValueError):
        store(a, "f16")


def test_softplus_closed_forms():
    assert softplus(0.0) == pytest.approx(math.log(2.0), rel=1e-15)
    for v in np.linspace(-30, 30, 121):
        assert softplus(v) == pytest.approx(math.log1p(math.exp(v)), rel=1e-13)
    assert softplus(800.0) == 800.0          # no overflow for large v
    assert softplus(-800.0) == 0.0 or softplus(-800.0) < 1e-300
    assert softplus(-50.0) == pytest.approx(math.exp(-50.0), rel=1e-12)


def test_silu_gate_values():
    y = np.array([2.0, 2.0, 2.0, 2.0])
    z = np.array([0.0, 1.0, -1.0, 40.0])
    got = silu_gate(y, z)
    want = [0.0, 2.0 / (1 + math.exp(-1.0)), -2.0 / (1 + math.exp(1.0)), 80.0]
    assert np.allclose(got, want, rtol=1e-14, atol=0)
