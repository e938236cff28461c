"""GPU parity of the KDA kernels (gated delta rule with a per-key-channel
gate: recurrent update and ReplaySSM ring decode) against the float64
oracle, through the C ABI."""

import pytest
import torch

from harness import run_gdn
from workloads import KDA, GdnWorkload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")


@pytest.mark.parametrize("io,out", [("f32", torch.float32), ("bf16", torch.float32),
                                    ("bf16", torch.bfloat16), ("f32", torch.bfloat16)])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_kda_small_shapes_and_dtypes(io, out, dk, dv):
    wl = GdnWorkload(f"kda_small_{io}_{dk}x{dv}", 5, 2, 4, dk, dv, 4, 11, 9, io, "f32",
                     4000 + dk + dv, desync=True, kda=True)
    run_gdn(wl, sample=range(5), o_dtype=out)


@pytest.mark.parametrize("L", [1, 2])
def test_kda_short_rings(L):
    wl = GdnWorkload(f"kda_L{L}", 4, 2, 4, 128, 128, L, 9, 8, "f32", "f32", 4100 + L,
                     kda=True)
    run_gdn(wl, sample=range(4))


def test_kda_full_size():
    """256 rows, 32 heads (one value head per key head), K = V = 128, L = 16,
    bf16 q/k/v, fp32 state, 128 steps; all cursors, 8 rows against the
    oracle."""
    run_gdn(KDA, sample=[0, 31, 64, 100, 128, 170, 200, 255], check_every=2)


def test_kda_full_size_desynced_rows():
    wl = GdnWorkload("kda_b256_desync", 256, 32, 32, 128, 128, 16, 40, 512, "bf16", "f32",
                     1006, desync=True, kda=True)
    run_gdn(wl, sample=[3, 77, 150, 222], standard=False)


@pytest.mark.parametrize("L,dk,dv", [(5, 128, 128), (17, 128, 128), (32, 128, 128),
                                     (48, 128, 128), (64, 64, 64)])
def test_kda_long_rings(L, dk, dv):
    """Rings past 16 entries up to the longest whose gate rows still fit the
    workgroup's LDS with bf16 inputs (48 at K = V = 128, 64 at K = V = 64)."""
    wl = GdnWorkload(f"kda_L{L}_{dk}x{dv}", 3, 2, 4, dk, dv, L, 2 * L + 3, 6, "bf16", "f32",
                     4200 + L, desync=True, kda=True)
    run_gdn(wl, sample=range(3), check_every=max(1, L // 8))


def test_kda_longest_fp32_ring():
    """fp32 q/k/v rows and the gate rows: 40 entries is the longest ring that
    fits at K = V = 128."""
    wl = GdnWorkload("kda_L40_f32", 3, 2, 4, 128, 128, 40, 2 * 40 + 3, 6, "f32", "f32", 4300,
                     desync=True, kda=True)
    run_gdn(wl, sample=range(3), check_every=5)
