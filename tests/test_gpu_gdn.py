"""GPU parity of the gated-delta-rule kernels (recurrent update and ReplaySSM
ring decode) against the float64 oracle, through the C ABI."""

import pytest
import torch

from harness import run_gdn
from workloads import GDN, GdnWorkload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")


@pytest.mark.parametrize("io,out", [("f32", torch.float32), ("bf16", torch.float32),
                                    ("bf16", torch.bfloat16), ("f32", torch.bfloat16)])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_gdn_small_shapes_and_dtypes(io, out, dk, dv):
    wl = GdnWorkload(f"gdn_small_{io}_{dk}x{dv}", 5, 2, 4, dk, dv, 4, 11, 9, io, "f32",
                     3000 + dk + dv, desync=True)
    run_gdn(wl, sample=range(5), o_dtype=out)


@pytest.mark.parametrize("L", [1, 2])
def test_gdn_short_rings(L):
    wl = GdnWorkload(f"gdn_L{L}", 4, 2, 4, 128, 128, L, 9, 8, "f32", "f32", 3100 + L)
    run_gdn(wl, sample=range(4))


def test_gdn_full_size():
    """256 rows, 16 key heads, 32 value heads, K = V = 128, L = 16, bf16 q/k/v,
    fp32 state, 128 steps; all cursors, 8 rows against the oracle."""
    run_gdn(GDN, sample=[0, 31, 64, 100, 128, 170, 200, 255], check_every=2)


def test_gdn_full_size_desynced_rows():
    wl = GdnWorkload("gdn_b256_desync", 256, 16, 32, 128, 128, 16, 40, 512, "bf16", "f32",
                     1004, desync=True)
    run_gdn(wl, sample=[3, 77, 150, 222], standard=False)


def test_gdn_flush_first_row_order_with_a_ragged_row_group():
    """100 desynced rows (a 64-row group and a ragged one of 36): replay tiles
    take each group's flush rows first; cursors of every row bit-exact."""
    wl = GdnWorkload("gdn_b100_desync", 100, 16, 32, 128, 128, 16, 40, 256, "bf16", "f32",
                     1007, desync=True)
    run_gdn(wl, sample=[1, 63, 64, 99])


@pytest.mark.parametrize("L", [5, 17, 32, 64])
def test_gdn_long_rings(L):
    """Rings past one 16-lane row of gates (suffix products over the wave),
    up to the 64-entry maximum; bf16 q/k/v keep the staged rows within LDS."""
    wl = GdnWorkload(f"gdn_L{L}", 3, 2, 4, 128, 128, L, 2 * L + 3, 6, "bf16", "f32",
                     3200 + L, desync=True)
    run_gdn(wl, sample=range(3), check_every=max(1, L // 8))


def test_gdn_longest_fp32_ring():
    """fp32 q/k/v rows take twice the LDS: 57 entries is the longest ring that
    fits at K = V = 128."""
    wl = GdnWorkload("gdn_L57_f32", 3, 2, 4, 128, 128, 57, 2 * 57 + 3, 6, "f32", "f32", 3300,
                     desync=True)
    run_gdn(wl, sample=range(3), check_every=8)
