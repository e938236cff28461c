"""Stochastic rounding of the bf16 state write-back on the GPU.

Exactness test: with A = 0, dt = 1 and inputs on a coarse binary grid every
fp32 intermediate of the update is exact, so the GPU and the oracle round
the very same fp32 values with the very same Philox bits: the stored bf16
states must agree bit for bit (standard update and replay flush, every
lane-pairing path of the kernels).  Then a realistic parity run with SR."""

import numpy as np
import pytest
import torch

import linear_recurrence_amd as R
from harness import run_mamba2
from oracle import mamba2 as OM
from oracle import numerics as NU
from workloads import LARGE_BATCH

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")


def _grid_inputs(rng, nb, H, P, N, steps):
    xs = [(rng.integers(-15, 16, (nb, H, P)) / 16.0) for _ in range(steps)]
    Bs = [(rng.integers(-7, 8, (nb, 1, N)) / 4.0) for _ in range(steps)]
    Cs = [rng.normal(size=(nb, 1, N)) for _ in range(steps)]
    return xs, Bs, Cs


SHAPES = [(64, 128), (32, 16), (128, 256), (32, 64), (64, 32)]


@pytest.mark.parametrize("P,N", SHAPES)
@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16])
def test_sr_bits_exact(P, N, io):
    print(f"case: SR exact bits P={P} N={N} io={io}", flush=True)
    rng = np.random.default_rng(P * 1000 + N + (io == torch.bfloat16))
    dev = torch.device("cuda:0")
    nb, H, L, ns = 3, 4, 4, 5
    slots = np.array([4, 0, 2], np.int32)
    pool = (rng.integers(-255, 256, (ns, H, P, N)) / 64.0)
    gA = torch.zeros(H, device=dev)
    sl = torch.tensor(slots, device=dev)
    seed, off = 0x1234ABCD5678, 77
    xs, Bs, Cs = _grid_inputs(rng, nb, H, P, N, L)
    dt = torch.ones((nb, H), dtype=io, device=dev)
    g = lambda a: torch.tensor(a, dtype=io, device=dev)

    # standard update: S = S0 + x (x) B, stochastically rounded
    st = torch.tensor(pool, dtype=torch.bfloat16, device=dev)
    R.ssu_standard_decode(st, sl, g(xs[0]), dt, gA, g(Bs[0]), g(Cs[0]), dt_softplus=False,
                          rounding="stochastic", sr_seed=seed, sr_offset=off)
    o = pool.copy()
    OM.ssu_standard_step(o, slots, xs[0], np.ones((nb, H)), np.zeros(H), Bs[0], Cs[0],
                         dt_softplus=False, state_dtype="bf16", rounding="stochastic",
                         sr_seed=seed, sr_offset=off)
    got = st.double().cpu().numpy()
    np.testing.assert_array_equal(got, o)
    rne = NU.round_bf16(pool[slots] + xs[0][..., None] * np.repeat(Bs[0], H, 1)[:, :, None, :])
    assert (got[slots] != rne).any(), "stochastic rounding changed nothing"

    # replay: 3 output-only steps, then a flush folding 4 entries
    st = torch.tensor(pool, dtype=torch.bfloat16, device=dev)
    xr = torch.zeros((ns, H, L, P), dtype=io, device=dev)
    dr = torch.zeros((ns, H, L), device=dev)
    br = torch.zeros((ns, 1, L, N), dtype=io, device=dev)
    o = pool.copy()
    oxr, odr, obr = np.zeros((ns, H, L, P)), np.zeros((ns, H, L)), np.zeros((ns, 1, L, N))
    for w in range(L):
        f = np.full(nb, 1 if w == L - 1 else 0, np.uint8)
        wp = np.full(nb, w, np.int32)
        R.replayssm_decode(st, xr, dr, br, sl, torch.tensor(wp, device=dev),
                           torch.tensor(f, device=dev), g(xs[w]), dt, gA, g(Bs[w]), g(Cs[w]),
                           dt_softplus=False, rounding="stochastic", sr_seed=seed,
                           sr_offset=off + w)
        OM.replay_step(o, oxr, odr, obr, slots, wp, f, xs[w], np.ones((nb, H)), np.zeros(H),
                       Bs[w], Cs[w], dt_softplus=False, state_dtype="bf16",
                       rounding="stochastic", sr_seed=seed, sr_offset=off + w)
    np.testing.assert_array_equal(st.double().cpu().numpy(), o)


def test_sr_offsets_draw_new_bits_and_repeat_exactly():
    print("case: SR offsets", flush=True)
    rng = np.random.default_rng(11)
    dev = torch.device("cuda:0")
    nb, H, P, N, ns = 2, 2, 64, 128, 2
    pool = torch.tensor(rng.normal(0, 0.3, (ns, H, P, N)), dtype=torch.bfloat16, device=dev)
    sl = torch.tensor([1, 0], dtype=torch.int32, device=dev)
    x = torch.randn((nb, H, P), device=dev)
    dt = torch.randn((nb, H), device=dev)
    A = -torch.rand(H, device=dev)
    B = torch.randn((nb, 1, N), device=dev) / 4
    C = torch.randn((nb, 1, N), device=dev) / 4
    outs = []
    for off in (5, 6, 5):
        st = pool.clone()
        R.ssu_standard_decode(st, sl, x, dt, A, B, C, rounding="stochastic", sr_seed=3,
                              sr_offset=off)
        outs.append(st)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[2])
    assert not torch.equal(outs[0], outs[1])


def test_sr_parity_bench_configuration():
    """The batch-512 bf16-pool workload with stochastic rounding on both the
    replay flushes and the standard update, 24 steps, against the oracle."""
    print("case: SR parity, mamba2_b512 bf16 pool, 24 steps", flush=True)
    run_mamba2(LARGE_BATCH, sample=[0, 101, 255, 300, 511], steps=24, rounding="stochastic")
