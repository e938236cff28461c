"""GPU parity of the Mamba2 kernels (standard update and ReplaySSM decode)
against the float64 oracle, through the C ABI.

Tolerances: fp32 inputs and state -> normwise relative 2e-5 per step and
tensor; bf16 inputs or state -> 1e-2 absolute (per element, at least one
bf16 ulp of the reference when y itself is bf16); cursors and ring copies
bit-exact.
"""

import numpy as np
import pytest
import torch

from harness import Tol, log, run_mamba2
from oracle import mamba2 as OM
from workloads import (GROUPED, GROUPED_RINGS, LARGE_BATCH, LAYER_2P7B, TINY,
                       Mamba2Inputs, Mamba2Workload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import linear_recurrence_amd as R
    R.load()


def test_one_hip_runtime_in_process():
    """The library binds to the HIP runtime torch loaded (one copy mapped)."""
    import linear_recurrence_amd as R
    R.load()
    torch.zeros(1, device="cuda")
    maps = open("/proc/self/maps").read()
    libs = {line.split()[-1] for line in maps.splitlines() if "libamdhip64" in line}
    log(f"hip runtimes mapped: {sorted(libs)}")
    assert len(libs) == 1
    assert any("libreplayssm.so" in line for line in maps.splitlines())


def test_tiny_all_rows_all_steps():
    """4 rows, 8 heads, headdim 64, dstate 16, L=4, 32 steps, all fp32."""
    run_mamba2(TINY, sample=range(TINY.batch))


@pytest.mark.parametrize("state_dt,io_dt,out_dt", [
    (s, i, o) for s in ("f32", "bf16") for i in ("f32", "bf16")
    for o in (torch.float32, torch.bfloat16)])
def test_dtype_combinations_ragged(state_dt, io_dt, out_dt):
    """Every dtype combination on a ragged shape: 5 rows, 6 heads in 3 groups."""
    wl = Mamba2Workload(f"ragged_{state_dt}_{io_dt}", 5, 6, 64, 32, 3, 4, 13, 11,
                        io_dt, state_dt, 2000, desync=True)
    run_mamba2(wl, sample=range(5), y_dtype=out_dt)


@pytest.mark.parametrize("P", [32, 64, 128])
@pytest.mark.parametrize("N", [16, 32, 64, 128, 256])
def test_every_supported_tile_shape(P, N):
    wl = Mamba2Workload(f"shape_p{P}_n{N}", 3, 2, P, N, 1, 3, 7, 6, "f32", "f32",
                        2100 + P + N, desync=True)
    run_mamba2(wl, sample=range(3))


def _one_wave_grid(P, N, state_dt, H=16):
    """Rows enough that the replay grid takes the one-wave-per-16-KB path
    (at least 8192 waves of 16 state vectors per lane)."""
    tile = P * N * (2 if state_dt == "bf16" else 4)
    per_tile = max(1, tile // 16384)
    return -(-8192 // (H * per_tile))


@pytest.mark.parametrize("P", [32, 64, 128])
@pytest.mark.parametrize("N", [16, 32, 64, 128, 256])
def test_every_tile_shape_on_a_full_grid(P, N):
    """The same shapes on grids large enough for 16 vectors per lane (the
    small grids above run 4 per lane); alternating dtypes; sampled rows."""
    state_dt, io_dt = (("bf16", "bf16") if (P // 32 + N // 16) % 2 else ("f32", "bf16"))
    nb = _one_wave_grid(P, N, state_dt)
    print(f"case: full grid P={P} N={N} batch={nb} state={state_dt}", flush=True)
    wl = Mamba2Workload(f"grid_p{P}_n{N}", nb, 16, P, N, 2, 3, 4, nb, io_dt, state_dt,
                        2200 + P + N, desync=True)
    run_mamba2(wl, sample=[0, nb // 2, nb - 1], standard=False)


@pytest.mark.parametrize("L,P,N,io,state_dt", [
    (17, 32, 64, "bf16", "f32"), (32, 64, 128, "f32", "f32"), (64, 64, 128, "bf16", "bf16"),
    (64, 64, 128, "f32", "f32")])
def test_long_rings_up_to_the_maximum(L, P, N, io, state_dt):
    """Rings past one 16-lane row of dt (the wave-wide suffix scan and the
    ring-term loop past 16 entries) up to the 64-entry maximum; start positions
    uniform, so every write position and a flush of every row occur."""
    print(f"case: long ring L={L} P={P} N={N} io={io} state={state_dt}", flush=True)
    wl = Mamba2Workload(f"ring_L{L}_p{P}_n{N}_{io}", 4, 6, P, N, 2, L, 2 * L + 3, 8, io,
                        state_dt, 2300 + L, desync=True)
    run_mamba2(wl, sample=range(4), check_every=max(1, L // 8))


def test_layer_2p7b_full_size():
    """64 rows, 80 heads, dstate 128, L=16, bf16 io, fp32 pool of 1024 slots,
    256 steps; every row's cursors checked, 8 rows against the oracle."""
    run_mamba2(LAYER_2P7B, sample=[0, 9, 17, 30, 41, 50, 58, 63])


def _large_batch_sample():
    w0 = Mamba2Inputs(LARGE_BATCH).start_positions().numpy()
    rows = []
    for res in range(LARGE_BATCH.ring_len):       # one row per start position
        rows.append(int(np.nonzero(w0 == res)[0][0]))
    return rows


def test_large_batch_full_size_bench_configuration():
    """512 rows, bf16 state and io, start positions uniform in [0, 16) so that
    flush rows interleave every step, 128 steps; bf16 y as the bench runs it."""
    run_mamba2(LARGE_BATCH, sample=_large_batch_sample(), y_dtype=torch.bfloat16)


def test_flush_first_row_order_with_a_ragged_row_group():
    """Replay tiles visit the flush rows first, dealt over the XCDs by the
    kernel (110 rows: the last lane of the flag load holds a ragged 6 rows)
    with uniform start positions: every row is still advanced exactly once
    per step (all cursors bit-exact) and sampled rows across the batch match
    the oracle."""
    wl = LARGE_BATCH.with_batch(110, steps=40, num_slots=256, name="mamba2_b110_desync")
    run_mamba2(wl, sample=[0, 37, 63, 64, 90, 109], y_dtype=torch.float32)


def test_batch_over_512_rows_takes_the_per_group_order():
    """600 rows x 16 heads (a full grid of one-wave tiles): past 512 rows the
    kernel takes each aligned 64-row group's flush rows first instead of
    dealing the batch's; all cursors bit-exact, sampled rows in the first,
    a middle and the ragged last group against the oracle."""
    print("case: batch 600, 16 heads, per-group flush order", flush=True)
    wl = Mamba2Workload("mamba2_b600_h16", 600, 16, 64, 128, 1, 16, 35, 1200, "bf16", "bf16",
                        2950, desync=True)
    run_mamba2(wl, sample=[0, 63, 64, 300, 575, 576, 599], y_dtype=torch.float32,
               standard=False)


def test_unaligned_flush_flags_give_the_same_results():
    """Flush flags at an odd byte address turn the kernel's own dealing off
    (it reads the flags 8 bytes at a time); the rows are then taken per
    64-row group, and y, checkpoints, rings and cursors stay bit for bit
    those of the aligned launch."""
    import linear_recurrence_amd as R
    from workloads import TORCH_DTYPES
    print("case: unaligned flush flags, 130 rows x 64 heads", flush=True)
    dev = torch.device("cuda:0")
    nb, H, P, N, G, L = 130, 64, 64, 128, 1, 16
    wl = Mamba2Workload("unaligned_flags", nb, H, P, N, G, L, 2 * L + 3, 2 * nb + 8, "bf16",
                        "bf16", 2960, desync=True)
    gen = Mamba2Inputs(wl)
    prm = {k: v.to(dev) for k, v in gen.params().items()}
    slots = gen.slot_idx().to(dev)
    iot = TORCH_DTYPES["bf16"]
    pool = gen.state_pool(gen.slot_idx().tolist())
    runs = {}
    for name, off in (("aligned", 0), ("unaligned", 1)):
        ns = wl.num_slots
        fl_a = torch.zeros(nb + 1, dtype=torch.uint8, device=dev)[off:off + nb]
        fl_b = torch.zeros(nb + 1, dtype=torch.uint8, device=dev)[off:off + nb]
        assert (fl_a.data_ptr() % 8 == 0) == (off == 0)
        fl_a.copy_((gen.start_positions() == L - 1).to(torch.uint8).to(dev))
        runs[name] = {"state": pool.clone().to(dev),
                      "xr": torch.zeros((ns, H, L, P), dtype=iot, device=dev),
                      "dr": torch.zeros((ns, H, L), device=dev),
                      "br": torch.zeros((ns, G, L, N), dtype=iot, device=dev),
                      "wp": gen.start_positions().to(dev), "nwp": torch.empty(nb, dtype=torch.int32,
                                                                              device=dev),
                      "fl": fl_a, "nfl": fl_b, "ys": []}
    for t in range(wl.steps):
        inp = {k: v.to(dev) for k, v in gen.step(t).items()}
        for r in runs.values():
            y = R.replayssm_decode(r["state"], r["xr"], r["dr"], r["br"], slots, r["wp"], r["fl"],
                                   inp["x"], inp["dt"], prm["A"], inp["B"], inp["C"], D=prm["D"],
                                   z=inp["z"], dt_bias=prm["dt_bias"], next_write_pos=r["nwp"],
                                   next_is_flush=r["nfl"])
            r["ys"].append(y.clone())
            r["wp"], r["nwp"] = r["nwp"], r["wp"]
            r["fl"], r["nfl"] = r["nfl"], r["fl"]
    torch.cuda.synchronize()
    a, u = runs["aligned"], runs["unaligned"]
    for t in range(wl.steps):
        assert torch.equal(a["ys"][t].view(torch.int16), u["ys"][t].view(torch.int16)), f"y {t}"
    for k in ("state", "xr", "br"):
        assert torch.equal(a[k].view(torch.int16), u[k].view(torch.int16)), k
    assert torch.equal(a["dr"].view(torch.int32), u["dr"].view(torch.int32))
    assert torch.equal(a["wp"], u["wp"]) and torch.equal(a["fl"], u["fl"])
    log(f"{wl.steps} steps: unaligned flags give the aligned launch's results bit for bit")


def test_large_batch_full_size_fp32_output():
    run_mamba2(LARGE_BATCH, sample=_large_batch_sample()[::3], y_dtype=torch.float32,
               standard=False)


@pytest.mark.parametrize("L", GROUPED_RINGS)
def test_grouped_with_resets_full_size(L):
    """256 rows, 128 heads in 8 groups, fp32 pool, 192 steps, slot reuse at
    steps 37, 101 and 150 (fresh checkpoint, cursors reset mid-ring, stale ring
    entries poisoned)."""
    wl = GROUPED.with_ring(L)
    gen = Mamba2Inputs(wl)
    reset_rows = sorted({r for t in wl.reset_steps for r in gen.resets(t)[0]})
    sample = sorted(set(reset_rows[:4] + [1, 128, 255]))
    run_mamba2(wl, sample=sample, check_every=3)


def _small(dev, L=1, state_dt=torch.float32, io=torch.bfloat16, nb=6, H=4, P=64, N=128):
    g = torch.Generator().manual_seed(7)
    ns = nb + 3
    d = dict(
        state=(torch.randn(ns, H, P, N, generator=g) * 0.1).to(state_dt).to(dev),
        x=torch.randn(nb, H, P, generator=g).to(io).to(dev),
        z=torch.randn(nb, H, P, generator=g).to(io).to(dev),
        dt=torch.randn(nb, H, generator=g).to(io).to(dev),
        B=(torch.randn(nb, 1, N, generator=g) / 4).to(io).to(dev),
        C=(torch.randn(nb, 1, N, generator=g) / 4).to(io).to(dev),
        A=-torch.rand(H, generator=g).add(0.5).to(dev),
        D=torch.randn(H, generator=g).to(dev),
        dt_bias=torch.randn(H, generator=g).sub(3).to(dev),
        slot=torch.randperm(ns, generator=g)[:nb].int().to(dev),
    )
    d["x_ring"] = torch.zeros(ns, H, L, P, dtype=io, device=dev)
    d["dt_ring"] = torch.zeros(ns, H, L, device=dev)
    d["B_ring"] = torch.zeros(ns, 1, L, N, dtype=io, device=dev)
    return d


@pytest.mark.parametrize("state_dt", [torch.float32, torch.bfloat16])
def test_L1_replay_is_the_standard_update_bit_for_bit(state_dt):
    import linear_recurrence_amd as R
    dev = torch.device("cuda")
    d = _small(dev, L=1, state_dt=state_dt)
    s2 = d["state"].clone()
    wp = torch.zeros(6, dtype=torch.int32, device=dev)
    fl = torch.ones(6, dtype=torch.uint8, device=dev)
    for _ in range(3):
        y1 = R.replayssm_decode(d["state"], d["x_ring"], d["dt_ring"], d["B_ring"], d["slot"],
                                wp, fl, d["x"], d["dt"], d["A"], d["B"], d["C"], D=d["D"],
                                z=d["z"], dt_bias=d["dt_bias"], out_dtype=torch.float32)
        y2 = R.ssu_standard_decode(s2, d["slot"], d["x"], d["dt"], d["A"], d["B"], d["C"],
                                   D=d["D"], z=d["z"], dt_bias=d["dt_bias"],
                                   out_dtype=torch.float32)
        assert torch.equal(y1, y2)
        assert torch.equal(d["state"].view(torch.int16) if state_dt == torch.bfloat16
                           else d["state"].view(torch.int32),
                           s2.view(torch.int16) if state_dt == torch.bfloat16
                           else s2.view(torch.int32))


def test_optional_operands_and_no_softplus():
    """D, z, dt_bias absent and dt used as given: compared with the oracle."""
    import linear_recurrence_amd as R
    dev = torch.device("cuda")
    d = _small(dev, L=4, io=torch.float32)
    pool = d["state"].double().cpu().numpy()
    wp = torch.zeros(6, dtype=torch.int32, device=dev)
    fl = torch.zeros(6, dtype=torch.uint8, device=dev)
    nwp, nfl = torch.empty_like(wp), torch.empty_like(fl)
    dtp = d["dt"].abs() * 0.1
    o_xr = np.zeros((9, 4, 4, 64))
    o_dr = np.zeros((9, 4, 4))
    o_br = np.zeros((9, 1, 4, 128))
    o_wp, o_fl = np.zeros(6, np.int32), np.zeros(6, np.uint8)
    for t in range(6):
        y = R.replayssm_decode(d["state"], d["x_ring"], d["dt_ring"], d["B_ring"], d["slot"],
                               wp, fl, d["x"], dtp, d["A"], d["B"], d["C"],
                               next_write_pos=nwp, next_is_flush=nfl, dt_softplus=False,
                               out_dtype=torch.float32)
        wp, nwp, fl, nfl = nwp, wp, nfl, fl
        y_ref, o_wp, o_fl, _ = OM.replay_step(
            pool, o_xr, o_dr, o_br, d["slot"].cpu().numpy(), o_wp, o_fl,
            d["x"].double().cpu().numpy(), dtp.double().cpu().numpy(),
            d["A"].double().cpu().numpy(), d["B"].double().cpu().numpy(),
            d["C"].double().cpu().numpy(), dt_softplus=False, state_dtype="f32")
        Tol("rel", 2e-5).check(f"step {t}", y.double().cpu().numpy(), y_ref)
        assert np.array_equal(wp.cpu().numpy(), o_wp)


def test_status_bits_and_safe_handling():
    """Out-of-contract metadata (forced from the host) sets the status bits;
    the kernel's own bounds handling keeps every access in range, and rows
    within the contract are unaffected."""
    import linear_recurrence_amd as R
    dev = torch.device("cuda")
    d = _small(dev, L=4)
    slot = d["slot"].clone()
    slot[1] = 10_000                 # outside the pool
    slot[2] = -3
    wp = torch.tensor([0, 0, 0, 9, 3, -1], dtype=torch.int32, device=dev)
    fl = torch.tensor([0, 0, 0, 0, 0, 0], dtype=torch.uint8, device=dev)
    nwp = torch.full_like(wp, 77)
    nfl = torch.full_like(fl, 77)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    y = R.replayssm_decode(d["state"], d["x_ring"], d["dt_ring"], d["B_ring"], slot, wp, fl,
                           d["x"], d["dt"], d["A"], d["B"], d["C"], D=d["D"], z=d["z"],
                           dt_bias=d["dt_bias"], next_write_pos=nwp, next_is_flush=nfl,
                           status=status, out_dtype=torch.float32)
    torch.cuda.synchronize()
    st = int(status.item())
    assert st == R.ST_BAD_SLOT | R.ST_BAD_WRITE_POS | R.ST_RING_OVERFLOW
    assert torch.isnan(y[1]).all() and torch.isnan(y[2]).all()
    assert torch.isfinite(y[[0, 3, 4, 5]]).all()
    assert nwp.tolist() == [1, 0, 0, 0, 0, 0]
    assert nfl.tolist() == [0, 0, 0, 0, 0, 0]
    # ring reset with a row out of range
    status.zero_()
    R.replayssm_ring_reset(nwp, nfl, torch.tensor([0, 99], dtype=torch.int32, device=dev), 4,
                           status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == R.ST_BAD_ROW and nwp[0].item() == 0


def test_empty_batch_is_a_no_op():
    import linear_recurrence_amd as R
    dev = torch.device("cuda")
    d = _small(dev, L=4, nb=6)
    e = lambda *s, dt=torch.bfloat16: torch.empty(*s, dtype=dt, device=dev)
    before = d["state"].clone()
    y = R.replayssm_decode(d["state"], d["x_ring"], d["dt_ring"], d["B_ring"],
                           e(0, dt=torch.int32), e(0, dt=torch.int32), e(0, dt=torch.uint8),
                           e(0, 4, 64), e(0, 4), d["A"], e(0, 1, 128), e(0, 1, 128))
    y2 = R.ssu_standard_decode(d["state"], e(0, dt=torch.int32), e(0, 4, 64), e(0, 4), d["A"],
                               e(0, 1, 128), e(0, 1, 128))
    R.replayssm_ring_reset(e(0, dt=torch.int32), e(0, dt=torch.uint8), e(0, dt=torch.int32), 4)
    torch.cuda.synchronize()
    assert y.shape == (0, 4, 64) and y2.shape == (0, 4, 64)
    assert torch.equal(before, d["state"])


def test_output_only_rows_never_write_the_pool():
    """Non-flush rows read S0 and leave every pool byte unchanged; pool slots
    no row uses stay NaN."""
    import linear_recurrence_amd as R
    dev = torch.device("cuda")
    d = _small(dev, L=8)
    used = d["slot"].long()
    unused = torch.tensor(sorted(set(range(9)) - set(used.tolist())), device=dev)
    d["state"][unused] = float("nan")
    before = d["state"].clone()
    wp = torch.zeros(6, dtype=torch.int32, device=dev)
    fl = torch.zeros(6, dtype=torch.uint8, device=dev)
    nwp, nfl = torch.empty_like(wp), torch.empty_like(fl)
    for _ in range(6):                          # 6 < L-1: no flush yet
        R.replayssm_decode(d["state"], d["x_ring"], d["dt_ring"], d["B_ring"], d["slot"],
                           wp, fl, d["x"], d["dt"], d["A"], d["B"], d["C"], D=d["D"],
                           z=d["z"], dt_bias=d["dt_bias"], next_write_pos=nwp,
                           next_is_flush=nfl)
        wp, nwp, fl, nfl = nwp, wp, nfl, fl
    torch.cuda.synchronize()
    assert torch.equal(before[used], d["state"][used])
    assert torch.isnan(d["state"][unused]).all()
    assert wp.tolist() == [6] * 6 and fl.tolist() == [0] * 6


@pytest.mark.parametrize("nb,H,P,N,G,L,io", [
    (110, 6, 64, 32, 3, 5, "bf16"), (70, 80, 64, 16, 1, 16, "f32"), (4, 8, 64, 16, 2, 4, "f32"),
    (130, 64, 64, 128, 1, 16, "bf16")])  # the last: 16 vectors per lane, two waves per tile
def test_ring_appends_of_every_row(nb, H, P, N, G, L, io):
    """Every row that does not flush gets ring entry w: its x and B rows bit
    for bit (B once per group) and its dt after bias and softplus; every
    other ring element keeps its bits.  All rows and all ring elements are
    checked over several steps, with a full and a ragged 64-row group, more
    heads than rows in a group, rows forced to flush early, and rows with bad
    metadata (a full ring without the flush flag and a write position past
    the ring at step 0, a slot out of range throughout), which must not
    append."""
    import linear_recurrence_amd as R
    from oracle import numerics as ON
    from workloads import TORCH_DTYPES
    print(f"case: ring appends nb={nb} H={H} P={P} N={N} G={G} L={L} io={io}", flush=True)
    dev = torch.device("cuda:0")
    wl = Mamba2Workload(f"appends_b{nb}_h{H}", nb, H, P, N, G, L, 4, 2 * nb + 8, io, "f32",
                        2500 + nb, desync=True)
    gen = Mamba2Inputs(wl)
    prm = {k: v.to(dev) for k, v in gen.params().items()}
    slots = gen.slot_idx()
    ns, iot = wl.num_slots, TORCH_DTYPES[io]
    state = gen.state_pool(slots.tolist()).to(dev)
    g = torch.Generator().manual_seed(2600 + nb)
    # rings hold arbitrary earlier contents: any element not appended must keep its bits
    xr = torch.randn((ns, H, L, P), generator=g).to(iot).to(dev)
    dr = torch.rand((ns, H, L), generator=g).to(dev)
    br = torch.randn((ns, G, L, N), generator=g).to(iot).to(dev)
    wp = gen.start_positions().to(dev)
    fl = (wp == L - 1).to(torch.uint8)
    fl |= (torch.rand(nb, generator=g) < 0.2).to(torch.uint8).to(dev)  # forced flushes
    # bad metadata: row 1 at the last position without the flag (overflow),
    # row 2 past the ring, row 3 (when present) with a slot out of range
    wp[1], fl[1], wp[2] = L - 1, 0, L + 3
    if nb > 3:
        slots[3] = -1
    nwp, nfl = torch.empty_like(wp), torch.empty_like(fl)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    s_np = slots.numpy()
    bias = prm["dt_bias"].double().cpu().numpy()
    for t in range(wl.steps):
        inp = {k: v.to(dev) for k, v in gen.step(t).items()}
        xr0, dr0, br0 = xr.clone(), dr.clone(), br.clone()
        w_np, f_np = wp.cpu().numpy(), fl.cpu().numpy()
        R.replayssm_decode(state, xr, dr, br, slots.to(dev), wp, fl, inp["x"], inp["dt"],
                           prm["A"], inp["B"], inp["C"], D=prm["D"], z=inp["z"],
                           dt_bias=prm["dt_bias"], next_write_pos=nwp, next_is_flush=nfl,
                           status=status)
        torch.cuda.synchronize()
        exp_x, exp_b, exp_d = xr0.clone(), br0.clone(), dr0.clone()
        dt_in = inp["dt"].double().cpu().numpy()
        app_rows = [r for r in range(nb)
                    if not f_np[r] and 0 <= w_np[r] <= L - 2 and 0 <= s_np[r] < ns]
        for r in app_rows:
            s, w = int(s_np[r]), int(w_np[r])
            exp_x[s, :, w, :] = inp["x"][r]
            exp_b[s, :, w, :] = inp["B"][r]
            exp_d[s, :, w] = torch.from_numpy(ON.softplus(dt_in[r] + bias)).float()
        assert torch.equal(xr.view(torch.int8 if io == "f32" else torch.int16),
                           exp_x.view(torch.int8 if io == "f32" else torch.int16)), f"step {t}: x ring"
        assert torch.equal(br.view(torch.int8 if io == "f32" else torch.int16),
                           exp_b.view(torch.int8 if io == "f32" else torch.int16)), f"step {t}: B ring"
        mask = torch.zeros((ns, H, L), dtype=torch.bool)
        for r in app_rows:
            mask[int(s_np[r]), :, int(w_np[r])] = True
        got_d, ref_d = dr.cpu(), exp_d.cpu()
        assert torch.equal(got_d[~mask].view(torch.int32), ref_d[~mask].view(torch.int32)), \
            f"step {t}: dt ring elements that were not appended changed"
        if app_rows:
            err = ((got_d[mask].double() - ref_d[mask].double()).abs()
                   / ref_d[mask].double().abs().clamp(min=1.0)).max().item()
            assert err <= 1e-6, f"step {t}: dt ring append error {err:.3e}"
        log(f"step {t}: {len(app_rows)} of {nb} rows appended, rings exact")
        wp, nwp = nwp, wp
        fl, nfl = nfl, fl
    bits = R.ST_RING_OVERFLOW | R.ST_BAD_WRITE_POS | (R.ST_BAD_SLOT if nb > 3 else 0)
    assert int(status.item()) == bits


@pytest.mark.parametrize("nb,H,P,N,G,L", [(200, 8, 64, 32, 2, 8), (130, 64, 64, 128, 1, 16)])
def test_row_order_gives_the_same_results(nb, H, P, N, G, L):
    """replayssm_decode_ordered with the host's flush-first order, and with an
    arbitrary permutation, gives bit for bit what replayssm_decode gives (y,
    checkpoints, rings, cursors) over steps that cross flushes; a row index
    outside the batch is clamped and reported.  Small grids (4 vectors per
    lane) and full grids (16) with ragged 64-row groups."""
    import linear_recurrence_amd as R
    from workloads import TORCH_DTYPES
    print(f"case: row order nb={nb} H={H} P={P} N={N} L={L}", flush=True)
    dev = torch.device("cuda:0")
    wl = Mamba2Workload(f"order_b{nb}_h{H}", nb, H, P, N, G, L, 2 * L + 3, 2 * nb + 8, "bf16",
                        "bf16", 2700 + nb, desync=True)
    gen = Mamba2Inputs(wl)
    prm = {k: v.to(dev) for k, v in gen.params().items()}
    slots = gen.slot_idx().to(dev)
    iot = TORCH_DTYPES["bf16"]
    pool = gen.state_pool(gen.slot_idx().tolist())
    g = torch.Generator().manual_seed(2800 + nb)
    perm = torch.randperm(nb, generator=g).to(torch.int32).to(dev)

    def fresh():
        ns = wl.num_slots
        return {"state": pool.clone().to(dev),
                "xr": torch.zeros((ns, H, L, P), dtype=iot, device=dev),
                "dr": torch.zeros((ns, H, L), device=dev),
                "br": torch.zeros((ns, G, L, N), dtype=iot, device=dev),
                "wp": gen.start_positions().to(dev),
                "fl": (gen.start_positions() == L - 1).to(torch.uint8).to(dev)}

    runs = {"plain": fresh(), "flush_first": fresh(), "permuted": fresh()}
    for t in range(wl.steps):
        inp = {k: v.to(dev) for k, v in gen.step(t).items()}
        ys = {}
        for name, r in runs.items():
            order = None
            if name == "flush_first":
                order = torch.from_numpy(R.flush_first_order(r["fl"].cpu().numpy())).to(dev)
            elif name == "permuted":
                order = perm
            nwp, nfl = torch.empty_like(r["wp"]), torch.empty_like(r["fl"])
            ys[name] = R.replayssm_decode(
                r["state"], r["xr"], r["dr"], r["br"], slots, r["wp"], r["fl"], inp["x"],
                inp["dt"], prm["A"], inp["B"], inp["C"], D=prm["D"], z=inp["z"],
                dt_bias=prm["dt_bias"], next_write_pos=nwp, next_is_flush=nfl,
                row_order=order)
            r["wp"], r["fl"] = nwp, nfl
        torch.cuda.synchronize()
        ref = runs["plain"]
        for name in ("flush_first", "permuted"):
            r = runs[name]
            assert torch.equal(ys[name].view(torch.int16), ys["plain"].view(torch.int16)), \
                f"step {t} {name}: y"
            for k in ("state", "xr", "br"):
                assert torch.equal(r[k].view(torch.int16), ref[k].view(torch.int16)), \
                    f"step {t} {name}: {k}"
            assert torch.equal(r["dr"].view(torch.int32), ref["dr"].view(torch.int32))
            assert torch.equal(r["wp"], ref["wp"]) and torch.equal(r["fl"], ref["fl"])
    log(f"{wl.steps} steps: ordered launches equal the plain ones bit for bit")
    # stochastic rounding of the write-back draws its bits by (slot, head,
    # element), not by the order the rows are processed in
    for t in range(wl.steps, wl.steps + L):
        inp = {k: v.to(dev) for k, v in gen.step(t).items()}
        for name in ("plain", "permuted"):
            r = runs[name]
            nwp, nfl = torch.empty_like(r["wp"]), torch.empty_like(r["fl"])
            R.replayssm_decode(r["state"], r["xr"], r["dr"], r["br"], slots, r["wp"], r["fl"],
                               inp["x"], inp["dt"], prm["A"], inp["B"], inp["C"], D=prm["D"],
                               z=inp["z"], dt_bias=prm["dt_bias"], next_write_pos=nwp,
                               next_is_flush=nfl, rounding="stochastic", sr_seed=31,
                               sr_offset=t, row_order=perm if name == "permuted" else None)
            r["wp"], r["fl"] = nwp, nfl
    torch.cuda.synchronize()
    assert torch.equal(runs["permuted"]["state"].view(torch.int16),
                       runs["plain"]["state"].view(torch.int16)), "stochastic rounding: state"
    # an entry outside the batch is reported, and its position processes
    # nothing: every other row gets exactly what the plain launch gives it,
    # the missing row gets no y, cursor or fold (its checkpoint is untouched)
    # and the ring appends, which do not depend on the order, all happen.
    # Step 0 of the workload has flush rows; the missing row is one of them.
    inp = {k: v.to(dev) for k, v in gen.step(0).items()}
    flags0 = fresh()["fl"].cpu().numpy()
    missing_pos = int(np.nonzero(flags0[perm.cpu().numpy()])[0][0])
    missing = int(perm[missing_pos].item())
    bad = perm.clone()
    bad[missing_pos] = nb + 5
    outs = {}
    for name, order in (("plain", None), ("bad", bad)):
        r = fresh()
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        sentinel_wp = torch.full_like(r["wp"], -7)
        sentinel_fl = torch.full_like(r["fl"], 7)
        y = torch.full((nb, H, P), float("nan"), device=dev)
        R.replayssm_decode(r["state"], r["xr"], r["dr"], r["br"], slots, r["wp"], r["fl"],
                           inp["x"], inp["dt"], prm["A"], inp["B"], inp["C"], D=prm["D"],
                           z=inp["z"], dt_bias=prm["dt_bias"], y=y,
                           next_write_pos=sentinel_wp, next_is_flush=sentinel_fl,
                           status=status, row_order=order)
        torch.cuda.synchronize()
        outs[name] = (r, y, sentinel_wp, sentinel_fl, int(status.item()))
    (rp, yp, wpp, flp, stp), (rb, yb, wpb, flb, stb) = outs["plain"], outs["bad"]
    assert stp == 0 and stb == R.ST_BAD_ROW, (stp, stb)
    keep = torch.tensor([i for i in range(nb) if i != missing], device=dev)
    assert torch.equal(yb[keep], yp[keep]), "bad order entry: other rows' y"
    assert torch.isnan(yb[missing]).all(), "bad order entry: the missing row got a y"
    assert torch.equal(wpb[keep], wpp[keep]) and torch.equal(flb[keep], flp[keep])
    assert int(wpb[missing]) == -7 and int(flb[missing]) == 7, "missing row's cursors"
    s_miss = int(slots[missing])
    other = torch.tensor([i for i in range(wl.num_slots) if i != s_miss], device=dev)
    assert torch.equal(rb["state"][other].view(torch.int16), rp["state"][other].view(torch.int16))
    assert torch.equal(rb["state"][s_miss].cpu(), pool[s_miss]), "missing row's checkpoint"
    for k in ("xr", "br", "dr"):
        assert torch.equal(rb[k], rp[k]), f"bad order entry: ring {k}"
