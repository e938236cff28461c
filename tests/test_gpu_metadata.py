"""The host metadata builder driving the GPU replay kernel: align-mode and
forced flushes, a resumed (re-anchored) request, one-token prefills; y and
stored checkpoints against the float64 oracle, device cursors against the
builder."""

import numpy as np
import pytest
import torch

import linear_recurrence_amd as R
from oracle import mamba2 as OM
from oracle import metadata as OMD

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")


def test_host_metadata_drives_replay_kernel():
    print("case: host metadata, batch 6, H 4, P 32, N 16, L 8, align 4, fp32", flush=True)
    rng = np.random.default_rng(2024)
    dev = torch.device("cuda:0")
    nb, H, P, N, G, L, ns, T = 6, 4, 32, 16, 1, 8, 9, 40
    slots = np.array([3, 0, 8, 5, 1, 6], np.int32)
    A = -np.exp(rng.uniform(0, np.log(16), H)).astype(np.float32)
    D = rng.normal(size=H).astype(np.float32)
    dtb = np.log(np.expm1(rng.uniform(1e-3, 1e-1, H))).astype(np.float32)
    pool = rng.normal(0, 0.1, (ns, H, P, N)).astype(np.float32)
    st = torch.tensor(pool, device=dev)
    o_pool = pool.astype(np.float64)
    xr = torch.full((ns, H, L, P), float("nan"), device=dev)
    dr = torch.full((ns, H, L), float("nan"), device=dev)
    br = torch.full((ns, G, L, N), float("nan"), device=dev)
    o_xr = np.full((ns, H, L, P), np.nan)
    o_dr = np.full((ns, H, L), np.nan)
    o_br = np.full((ns, G, L, N), np.nan)
    prefill = np.array([1, 5, 12, 3, 8, 30], np.int64)   # one-token prefill included
    pos, base = prefill.copy(), prefill.copy()
    sl = torch.tensor(slots, device=dev)
    nwp = torch.empty(nb, dtype=torch.int32, device=dev)
    nfl = torch.empty(nb, dtype=torch.uint8, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    gA, gD, gb = (torch.tensor(v, device=dev) for v in (A, D, dtb))
    for t in range(T):
        if t == 13:                      # row 2 resumes after preemption: fresh checkpoint
            fresh = rng.normal(0, 0.1, (H, P, N)).astype(np.float32)
            st[int(slots[2])] = torch.tensor(fresh, device=dev)
            o_pool[slots[2]] = fresh
            base[2] = pos[2]
        force = (rng.random(nb) < 0.08).astype(np.uint8)
        ow, of, onb = OMD.build_metadata(pos.tolist(), base.tolist(), L, force.tolist(), 4)
        w, f = R.build_metadata(pos, base, L, force, align_block=4)
        np.testing.assert_array_equal(w, ow)
        np.testing.assert_array_equal(f, of)
        np.testing.assert_array_equal(base, onb)
        x = rng.normal(size=(nb, H, P)).astype(np.float32)
        z = rng.normal(size=(nb, H, P)).astype(np.float32)
        dt = rng.normal(size=(nb, H)).astype(np.float32)
        B = (rng.normal(size=(nb, G, N)) / 4).astype(np.float32)
        C = (rng.normal(size=(nb, G, N)) / 4).astype(np.float32)
        y = R.replayssm_decode(st, xr, dr, br, sl, torch.tensor(w, device=dev),
                               torch.tensor(f, device=dev), torch.tensor(x, device=dev),
                               torch.tensor(dt, device=dev), gA, torch.tensor(B, device=dev),
                               torch.tensor(C, device=dev), D=gD, z=torch.tensor(z, device=dev),
                               dt_bias=gb, next_write_pos=nwp, next_is_flush=nfl, status=status)
        oy, onw, onf, ost = OM.replay_step(o_pool, o_xr, o_dr, o_br, slots, w, f, x, dt, A, B, C,
                                           D=D, z=z, dt_bias=dtb, state_dtype="f32")
        yy = y.double().cpu().numpy()
        err = np.abs(yy - oy).max() / np.abs(oy).max()
        assert err <= 2e-5, f"step {t}: y error {err:.2e}"
        np.testing.assert_array_equal(nwp.cpu().numpy(), onw)
        np.testing.assert_array_equal(nfl.cpu().numpy(), onf)
        for r in np.nonzero(f)[0]:
            s = int(slots[r])
            e = np.abs(st[s].double().cpu().numpy() - o_pool[s]).max() / np.abs(o_pool[s]).max()
            assert e <= 2e-5, f"step {t} row {r}: checkpoint error {e:.2e}"
        pos = pos + 1
    torch.cuda.synchronize()
    assert status.item() == 0
