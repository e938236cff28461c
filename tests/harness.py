"""Parity harness: run a workload through the HIP library on the GPU and the
float64 oracle on sampled rows, side by side, step by step.

Rows are independent (each owns its slot, ring and cursors), so the oracle
runs only the sampled rows on a compact pool and is exact for them.

Checks per step:
  * y of the sampled rows against the oracle (tolerance by workload);
  * every row's next cursors against the oracle's cursor rule (bit-exact);
  * for sampled output-only rows, the ring entry written this step is a bit
    copy of the step's x and B, and the stored dt matches the oracle's;
  * for sampled flush rows, the stored checkpoint against the oracle's;
  * the standard update's y (and at the end its state) against the
    recurrent oracle.
"""

import math
import sys
import time

import numpy as np
import torch

import linear_recurrence_amd as R
from oracle import gdn as OG
from oracle import kda as OK
from oracle import mamba2 as OM
from workloads import TORCH_DTYPES, GdnInputs, Mamba2Inputs


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_ulp(a):
    a = np.abs(np.asarray(a, np.float64))
    e = np.floor(np.log2(np.maximum(a, 1e-38)))
    return np.exp2(e - 7)


class Tol:
    """Tolerance of one comparison.

    kind 'rel': max|d| / max|ref| <= tol (normwise relative, fp32 paths);
    kind 'abs': max|d| <= tol (paths with bf16 inputs or state).
    With a bf16 output the output format itself adds up to half a bf16 ulp of
    rounding: the bound per element becomes one bf16 ulp of the reference plus
    the fp32 bound ('rel'), or the larger of the two ('abs').
    """

    def __init__(self, kind, tol, bf16_out=False, ulps=1):
        self.kind, self.tol, self.bf16_out, self.ulps = kind, tol, bf16_out, ulps

    def err(self, got, ref):
        got = np.asarray(got, np.float64)
        ref = np.asarray(ref, np.float64)
        assert got.shape == ref.shape, (got.shape, ref.shape)
        assert np.isfinite(got).all(), "non-finite output"
        d = np.abs(got - ref)
        if self.kind == "rel":
            scale = max(np.abs(ref).max(), 1e-30)
            if self.bf16_out:
                bound = bf16_ulp(ref) + self.tol * scale
                return float((d / bound).max() * self.tol)
            return float(d.max() / scale)
        if self.bf16_out:
            return float((d / np.maximum(self.tol, self.ulps * bf16_ulp(ref))).max() * self.tol)
        return float(d.max())

    def check(self, what, got, ref):
        e = self.err(got, ref)
        if e > self.tol:
            raise AssertionError(f"{what}: error {e:.3e} > {self.tol:.1e} ({self.kind})")
        return e


def _np(t):
    return t.detach().double().cpu().numpy()


SR_SEED = 0x5EED5EED


def run_mamba2(wl, sample, y_dtype=torch.float32, steps=None, tol_state=None,
               tol_y=None, standard=True, check_every=1, dev="cuda:0", rounding="nearest"):
    """Run a Mamba2 workload; returns a dict of worst errors seen.

    rounding="stochastic" (bf16 pools): every state store on both sides uses
    the same Philox bits (key (SR_SEED, call counter)); values that land
    between the two sides' fp32 results may round apart, so stored states
    are compared with a two-ulp allowance, and the final replay-vs-recurrence
    comparison is skipped (per-step stochastic rounding of the recurrence is
    a random walk that the once-per-ring replay does not take)."""
    t0 = time.time()
    dev = torch.device(dev)
    gen = Mamba2Inputs(wl)
    nb, H, P, N, G, L = wl.batch, wl.nheads, wl.headdim, wl.dstate, wl.ngroups, wl.ring_len
    ns = wl.num_slots
    steps = wl.steps if steps is None else steps
    io = TORCH_DTYPES[wl.io_dtype]
    sdt = wl.state_dtype
    fp32_path = wl.io_dtype == "f32" and sdt == "f32"
    if tol_y is None:
        bf16_y = y_dtype == torch.bfloat16
        tol_y = Tol("rel", 2e-5, bf16_y) if fp32_path else Tol("abs", 1e-2, bf16_y)
    if tol_state is None:
        tol_state = Tol("rel", 2e-5) if fp32_path else Tol("abs", 1e-2)
        if rounding == "stochastic":
            tol_state = Tol("abs", 1e-2, True, ulps=2)
    sr_on = rounding == "stochastic"
    calls = [0]
    sample = sorted(set(int(r) for r in sample))
    k = len(sample)

    prm = gen.params()
    slots = gen.slot_idx()
    slots_np = slots.numpy()
    pool = gen.state_pool(slots.tolist())
    gp = {n: v.to(dev) for n, v in prm.items()}
    pn = {n: v.double().numpy() for n, v in prm.items()}
    st_r = pool.to(dev)
    st_s = pool.to(dev) if standard else None
    del pool
    xr = torch.full((ns, H, L, P), float("nan"), dtype=io, device=dev)
    dr = torch.full((ns, H, L), float("nan"), dtype=torch.float32, device=dev)
    br = torch.full((ns, G, L, N), float("nan"), dtype=io, device=dev)
    wp = torch.zeros(nb, dtype=torch.int32, device=dev)
    fl = torch.full((nb,), 1 if L == 1 else 0, dtype=torch.uint8, device=dev)
    nwp, nfl = torch.empty_like(wp), torch.empty_like(fl)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    sl = slots.to(dev)

    # oracle on the sampled rows, compact pool: sampled row j owns slot j
    o_pool = np.stack([gen.slot_state(int(slots_np[r])).double().numpy() for r in sample])
    o_rec = o_pool.copy()
    o_xr = np.full((k, H, L, P), np.nan)
    o_dr = np.full((k, H, L), np.nan)
    o_br = np.full((k, G, L, N), np.nan)
    o_sl = np.arange(k)
    o_wp = np.zeros(k, np.int32)
    o_fl = np.full(k, 1 if L == 1 else 0, np.uint8)
    c_wp = np.zeros(nb, np.int32)                 # cursor model, all rows
    c_fl = np.full(nb, 1 if L == 1 else 0, np.uint8)
    samp_t = torch.tensor(sample, dtype=torch.long)
    worst = {"y": 0.0, "y_std": 0.0, "state_flush": 0.0, "dt_ring": 0.0}

    def one_step(inp, label, compare):
        nonlocal wp, fl, nwp, nfl, o_wp, o_fl, c_wp, c_fl
        gi = {n: v.to(dev) for n, v in inp.items()}
        flushing = c_fl.astype(bool).copy()
        w_before = c_wp.copy()
        calls[0] += 1
        sr_g = dict(rounding=rounding, sr_seed=SR_SEED, sr_offset=calls[0]) if sr_on else {}
        sr_o = dict(sr_g, sr_slots=slots_np[sample]) if sr_on else {}
        y = R.replayssm_decode(st_r, xr, dr, br, sl, wp, fl, gi["x"], gi["dt"], gp["A"],
                               gi["B"], gi["C"], D=gp["D"], z=gi["z"],
                               dt_bias=gp["dt_bias"], next_write_pos=nwp,
                               next_is_flush=nfl, status=status, out_dtype=y_dtype, **sr_g)
        ys = None
        if standard:
            ys = R.ssu_standard_decode(st_s, sl, gi["x"], gi["dt"], gp["A"], gi["B"],
                                       gi["C"], D=gp["D"], z=gi["z"],
                                       dt_bias=gp["dt_bias"], status=status,
                                       out_dtype=y_dtype, **sr_g)
        wp, nwp = nwp, wp
        fl, nfl = nfl, fl
        ni = {n: v[samp_t].double().numpy() for n, v in inp.items()}
        y_ref, o_wp, o_fl, ost = OM.replay_step(
            o_pool, o_xr, o_dr, o_br, o_sl, o_wp, o_fl, ni["x"], ni["dt"], pn["A"],
            ni["B"], ni["C"], D=pn["D"], z=ni["z"], dt_bias=pn["dt_bias"],
            state_dtype=sdt, **sr_o)
        assert ost == 0
        # the recurrence always advances: it is also the reference for the
        # state the GPU's checkpoint + ring represent at the end
        ys_ref = OM.ssu_standard_step(o_rec, o_sl, ni["x"], ni["dt"], pn["A"], ni["B"],
                                      ni["C"], D=pn["D"], z=ni["z"],
                                      dt_bias=pn["dt_bias"], state_dtype=sdt, **sr_o)
        c_wp, c_fl = OM.cursor_advance(c_wp, c_fl, L)
        if not compare:
            return
        got_wp = wp.cpu().numpy()
        got_fl = fl.cpu().numpy()
        if not (np.array_equal(got_wp, c_wp) and np.array_equal(got_fl, c_fl)):
            bad = np.nonzero((got_wp != c_wp) | (got_fl != c_fl))[0][:8]
            raise AssertionError(f"{label}: cursor mismatch at rows {bad.tolist()}")
        assert int(status.item()) == 0, f"{label}: status {int(status.item())}"
        worst["y"] = max(worst["y"], tol_y.check(f"{label} y", _np(y[samp_t]), y_ref))
        if standard:
            worst["y_std"] = max(worst["y_std"],
                                 tol_y.check(f"{label} y_std", _np(ys[samp_t]), ys_ref))
        for j, r in enumerate(sample):
            s = int(slots_np[r])
            if flushing[r]:
                e = tol_state.check(f"{label} row {r} stored state", _np(st_r[s]), o_pool[j])
                worst["state_flush"] = max(worst["state_flush"], e)
            else:
                w = int(w_before[r])
                assert torch.equal(xr[s, :, w, :].cpu(), inp["x"][r]), f"{label}: x ring copy"
                g_writer_ok = torch.equal(br[s, :, w, :].cpu(), inp["B"][r])
                assert g_writer_ok, f"{label}: B ring copy"
                e = float(np.abs(_np(dr[s, :, w]) - o_dr[j, :, w]).max())
                worst["dt_ring"] = max(worst["dt_ring"], e)
                assert e <= 1e-6 * max(1.0, np.abs(o_dr[j, :, w]).max()), f"{label}: dt ring"

    if wl.desync:
        for kstep in range(L):
            force = gen.warm_force_flush(kstep)
            fl |= force.to(dev)
            c_fl = c_fl | force.numpy()
            o_fl = o_fl | force.numpy()[sample]
            one_step(gen.warm_step(kstep), f"{wl.name} warm {kstep}", compare=True)
        assert np.array_equal(c_wp, gen.start_positions().numpy())
    for t in range(steps):
        rows, fresh = gen.resets(t)
        if rows:
            ss = sl[torch.tensor(rows, dtype=torch.long, device=dev)].long()
            st_r[ss] = fresh.to(dev)
            if standard:
                st_s[ss] = fresh.to(dev)
            # stale ring entries are poisoned: they must never be read again
            xr[ss] = float("nan")
            dr[ss] = float("nan")
            br[ss] = float("nan")
            R.replayssm_ring_reset(wp, fl, torch.tensor(rows, dtype=torch.int32, device=dev), L)
            c_wp, c_fl = OM.ring_reset(c_wp, c_fl, rows, L)
            for j, r in enumerate(sample):
                if r in rows:
                    o_pool[j] = fresh[rows.index(r)].double().numpy()
                    o_rec[j] = o_pool[j]
            o_wp, o_fl = OM.ring_reset(o_wp, o_fl, [j for j, r in enumerate(sample) if r in rows], L)
        one_step(gen.step(t), f"{wl.name} step {t}",
                 compare=(t % check_every == 0) or t == steps - 1)
    torch.cuda.synchronize()
    # end state: the state the GPU's checkpoint + ring represent, against the
    # recurrence; and the standard update's state
    for j, r in enumerate(sample):
        s = int(slots_np[r])
        if sr_on:
            if standard:
                tol_state.check(f"{wl.name} row {r} standard state", _np(st_s[s]), o_rec[j])
            continue
        logical = OM.replay_logical_state(
            _np(st_r[s])[None], _np(xr[s])[None], _np(dr[s])[None], _np(br[s])[None],
            0, int(c_wp[r]), pn["A"])
        tol_state.check(f"{wl.name} row {r} GPU checkpoint+ring vs recurrence",
                        logical, o_rec[j])
        if standard:
            tol_state.check(f"{wl.name} row {r} standard state", _np(st_s[s]), o_rec[j])
    worst["seconds"] = round(time.time() - t0, 1)
    log(f"{wl.name}: {worst}")
    return worst


def run_gdn(wl, sample, o_dtype=torch.float32, steps=None, standard=True,
            check_every=1, dev="cuda:0", tol=None):
    t0 = time.time()
    dev = torch.device(dev)
    gen = GdnInputs(wl)
    nb, HK, HV, K, V, L = wl.batch, wl.k_heads, wl.v_heads, wl.dk, wl.dv, wl.ring_len
    ns = wl.num_slots
    steps = wl.steps if steps is None else steps
    io = TORCH_DTYPES[wl.io_dtype]
    fp32_path = wl.io_dtype == "f32"
    if tol is None:
        bf16_o = o_dtype == torch.bfloat16
        tol = Tol("rel", 2e-5, bf16_o) if fp32_path else Tol("abs", 1e-2, bf16_o)
    tol_state = Tol("rel", 2e-5) if fp32_path else Tol("abs", 1e-2)
    sample = sorted(set(int(r) for r in sample))
    k = len(sample)
    kda = wl.kda
    gshape = (K,) if kda else ()  # per-entry gate: a [K] row (KDA) or a scalar (GDN)
    rep_fn = R.replayssm_kda_decode if kda else R.replayssm_gdn_decode
    std_fn = R.kda_standard_decode if kda else R.gdn_standard_decode
    rep_ref = OK.kda_replay_step if kda else OG.gdn_replay_step
    std_ref = OK.kda_standard_step if kda else OG.gdn_standard_step
    slots = gen.slot_idx()
    slots_np = slots.numpy()
    pool = gen.state_pool(slots.tolist())
    st_r = pool.to(dev)
    st_s = pool.to(dev) if standard else None
    del pool
    dr = torch.full((ns, HV, L, V), float("nan"), dtype=torch.float32, device=dev)
    kr = torch.full((ns, HK, L, K), float("nan"), dtype=io, device=dev)
    gr = torch.full((ns, HV, L) + gshape, float("nan"), dtype=torch.float32, device=dev)
    wp = torch.zeros(nb, dtype=torch.int32, device=dev)
    fl = torch.full((nb,), 1 if L == 1 else 0, dtype=torch.uint8, device=dev)
    nwp, nfl = torch.empty_like(wp), torch.empty_like(fl)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    sl = slots.to(dev)
    o_pool = np.stack([gen.slot_state(int(slots_np[r])).double().numpy() for r in sample])
    o_rec = o_pool.copy()
    o_dr = np.full((k, HV, L, V), np.nan)
    o_kr = np.full((k, HK, L, K), np.nan)
    o_gr = np.full((k, HV, L) + gshape, np.nan)
    o_sl = np.arange(k)
    o_wp = np.zeros(k, np.int32)
    o_fl = np.full(k, 1 if L == 1 else 0, np.uint8)
    c_wp = np.zeros(nb, np.int32)
    c_fl = np.full(nb, 1 if L == 1 else 0, np.uint8)
    samp_t = torch.tensor(sample, dtype=torch.long)
    worst = {"o": 0.0, "o_std": 0.0, "state_flush": 0.0}

    def one_step(inp, label, compare):
        nonlocal wp, fl, nwp, nfl, o_wp, o_fl, c_wp, c_fl
        gi = {n: v.to(dev) for n, v in inp.items()}
        flushing = c_fl.astype(bool).copy()
        w_before = c_wp.copy()
        o = rep_fn(st_r, dr, kr, gr, sl, wp, fl, gi["q"], gi["k"], gi["v"], gi["g"],
                   gi["beta"], next_write_pos=nwp, next_is_flush=nfl, status=status,
                   out_dtype=o_dtype)
        os_ = None
        if standard:
            os_ = std_fn(st_s, sl, gi["q"], gi["k"], gi["v"], gi["g"], gi["beta"],
                         status=status, out_dtype=o_dtype)
        wp, nwp = nwp, wp
        fl, nfl = nfl, fl
        ni = {n: v[samp_t].double().numpy() for n, v in inp.items()}
        o_ref, o_wp, o_fl, ost = rep_ref(
            o_pool, o_dr, o_kr, o_gr, o_sl, o_wp, o_fl, ni["q"], ni["k"], ni["v"],
            ni["g"], ni["beta"], state_dtype="f32")
        assert ost == 0
        # the recurrence always advances: it is also the reference for the
        # state the GPU's checkpoint + ring represent at the end
        os_ref = std_ref(o_rec, o_sl, ni["q"], ni["k"], ni["v"], ni["g"], ni["beta"],
                         state_dtype="f32")
        c_wp, c_fl = OM.cursor_advance(c_wp, c_fl, L)
        if not compare:
            return
        got_wp = wp.cpu().numpy()
        got_fl = fl.cpu().numpy()
        if not (np.array_equal(got_wp, c_wp) and np.array_equal(got_fl, c_fl)):
            raise AssertionError(f"{label}: cursor mismatch")
        assert int(status.item()) == 0, f"{label}: status {int(status.item())}"
        worst["o"] = max(worst["o"], tol.check(f"{label} o", _np(o[samp_t]), o_ref))
        if standard:
            worst["o_std"] = max(worst["o_std"],
                                 tol.check(f"{label} o_std", _np(os_[samp_t]), os_ref))
        for j, r in enumerate(sample):
            s = int(slots_np[r])
            if flushing[r]:
                e = tol_state.check(f"{label} row {r} stored state", _np(st_r[s]), o_pool[j])
                worst["state_flush"] = max(worst["state_flush"], e)
            else:
                w = int(w_before[r])
                hk_rows = inp["k"][r]
                assert torch.equal(kr[s, :, w, :].cpu(), hk_rows), f"{label}: k ring copy"
                tol_state.check(f"{label} d ring", _np(dr[s, :, w, :]), o_dr[j, :, w, :])
                assert torch.equal(gr[s, :, w].cpu(), inp["g"][r]), f"{label}: g ring copy"

    if wl.desync:
        for kstep in range(L):
            force = gen.warm_force_flush(kstep)
            fl |= force.to(dev)
            c_fl = c_fl | force.numpy()
            o_fl = o_fl | force.numpy()[sample]
            one_step(gen.warm_step(kstep), f"{wl.name} warm {kstep}", compare=True)
    for t in range(steps):
        one_step(gen.step(t), f"{wl.name} step {t}",
                 compare=(t % check_every == 0) or t == steps - 1)
    torch.cuda.synchronize()
    # end state: the state the GPU's checkpoint + ring represent (its ring
    # entries 0..w-1 folded by the oracle), against the recurrence; and the
    # standard update's state
    logical_of = OK.kda_replay_logical_state if kda else OG.gdn_replay_logical_state
    worst["end_state"] = 0.0
    for j, r in enumerate(sample):
        s = int(slots_np[r])
        logical = logical_of(_np(st_r[s])[None], _np(dr[s])[None], _np(kr[s])[None],
                             _np(gr[s])[None], 0, int(c_wp[r]))
        e = tol_state.check(f"{wl.name} row {r} GPU checkpoint+ring vs recurrence",
                            logical, o_rec[j])
        worst["end_state"] = max(worst["end_state"], e)
        if standard:
            tol_state.check(f"{wl.name} row {r} standard state", _np(st_s[s]), o_rec[j])
    worst["seconds"] = round(time.time() - t0, 1)
    log(f"{wl.name}: {worst}")
    return worst
