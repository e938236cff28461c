"""Decode throughput of the ReplaySSM kernels on one MI355X.

Headline: Mamba2 ReplaySSM decode (replayssm_decode) at batch 512, 80 heads,
headdim 64, dstate 128, ngroups 1, ring L = 16, bf16 inputs and bf16 state
pool (fp32 arithmetic), start positions uniform in [0, L) so flush rows
interleave every step.  One step = one replayssm_decode launch over the whole
batch for one layer; ``--layers`` (16) independent layers (state pool + rings
+ cursors each) are used round-robin, as consecutive decode steps of a model
with many layers would see them: between two steps of one layer the other
layers stream ~12 GB of checkpoints and ~1.5 GB of ring and write-back
traffic, so nothing a step reads is still in the 256 MB last-level cache.
(With only 4 layers a layer's ring entries and freshly flushed checkpoints
can still be cached when its next step reads them; that figure is reported
as ``layers4_context``.)
value = batch * steps / seconds (state-updates/s: one row advanced one step
through one layer), from the median of ``--reps`` timed regions of exactly
``--steps`` launches each.

Also measured in the same run (separate timed regions, each repeated):
replayssm_decode_ordered (the same step with the host's flush-first row
order; same results, bit for bit); the standard read+write update
(ssu_standard_decode) on the same workload; both again with stochastic
rounding of the bf16 write-back; one tensor-parallel rank's share of the
layer (10 of 80 heads); the GDN replay/standard decode at batch 256 (16 key
/ 32 value heads, K = V = 128, L = 16, bf16 q/k/v, fp32 state) and its
speculative verify + commit with 4 drafts per round (and the deferred-fold
rounds: a verify that folds the rows marked by the previous round, then the
cursor advance); the KDA
(per-key-channel gate) replay/standard decode at batch 256, 32 heads,
K = V = 128, L = 16; the host metadata builder; and the float64 CPU oracle
on a bounded sample, both the ReplaySSM reconstruction and the standard
recurrence on one thread (``cpu_baseline``, ``cpu_baseline_standard``) and
the reconstruction sharded by rows over up to 16 processes
(``cpu_baseline_parallel``), with the host's core count.

Roofline: algorithmic bytes per launch (checkpoint reads, ring reads of the
live entries, ring appends, flush write-backs, step inputs, outputs and
metadata, evaluated exactly from every row's cursor at that step) divided by
the average launch time measured with HIP events on the launch stream.
``traffic`` is the HBM bytes per replay launch from rocprofv3 FETCH_SIZE /
WRITE_SIZE counters (profiles/replayssm_decode_mamba2_b512_traffic.json),
reported only while its source fingerprint matches the kernel sources.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--reps R] [--layers 4]
       python bench.py --copy-probe      (copy kernel for counter calibration)
"""

import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "replayssm_decode_mamba2_b512_traffic.json")
METRIC = "decode state-updates/s + achieved HBM GB/s (% peak), Mamba2 B=512 L=16"


def _sizes(dt):
    return 2 if dt == torch.bfloat16 else 4


class Mamba2Layers:
    """`layers` independent Mamba2 layers of one workload, resident on the GPU."""

    def __init__(self, wl, layers, dev, y_dtype, seed=7):
        from workloads import TORCH_DTYPES, Mamba2Inputs, device_normal_
        self.wl, self.dev, self.nl = wl, dev, layers
        gen = Mamba2Inputs(wl)
        self.gen = gen
        H, P, N, G, L, ns = wl.nheads, wl.headdim, wl.dstate, wl.ngroups, wl.ring_len, wl.num_slots
        io = TORCH_DTYPES[wl.io_dtype]
        sdt = TORCH_DTYPES[wl.state_dtype]
        self.io, self.sdt, self.y_dtype = io, sdt, y_dtype
        self.prm = {k: v.to(dev) for k, v in gen.params().items()}
        self.slots = gen.slot_idx().to(dev)
        self.w0 = gen.start_positions().numpy()
        self.state, self.xr, self.dr, self.br = [], [], [], []
        self.std_state = []
        for l in range(layers):
            st = torch.empty((ns, H, P, N), dtype=sdt, device=dev)
            device_normal_(st, 0.1, seed + l)
            self.state.append(st)
            self.xr.append(torch.zeros((ns, H, L, P), dtype=io, device=dev))
            self.dr.append(torch.zeros((ns, H, L), dtype=torch.float32, device=dev))
            self.br.append(torch.zeros((ns, G, L, N), dtype=io, device=dev))
        nb = wl.batch
        self.wp = [torch.zeros(nb, dtype=torch.int32, device=dev) for _ in range(layers)]
        self.fl = [torch.full((nb,), 1 if L == 1 else 0, dtype=torch.uint8, device=dev)
                   for _ in range(layers)]
        self.nwp = [torch.empty_like(t) for t in self.wp]
        self.nfl = [torch.empty_like(t) for t in self.fl]
        self.steps_done = [0] * layers
        self.inputs = [{k: v.to(dev) for k, v in gen.step(t).items()} for t in range(8)]
        self.y = torch.empty((nb, H, P), dtype=y_dtype, device=dev)
        # per-row byte accounting
        sst, sio, sy = _sizes(sdt), _sizes(io), _sizes(y_dtype)
        self.tile = H * P * N * sst
        self.entry = H * P * sio + G * N * sio + 4 * H
        self.inp = 2 * H * P * sio + H * sio + 2 * G * N * sio + H * P * sy
        self.params = 3 * 4 * H

    def warm_rings(self):
        """Run the L warm-up steps that leave row r with w0[r] ring entries."""
        L = self.wl.ring_len
        for l in range(self.nl):
            for k in range(L):
                force = self.gen.warm_force_flush(k).to(self.dev)
                self.fl[l] |= force
                self.replay(l, self.inputs[k % 8])
            self.steps_done[l] = 0
        torch.cuda.synchronize()
        for l in range(self.nl):
            assert np.array_equal(self.wp[l].cpu().numpy(), self.w0), "warm-up cursors"

    def phase_orders(self):
        """Flush-first row orders for each step phase k (mod L) after the
        warm-up: row r flushes at phase k iff (w0[r] + k) % L == L-1, the flag
        the host metadata path holds; built by the library's host helper."""
        import linear_recurrence_amd as R
        L = self.wl.ring_len
        out = []
        for k in range(L):
            fl = ((self.w0 + k) % L == L - 1).astype(np.uint8)
            out.append(torch.from_numpy(R.flush_first_order(fl)).to(self.dev))
        return out

    def replay(self, l, inp, sr=None, order=None):
        import linear_recurrence_amd as R
        kw = {} if sr is None else dict(rounding="stochastic", sr_seed=17, sr_offset=sr)
        if order is not None:
            kw["row_order"] = order
        R.replayssm_decode(self.state[l], self.xr[l], self.dr[l], self.br[l], self.slots,
                           self.wp[l], self.fl[l], inp["x"], inp["dt"], self.prm["A"],
                           inp["B"], inp["C"], D=self.prm["D"], z=inp["z"],
                           dt_bias=self.prm["dt_bias"], y=self.y,
                           next_write_pos=self.nwp[l], next_is_flush=self.nfl[l], **kw)
        self.wp[l], self.nwp[l] = self.nwp[l], self.wp[l]
        self.fl[l], self.nfl[l] = self.nfl[l], self.fl[l]

    def standard(self, l, inp, sr=None):
        import linear_recurrence_amd as R
        kw = {} if sr is None else dict(rounding="stochastic", sr_seed=17, sr_offset=sr)
        R.ssu_standard_decode(self.state[l], self.slots, inp["x"], inp["dt"], self.prm["A"],
                              inp["B"], inp["C"], D=self.prm["D"], z=inp["z"],
                              dt_bias=self.prm["dt_bias"], y=self.y, **kw)

    def replay_bytes(self, step_in_layer, ordered=False):
        """Algorithmic bytes of one replay launch, from every row's cursor
        (plus the 4-byte row order entry when the launch takes one)."""
        L = self.wl.ring_len
        w = (self.w0 + step_in_layer) % L
        flush = w == L - 1
        per_row = (self.tile + w * self.entry + np.where(flush, self.tile, self.entry)
                   + self.inp + 14 + (4 if ordered else 0))
        return float(per_row.sum() + self.params)

    def standard_bytes(self):
        return float(self.wl.batch * (2 * self.tile + self.inp + 4) + self.params)


def time_region(fn, steps, warmup):
    """W untimed steps, then exactly K timed steps between synchronisations.
    The events are recorded on torch's current stream, which is the stream
    the binding launches every kernel on."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        fn(warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3  # seconds


def timed_reps(fn, steps, warmup, reps):
    """W untimed steps, then `reps` timed regions of exactly K steps each
    (the step index keeps counting across regions); seconds per region."""
    out = []
    for r in range(reps):
        out.append(time_region(lambda i: fn(r * steps + i + (0 if r == 0 else warmup)),
                               steps, warmup if r == 0 else 0))
    return out


def median(v):
    return float(np.median(np.asarray(v, dtype=np.float64)))


def spread(v):
    """Relative spread (max - min) / median of repeated measurements."""
    v = np.asarray(v, dtype=np.float64)
    return float((v.max() - v.min()) / np.median(v))


def bench_mamba2(wl, layers, steps, warmup, y_dtype, dev, reps, sr=False, ordered=True):
    """Timed regions of the replay (plain replayssm_decode: the headline),
    the standard update and, with `ordered`, replayssm_decode_ordered with
    the host's flush-first row lists; with sr, replay and standard again with
    stochastic rounding of the bf16 write-back (a fresh Philox offset every
    call).  Each kernel is timed in `reps` regions of `steps` launches; the
    median region is reported with the spread."""
    M = Mamba2Layers(wl, layers, dev, y_dtype)
    M.warm_rings()
    orders = M.phase_orders() if ordered else None
    # replay: step i uses layer i % layers; bytes are accounted per launch
    # from the cursors that layer has at that step
    step_of = [0] * layers
    base = [0]

    def rep(i, sr_on=False, use_order=False):
        l = i % layers
        order = orders[step_of[l] % wl.ring_len] if use_order else None
        M.replay(l, M.inputs[i % 8], sr=i if sr_on else None, order=order)
        step_of[l] += 1

    def replay_regions(sr_on, use_order):
        first = base[0]
        for i in range(warmup):
            rep(first + i, sr_on, use_order)
        torch.cuda.synchronize()
        ts, bs = [], []
        for r in range(reps):
            local = list(step_of)
            total = 0.0
            start = first + warmup + r * steps
            for i in range(steps):
                l = (start + i) % layers
                total += M.replay_bytes(local[l], use_order)
                local[l] += 1
            ts.append(time_region(lambda i: rep(start + i, sr_on, use_order), steps, 0))
            bs.append(total / steps)
        base[0] = first + warmup + reps * steps
        for l in range(layers):
            got = M.wp[l].cpu().numpy()
            assert np.array_equal(got, (M.w0 + step_of[l]) % wl.ring_len), "cursor drift"
        return ts, bs

    def summary(ts, bs, entry):
        k = int(np.argsort(ts)[len(ts) // 2])  # the median region
        gbps = [b * steps / t / 1e9 for t, b in zip(ts, bs)]
        return {"entry_point": entry, "seconds": ts[k], "bytes_per_launch": bs[k],
                "ms_per_step": ts[k] / steps * 1e3,
                "state_updates_per_s": wl.batch * steps / ts[k],
                "achieved_GBps": gbps[k], "frac": gbps[k] / PEAK_HBM_GBPS,
                "region_us_per_launch": [round(t / steps * 1e6, 2) for t in ts],
                "spread": spread(ts)}

    res = {"replay": summary(*replay_regions(False, False), "replayssm_decode")}

    def std(i, sr_on=False):
        M.standard(i % layers, M.inputs[i % 8], sr=i if sr_on else None)

    std_bytes = M.standard_bytes()
    ts = timed_reps(std, steps, warmup, reps)
    res["standard"] = summary(ts, [std_bytes] * reps, "ssu_standard_decode")
    if ordered:
        res["replay_ordered"] = summary(*replay_regions(False, True),
                                        "replayssm_decode_ordered")
        res["replay_ordered"]["note"] = (
            "host flush-first row lists, one per step phase (mod L), built by "
            "replayssm_flush_first_order and uploaded before the timed regions")
    if sr:
        res["sr_replay"] = summary(*replay_regions(True, False), "replayssm_decode")
        ts = timed_reps(lambda i: std(i, True), steps, warmup, reps)
        res["sr_standard"] = summary(ts, [std_bytes] * reps, "ssu_standard_decode")
    del M
    torch.cuda.empty_cache()
    return res


def bench_gdn(wl, layers, steps, warmup, dev, reps):
    import linear_recurrence_amd as R
    from workloads import TORCH_DTYPES, GdnInputs, device_normal_
    gen = GdnInputs(wl)
    HK, HV, K, V, L, ns, nb = wl.k_heads, wl.v_heads, wl.dk, wl.dv, wl.ring_len, wl.num_slots, wl.batch
    io = TORCH_DTYPES[wl.io_dtype]
    states = []
    for l in range(layers):
        st = torch.empty((ns, HV, V, K), dtype=torch.float32, device=dev)
        device_normal_(st, 0.1, 100 + l)
        states.append(st)
    gsh = (K,) if wl.kda else ()  # per-entry gate: a [K] row (KDA) or a scalar (GDN)
    rep_fn = R.replayssm_kda_decode if wl.kda else R.replayssm_gdn_decode
    std_fn = R.kda_standard_decode if wl.kda else R.gdn_standard_decode
    dr = [torch.zeros((ns, HV, L, V), device=dev) for _ in range(layers)]
    kr = [torch.zeros((ns, HK, L, K), dtype=io, device=dev) for _ in range(layers)]
    gr = [torch.zeros((ns, HV, L) + gsh, device=dev) for _ in range(layers)]
    wp = [torch.zeros(nb, dtype=torch.int32, device=dev) for _ in range(layers)]
    fl = [torch.zeros(nb, dtype=torch.uint8, device=dev) for _ in range(layers)]
    nwp = [torch.empty_like(t) for t in wp]
    nfl = [torch.empty_like(t) for t in fl]
    slots = gen.slot_idx().to(dev)
    inputs = [{k: v.to(dev) for k, v in gen.step(t).items()} for t in range(8)]
    o = torch.empty((nb, HV, V), dtype=io, device=dev)

    def rep(i):
        l = i % layers
        inp = inputs[i % 8]
        rep_fn(states[l], dr[l], kr[l], gr[l], slots, wp[l], fl[l], inp["q"], inp["k"],
               inp["v"], inp["g"], inp["beta"], o=o, next_write_pos=nwp[l],
               next_is_flush=nfl[l])
        wp[l], nwp[l] = nwp[l], wp[l]
        fl[l], nfl[l] = nfl[l], fl[l]

    def std(i):
        l = i % layers
        inp = inputs[i % 8]
        std_fn(states[l], slots, inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], o=o)

    # whole ring periods per layer keep the flush share exact (lock-step rows)
    steps_r = max(layers * L, (steps // (layers * L)) * layers * L)
    warm_r = layers * L
    ts_rep = timed_reps(rep, steps_r, warm_r, reps)
    ts_std = timed_reps(std, steps, warmup, reps)
    t_rep, t_std = median(ts_rep), median(ts_std)
    sio = _sizes(io)
    tile = HV * V * K * 4
    gate = HV * K * 4 if wl.kda else HV * 4  # one entry's gates
    entry = HV * V * 4 + HK * K * sio + gate
    inp_b = 2 * HK * K * sio + HV * V * sio + gate + HV * 4 + HV * V * sio
    # lock-step rows: over a ring period the positions are 0..L-1 once each
    ring_reads = sum(range(L)) / L * entry
    per_row_rep = tile + ring_reads + (L - 1) / L * entry + tile / L + inp_b + 14
    per_row_std = 2 * tile + inp_b + 4
    res = {
        "workload": wl.name,
        "replay_updates_per_s": nb * steps_r / t_rep,
        "standard_updates_per_s": nb * steps / t_std,
        "replay_GBps": per_row_rep * nb * steps_r / t_rep / 1e9,
        "standard_GBps": per_row_std * nb * steps / t_std / 1e9,
        "replay_us_per_step": t_rep / steps_r * 1e6,
        "standard_us_per_step": t_std / steps * 1e6,
        "replay_spread": spread(ts_rep), "standard_spread": spread(ts_std),
    }
    res["speedup"] = res["replay_updates_per_s"] / res["standard_updates_per_s"]
    del states, dr, kr, gr
    torch.cuda.empty_cache()
    return res


def bench_gdn_spec(wl, T, layers, rounds, warmup, dev, reps, deferred=False):
    """GDN speculative decoding from the ring: per round one verify of T drafts
    per row and one commit (accepted counts from a fixed seeded pattern; rows
    whose next verify would not fit fold their ring by the exact recurrence).
    deferred: the deferred-fold rounds instead, a verify that first folds the
    rows marked by the previous round, then the cursor advance (the fold then
    reuses the verify's read of the state tile).
    Every timed region starts from empty rings, runs `rounds` untimed rounds
    and then times the next `rounds` (the same rounds in every region);
    algorithmic bytes are counted per launch from every row's cursor."""
    import linear_recurrence_amd as R
    HK, HV, K, V, L, nb = wl.k_heads, wl.v_heads, wl.dk, wl.dv, wl.ring_len, wl.batch
    ns = 2 * nb
    io = torch.bfloat16
    sio = 2
    rng = np.random.default_rng(5)
    from workloads import device_normal_
    lay = []
    for l in range(layers):
        st = torch.empty((ns, HV, V, K), dtype=torch.float32, device=dev)
        device_normal_(st, 0.1, 300 + l)
        lay.append(dict(st=st, dr=torch.zeros((ns, HV, L, V), device=dev),
                        kr=torch.zeros((ns, HK, L, K), dtype=io, device=dev),
                        gr=torch.zeros((ns, HV, L), device=dev),
                        vr=torch.zeros((ns, HV, L, V), dtype=io, device=dev),
                        br=torch.zeros((ns, HV, L), device=dev),
                        wp=torch.zeros(nb, dtype=torch.int32, device=dev),
                        nwp=torch.zeros(nb, dtype=torch.int32, device=dev),
                        fl=torch.zeros(nb, dtype=torch.uint8, device=dev),
                        nfl=torch.zeros(nb, dtype=torch.uint8, device=dev),
                        w=np.zeros(nb, np.int64), f=np.zeros(nb, bool)))
    slots = torch.tensor(rng.permutation(ns)[:nb].astype(np.int32), device=dev)

    def unit(shape):
        a = torch.randn(shape, device=dev)
        return (a / a.norm(dim=-1, keepdim=True)).to(io)
    torch.manual_seed(5)
    inputs = [dict(q=unit((nb, T, HK, K)), k=unit((nb, T, HK, K)),
                   v=torch.randn((nb, T, HV, V), device=dev).to(io),
                   g=torch.exp(-torch.nn.functional.softplus(torch.randn((nb, T, HV), device=dev))),
                   beta=torch.sigmoid(torch.randn((nb, T, HV), device=dev))) for _ in range(4)]
    accepts = [rng.integers(0, T + 1, nb).astype(np.int32) for _ in range(8)]
    acc_t = [torch.tensor(a, device=dev) for a in accepts]
    o = torch.empty((nb, T, HV, V), dtype=io, device=dev)
    vpk = HV // HK
    tile = V * K * 4
    entry = V * 4 + K * sio / vpk + 4                    # d, k (shared per key head), g
    raw = V * sio + K * sio / vpk + 8                    # v, k, g, beta for the exact fold
    inp = T * (2 * K * sio / vpk + V * sio + 8 + V * sio)  # q, k, v, g, beta in; o out
    bytes_total = [0.0]

    def rnd(i, count=True):
        d = lay[i % layers]
        inp_i = inputs[i % 4]
        a = accepts[i % 8]
        w = d["w"]
        if deferred:
            R.replayssm_gdn_spec_verify_flush(d["st"], d["dr"], d["kr"], d["gr"], d["vr"],
                                              d["br"], slots, d["wp"], d["fl"], inp_i["q"],
                                              inp_i["k"], inp_i["v"], inp_i["g"], inp_i["beta"],
                                              o=o)
            R.replayssm_gdn_spec_advance(d["kr"], d["gr"], d["vr"], d["br"], slots, d["wp"],
                                         d["fl"], acc_t[i % 8], T, inp_i["k"], inp_i["v"],
                                         inp_i["g"], inp_i["beta"], d["nwp"], d["nfl"])
            d["fl"], d["nfl"] = d["nfl"], d["fl"]
            f = d["f"]
            wv = np.where(f, 0, w)
            if count:
                # verify: the tile, committed d, k, g rows, the drafts' d rows,
                # inputs and outputs; a folding row also writes its tile and
                # reads its raw rows (the tile read is the verify's); advance:
                # the kept drafts' v, k, g, beta rows read from the inputs
                # and written to the ring, and the cursors
                per_row = (tile + wv * entry + T * V * 4 + inp + 4) * HV \
                    + np.where(f, (tile + w * raw) * HV, 0) + 2 * a * raw * HV + 18
                bytes_total[0] += float(per_row.sum())
            d["w"] = wv + a
            d["f"] = d["w"] + T > L
        else:
            R.replayssm_gdn_spec_verify(d["st"], d["dr"], d["kr"], d["gr"], d["vr"], d["br"],
                                        slots, d["wp"], inp_i["q"], inp_i["k"], inp_i["v"],
                                        inp_i["g"], inp_i["beta"], o=o)
            R.replayssm_gdn_spec_commit(d["st"], d["kr"], d["gr"], d["vr"], d["br"], slots,
                                        d["wp"], acc_t[i % 8], T, d["nwp"])
            wn = w + a
            fold = wn + T > L
            if count:
                per_row = (tile + w * entry + T * (entry + V * sio + 4) + inp + 4) * HV \
                    + np.where(fold, (2 * tile + wn * raw) * HV, 0) + 12
                bytes_total[0] += float(per_row.sum())
            d["w"] = np.where(fold, 0, wn)
        d["wp"], d["nwp"] = d["nwp"], d["wp"]

    def reset():
        # every region starts from empty rings, so all regions run the same
        # rounds (the same folds, the same bytes)
        torch.cuda.synchronize()
        for d in lay:
            d["wp"].zero_()
            d["nwp"].zero_()
            d["fl"].zero_()
            d["nfl"].zero_()
            d["w"][:] = 0
            d["f"][:] = False

    # per region: empty rings, `rounds` untimed rounds (every row's fold cycle
    # is shorter), then `rounds` timed rounds, the same ones in every region
    for i in range(warmup):
        rnd(i, False)
    torch.cuda.synchronize()
    ts, bs = [], []
    for r in range(reps):
        reset()
        for i in range(rounds):
            rnd(i, False)
        bytes_total[0] = 0.0
        ts.append(time_region(lambda i: rnd(rounds + i), rounds, 0))
        bs.append(bytes_total[0])
        for l in range(layers):
            assert np.array_equal(lay[l]["wp"].cpu().numpy(), lay[l]["w"]), "spec cursor drift"
    assert max(bs) == min(bs)
    t = float(np.median(ts))
    bytes_total[0] = bs[0]
    acc_mean = float(np.mean([a.mean() for a in accepts]))
    res = {
        "workload": f"gdn_spec{'_deferred' if deferred else ''}_b{nb}_hk{HK}_hv{HV}_k{K}_L{L}_T{T}",
        "drafts_per_round": T, "mean_accepted": acc_mean,
        "rounds_per_s": rounds / t, "us_per_round": t / rounds * 1e6,
        "verified_tokens_per_s": nb * T * rounds / t,
        "committed_tokens_per_s": nb * acc_mean * rounds / t,
        "GBps": bytes_total[0] / t / 1e9, "frac": bytes_total[0] / t / 1e9 / PEAK_HBM_GBPS,
        "bytes_per_round": bytes_total[0] / rounds,
        "recurrent_verify_bytes_per_round": float(nb * HV * (1 + T) * tile),
        "spread": spread(ts),
    }
    del lay
    torch.cuda.empty_cache()
    return res


def _oracle_sample(wl, r0, r1, steps, kind="replay"):
    """The float64 oracle on batch rows [r0, r1) over `steps` steps from the
    workload's first (desync) warm-up step: kind "replay" runs the ReplaySSM
    reconstruction (replay_step, the rows' own flush schedule), kind
    "standard" the recurrence (ssu_standard_step) on the same inputs.  Inputs
    are drawn here; the returned function runs the steps on one thread and
    returns its start and end times."""
    from threadpoolctl import threadpool_limits

    from oracle import mamba2 as OM
    from workloads import Mamba2Inputs
    gen = Mamba2Inputs(wl)
    H, P, N, G, L = wl.nheads, wl.headdim, wl.dstate, wl.ngroups, wl.ring_len
    rows = r1 - r0
    slots = gen.slot_idx().numpy()[r0:r1]
    pool = np.stack([gen.slot_state(int(s)).double().numpy() for s in slots])
    prm = {n: v.double().numpy() for n, v in gen.params().items()}
    xr = np.full((rows, H, L, P), np.nan)
    dr = np.full((rows, H, L), np.nan)
    br = np.full((rows, G, L, N), np.nan)
    seq = []
    for t in range(steps):
        src = gen.warm_step(t) if t < L else gen.step(t - L)
        force = gen.warm_force_flush(t).numpy()[r0:r1] if t < L else np.zeros(rows, np.uint8)
        seq.append(({n: v[r0:r1].double().numpy() for n, v in src.items()}, force))

    def run():
        wp = np.zeros(rows, np.int32)
        fl = np.zeros(rows, np.uint8)
        idx = np.arange(rows)
        with threadpool_limits(1):
            t0 = time.perf_counter()
            for inp, force in seq:
                if kind == "standard":
                    OM.ssu_standard_step(pool, idx, inp["x"], inp["dt"], prm["A"], inp["B"],
                                         inp["C"], D=prm["D"], z=inp["z"],
                                         dt_bias=prm["dt_bias"], state_dtype=wl.state_dtype)
                    continue
                fl = fl | force
                _, wp, fl, _ = OM.replay_step(pool, xr, dr, br, idx, wp, fl,
                                              inp["x"], inp["dt"], prm["A"], inp["B"], inp["C"],
                                              D=prm["D"], z=inp["z"], dt_bias=prm["dt_bias"],
                                              state_dtype=wl.state_dtype)
            return t0, time.perf_counter()
    return run


def host_info():
    """Cores this process may run on, the machine's count, and the BLAS
    thread pools numpy would use (the oracle legs limit them to one)."""
    from threadpoolctl import threadpool_info
    pools = [{"api": p.get("internal_api"), "threads": p.get("num_threads")}
             for p in threadpool_info()]
    return {"affinity_cores": len(os.sched_getaffinity(0)), "cpu_count": os.cpu_count(),
            "blas_pools_default": pools}


def cpu_baseline(wl, rows, steps, kind="replay"):
    """The float64 oracle on a bounded sample of the workload: `rows` rows of
    the batch for `steps` steps, one thread; inputs drawn before the clock
    starts."""
    t0, t1 = _oracle_sample(wl, 0, rows, steps, kind)()
    dt = t1 - t0
    what = ("ReplaySSM reconstruction (replay_step)" if kind == "replay"
            else "standard recurrence (ssu_standard_step)")
    return {"value": rows * steps / dt, "unit": "state-updates/s", "cores": 1,
            "kind": "oracle",
            "sample": f"float64 NumPy {what}, {rows} of {wl.batch} rows x {steps} steps "
                      f"({wl.ring_len} desync warm-up steps first), one thread "
                      f"(BLAS limited to 1), {dt:.1f} s",
            "host": host_info()}


_SHARD_BARRIER = None


def _shard_init(barrier):
    global _SHARD_BARRIER
    _SHARD_BARRIER = barrier


def _shard_run(job):
    wl, r0, r1, steps = job
    run = _oracle_sample(wl, r0, r1, steps)
    _SHARD_BARRIER.wait()  # every shard has its inputs: start together
    return run()


def cpu_baseline_parallel(wl, rows_per_worker, steps, workers):
    """The same oracle sharded by rows over `workers` fresh processes (one
    thread each; each draws its rows' inputs, then all start together); rate =
    all row-steps / (last end - first start).  Called before this process
    initialises the GPU."""
    import multiprocessing as mp
    ctx = mp.get_context("spawn")
    nrows = min(wl.batch, rows_per_worker * workers)
    bounds = np.linspace(0, nrows, workers + 1).astype(int)
    jobs = [(wl, int(bounds[i]), int(bounds[i + 1]), steps) for i in range(workers)]
    with ctx.Pool(workers, initializer=_shard_init, initargs=(ctx.Barrier(workers),)) as pool:
        spans = pool.map(_shard_run, jobs, chunksize=1)
    dt = max(e for _, e in spans) - min(s for s, _ in spans)
    return {"value": nrows * steps / dt, "unit": "state-updates/s", "cores": workers,
            "kind": "oracle",
            "sample": f"float64 NumPy replay oracle, rows 0..{nrows - 1} of {wl.batch} x {steps} "
                      f"steps, {workers} processes of one thread, {dt:.1f} s",
            "host": host_info()}


def metadata_rate(rows, L, calls=2000):
    """Host metadata builder: rows per second on one core (decode bases and
    positions of a batch, align mode with 16-token blocks)."""
    import linear_recurrence_amd as R
    rng = np.random.default_rng(0)
    base = rng.integers(0, 4096, rows).astype(np.int64)
    pos = base + rng.integers(0, 8, rows).astype(np.int64)
    t0 = time.perf_counter()
    for _ in range(calls):
        R.build_metadata(pos, base, L, align_block=16)
        pos += 1
    dt = time.perf_counter() - t0
    fl = (rng.random(rows) < 1.0 / L).astype(np.uint8)
    t0 = time.perf_counter()
    for _ in range(calls):
        R.flush_first_order(fl)
    dto = time.perf_counter() - t0
    return {"rows_per_s": rows * calls / dt, "rows": rows, "calls": calls,
            "flush_first_order_rows_per_s": rows * calls / dto,
            "note": "host C++ through the Python binding, one core"}


def measured_traffic(path):
    """HBM bytes per replay launch from the committed counter summary, or
    None when there is none or the kernel sources changed since it was taken."""
    from profsum import source_sha256
    if not path or not os.path.exists(path):
        return None, "no counter summary"
    with open(path) as fh:
        t = json.load(fh)
    if t.get("source_sha256") != source_sha256("mamba2_decode_kernel"):
        return None, f"{os.path.relpath(path, ROOT)} predates the current kernel sources"
    return t["bytes_per_launch"], (
        f"{os.path.relpath(path, ROOT)}: FETCH_SIZE x {t['fetch_factor']:.3f} + "
        f"WRITE_SIZE x {t['write_factor']:.3f} per replay dispatch (copy-kernel scaled)")


def copy_probe(dev, gib=1.0, reps=5):
    """A plain device copy of known size, for scaling HBM counters."""
    n = int(gib * (1 << 30)) // 4
    a = torch.empty(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    a.fill_(1.0)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    t = time_region(lambda i: b.copy_(a), reps, 1)
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4,
                      "dispatches": reps + 1 + reps,
                      "copy_GBps": 2 * n * 4 * reps / t / 1e9}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--reps", type=int, default=5,
                    help="timed regions of --steps launches per kernel (median reported)")
    ap.add_argument("--layers", type=int, default=16,
                    help="independent layers used round-robin (Mamba2 80 heads, GDN, KDA)")
    ap.add_argument("--tp-layers", type=int, default=128,
                    help="independent layers for the 10-head tensor-parallel share")
    ap.add_argument("--y-dtype", choices=("bf16", "f32"), default="bf16")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle legs")
    ap.add_argument("--no-gdn", action="store_true", help="skip the GDN measurement")
    ap.add_argument("--no-kda", action="store_true", help="skip the KDA measurement")
    ap.add_argument("--cpu-rows", type=int, default=128)
    ap.add_argument("--cpu-steps", type=int, default=80)
    ap.add_argument("--cpu-std-rows", type=int, default=40)
    ap.add_argument("--traffic-json", default=TRAFFIC_JSON,
                    help="per-launch HBM bytes measured with rocprofv3 counters")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--no-sr", action="store_true",
                    help="skip the stochastic-rounding measurement")
    ap.add_argument("--no-ordered", action="store_true",
                    help="skip replayssm_decode_ordered (host row order)")
    ap.add_argument("--no-tp", action="store_true",
                    help="skip the one-rank tensor-parallel share (10 heads)")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the 4-layer comparison run of the headline workload")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the decode path has no cross-GPU exchange "
              "(rows and heads shard with zero communication), so only --gpus 1 is "
              "supported.", file=sys.stderr)
        sys.exit(2)
    if torch.cuda.device_count() < 1:  # counts devices without initialising them
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    from workloads import GDN, KDA, LARGE_BATCH
    cpu = cpu_std = cpu_par = None
    if not args.no_cpu and not args.copy_probe:
        # CPU legs first: the parallel one forks, which must happen before
        # this process initialises the GPU
        cpu = cpu_baseline(LARGE_BATCH, args.cpu_rows, args.cpu_steps)
        print(f"[bench] cpu oracle (replay) done: {cpu['sample']}", file=sys.stderr, flush=True)
        cpu_std = cpu_baseline(LARGE_BATCH, args.cpu_std_rows, args.cpu_steps, kind="standard")
        print(f"[bench] cpu oracle (standard) done: {cpu_std['sample']}", file=sys.stderr,
              flush=True)
        workers = min(16, len(os.sched_getaffinity(0)))
        cpu_par = cpu_baseline_parallel(LARGE_BATCH, 32, args.cpu_steps, workers)
        print(f"[bench] parallel cpu oracle done: {cpu_par['sample']}", file=sys.stderr,
              flush=True)
    import linear_recurrence_amd as R
    R.load()
    dev = torch.device("cuda:0")
    if args.copy_probe:
        copy_probe(dev)
        return

    wl = LARGE_BATCH
    reps = max(1, args.reps)
    y_dtype = torch.bfloat16 if args.y_dtype == "bf16" else torch.float32
    print(f"[bench] {wl.name}: layers={args.layers} steps={args.steps} warmup={args.warmup} "
          f"reps={reps}", file=sys.stderr, flush=True)
    m = bench_mamba2(wl, args.layers, args.steps, args.warmup, y_dtype, dev, reps,
                     sr=not args.no_sr, ordered=not args.no_ordered)
    rp, sd = m["replay"], m["standard"]
    print(f"[bench] mamba2 done: {rp['achieved_GBps']:.0f} GB/s replay, "
          f"{sd['achieved_GBps']:.0f} GB/s standard", file=sys.stderr, flush=True)
    tp = None
    if not args.no_tp:
        # one tensor-parallel rank's share of the same layer: 80 / 8 = 10 heads,
        # 16 rotated layers so the working set stays far above the last-level cache
        wl_tp = dataclasses.replace(wl, name="mamba2_b512_h10_L16_bf16state_tp8share",
                                    nheads=10)
        # warm-up: at least four passes over the rotated layers (a pass is
        # 128 launches here, ~3 ms)
        t = bench_mamba2(wl_tp, args.tp_layers, args.steps, max(args.warmup, 4 * args.tp_layers),
                         y_dtype, dev, reps, ordered=False)
        tp = {"workload": wl_tp.name, "nheads": 10, "layers_rotated": args.tp_layers,
              "replay_updates_per_s": t["replay"]["state_updates_per_s"],
              "replay_GBps": t["replay"]["achieved_GBps"], "replay_frac": t["replay"]["frac"],
              "replay_us_per_launch": t["replay"]["ms_per_step"] * 1e3,
              "standard_updates_per_s": t["standard"]["state_updates_per_s"],
              "standard_GBps": t["standard"]["achieved_GBps"],
              "standard_us_per_launch": t["standard"]["ms_per_step"] * 1e3,
              "replay_region_us_per_launch": t["replay"]["region_us_per_launch"],
              "standard_region_us_per_launch": t["standard"]["region_us_per_launch"],
              "speedup": t["replay"]["state_updates_per_s"]
              / t["standard"]["state_updates_per_s"],
              "spread": [t["replay"]["spread"], t["standard"]["spread"]]}
        print(f"[bench] tp8 share done: {tp['replay_GBps']:.0f} GB/s replay", file=sys.stderr,
              flush=True)
    ctx4 = None
    if args.layers != 4 and not args.no_context:
        # the same workload over only 4 rotated layers, for comparison: there
        # a layer's ring entries and freshly flushed checkpoints can still be
        # in the 256 MB last-level cache when its next step reads them, which
        # a model with many layers never sees
        c = bench_mamba2(wl, 4, args.steps, args.warmup, y_dtype, dev, reps, ordered=False)
        ctx4 = {"layers_rotated": 4,
                "replay_us_per_launch": c["replay"]["ms_per_step"] * 1e3,
                "replay_frac": c["replay"]["frac"],
                "standard_us_per_launch": c["standard"]["ms_per_step"] * 1e3,
                "standard_frac": c["standard"]["frac"]}
        print(f"[bench] 4-layer context done: {ctx4['replay_us_per_launch']:.1f} us replay",
              file=sys.stderr, flush=True)
    gdn = None
    if not args.no_gdn:
        gdn = bench_gdn(GDN, args.layers, args.steps, args.warmup, dev, reps)
        print(f"[bench] gdn done: {gdn['replay_GBps']:.0f} GB/s replay", file=sys.stderr,
              flush=True)
    kda = None
    if not args.no_kda:
        kda = bench_gdn(KDA, args.layers, args.steps, args.warmup, dev, reps)
        print(f"[bench] kda done: {kda['replay_GBps']:.0f} GB/s replay", file=sys.stderr,
              flush=True)
    spec = spec_def = None
    if not args.no_gdn:
        spec = bench_gdn_spec(GDN, 4, args.layers, 256, 16, dev, reps)
        print(f"[bench] gdn spec done: {spec['GBps']:.0f} GB/s", file=sys.stderr, flush=True)
        spec_def = bench_gdn_spec(GDN, 4, args.layers, 256, 16, dev, reps, deferred=True)
        print(f"[bench] gdn spec (deferred folds) done: {spec_def['us_per_round']:.1f} us/round",
              file=sys.stderr, flush=True)

    traffic, traffic_note = measured_traffic(args.traffic_json)
    line = {
        "metric": METRIC,
        "value": rp["state_updates_per_s"],
        "unit": "state-updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rp["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "batch": wl.batch, "nheads": wl.nheads,
            "headdim": wl.headdim, "dstate": wl.dstate, "ngroups": wl.ngroups,
            "ring_len": wl.ring_len, "num_slots": wl.num_slots,
            "io_dtype": wl.io_dtype, "state_dtype": wl.state_dtype,
            "y_dtype": args.y_dtype, "layers_rotated": args.layers,
            "start_positions": "uniform in [0, L)",
        },
        "timing": {"regions": reps, "launches_per_region": args.steps,
                   "reported": "median region", "events": "HIP events on the launch stream",
                   "replay_region_us_per_launch": rp["region_us_per_launch"],
                   "replay_spread": rp["spread"]},
        "hbm_GBps": rp["achieved_GBps"],
        "hbm_frac_of_peak": rp["frac"],
        "roofline": {
            "bound": "hbm", "achieved": rp["achieved_GBps"], "peak": PEAK_HBM_GBPS,
            "unit": "GB/s", "frac": rp["frac"], "traffic": traffic,
            "traffic_source": traffic_note,
            "kernel": "replayssm_decode (mamba2_decode_kernel, replay)",
            "algorithmic_bytes_per_launch": rp["bytes_per_launch"],
        },
        "cpu_baseline": cpu,
        "cpu_baseline_standard": cpu_std,
        "cpu_baseline_parallel": cpu_par,
        "standard": sd,
        "speedup_vs_standard": rp["state_updates_per_s"] / sd["state_updates_per_s"],
        "replay_ordered": m.get("replay_ordered"),
        "gdn": gdn,
        "kda": kda,
        "gdn_spec": spec,
        "gdn_spec_deferred": spec_def,
        "stochastic_rounding": (None if "sr_replay" not in m else {
            "replay_updates_per_s": m["sr_replay"]["state_updates_per_s"],
            "replay_GBps": m["sr_replay"]["achieved_GBps"],
            "standard_updates_per_s": m["sr_standard"]["state_updates_per_s"],
            "standard_GBps": m["sr_standard"]["achieved_GBps"]}),
        "tp8_share": tp,
        "layers4_context": ctx4,
        "metadata_builder": metadata_rate(wl.batch, wl.ring_len),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
