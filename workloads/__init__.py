"""Seeded synthetic decode workloads shared by the tests, the bench and smoke.

This module only draws random inputs and rounds them to their storage dtype.
It holds none of the decode method's arithmetic, and it is the only code the
oracle side and the device side have in common.

Recipe (one workload per decode shape; values drawn with NumPy PCG64):

* x, z ~ N(0, 1); dt_raw ~ N(0, 1); B, C ~ N(0, 1) / 4 (N(0,1)/sqrt(16) read
  literally at every dstate); D ~ N(0, 1); A = -exp(U[0, ln 16]);
  dt_bias = log(expm1(U[1e-3, 1e-1])) (the inverse of softplus, so that
  softplus(dt_bias) is uniform on [1e-3, 1e-1]); initial state ~ N(0, 0.1)
  (standard deviation 0.1).
* GDN: q, k = N(0, 1) rows normalised to unit L2 norm (in float64, before
  rounding); v ~ N(0, 1); beta = sigmoid(N(0, 1)); g = exp(-softplus(N(0,1))),
  one draw per (row, value head), or per (row, value head, key channel) for
  the KDA gate.
* Every draw is rounded to its storage dtype here (bf16 by round-to-nearest-
  even through ``torch.Tensor.to``); consumers read exactly those values.
* Streams are independent and addressable: the stream for (tag, index) is
  PCG64(SeedSequence(seed, spawn_key=(tag, index))), with tags for the
  parameters, each slot's initial state, each decode step, each warm-up step
  and each reset.  The seed of the i-th workload in ``ALL`` is 1000 + i.

Tensors are returned on the CPU; callers move them where they need them.
"""

from dataclasses import dataclass, field
import math

import numpy as np
import torch

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16,
                "f64": torch.float64}

_TAG_PARAMS, _TAG_STATE, _TAG_STEP, _TAG_WARM, _TAG_RESET, _TAG_LAYOUT = range(6)


def _rng(seed, tag, index=0):
    ss = np.random.SeedSequence(seed, spawn_key=(tag, index))
    return np.random.Generator(np.random.PCG64(ss))


def _to(a, dtype):
    """float32/float64 numpy -> torch CPU tensor in a storage dtype (RNE)."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(TORCH_DTYPES[dtype])


@dataclass(frozen=True)
class Mamba2Workload:
    """One Mamba2 decode shape and its input structure."""
    name: str
    batch: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    ring_len: int
    steps: int
    num_slots: int
    io_dtype: str
    state_dtype: str
    seed: int
    desync: bool = False             # per-row start position uniform in [0, L)
    reset_steps: tuple = ()          # steps at which some rows get a fresh slot
    reset_prob: float = 0.0

    @property
    def state_bytes_per_row(self):
        es = 2 if self.state_dtype == "bf16" else 4
        return self.nheads * self.headdim * self.dstate * es

    def with_ring(self, L, name=None):
        d = dict(self.__dict__)
        d["ring_len"] = L
        d["name"] = name or f"{self.name}_L{L}"
        return Mamba2Workload(**d)

    def with_batch(self, batch, steps=None, num_slots=None, name=None):
        d = dict(self.__dict__)
        d["batch"] = batch
        if steps is not None:
            d["steps"] = steps
        d["num_slots"] = num_slots or max(2 * batch, 8)
        d["name"] = name or f"{self.name}_b{batch}"
        return Mamba2Workload(**d)


@dataclass(frozen=True)
class GdnWorkload:
    name: str
    batch: int
    k_heads: int
    v_heads: int
    dk: int
    dv: int
    ring_len: int
    steps: int
    num_slots: int
    io_dtype: str
    state_dtype: str
    seed: int
    desync: bool = False
    kda: bool = False  # per-key-channel gate g [batch, HV, K] instead of [batch, HV]

    def with_batch(self, batch, steps=None, num_slots=None, name=None):
        d = dict(self.__dict__)
        d["batch"] = batch
        if steps is not None:
            d["steps"] = steps
        d["num_slots"] = num_slots or max(2 * batch, 8)
        d["name"] = name or f"{self.name}_b{batch}"
        return GdnWorkload(**d)


TINY = Mamba2Workload("tiny_b4_h8_p64_n16_L4", 4, 8, 64, 16, 1, 4, 32, 8,
                      "f32", "f32", 1000)
LAYER_2P7B = Mamba2Workload("mamba2_2p7b_layer_b64_L16", 64, 80, 64, 128, 1,
                            16, 256, 1024, "bf16", "f32", 1001)
LARGE_BATCH = Mamba2Workload("mamba2_b512_h80_L16_bf16state", 512, 80, 64,
                             128, 1, 16, 128, 1024, "bf16", "bf16", 1002,
                             desync=True)
GROUPED = Mamba2Workload("mamba2_grouped_b256_h128_g8", 256, 128, 64, 128, 8,
                         16, 192, 512, "bf16", "f32", 1003,
                         reset_steps=(37, 101, 150), reset_prob=1.0 / 8)
GROUPED_RINGS = (1, 4, 8, 16)
GDN = GdnWorkload("gdn_b256_hk16_hv32_k128_L16", 256, 16, 32, 128, 128, 16,
                  128, 512, "bf16", "f32", 1004)
KDA = GdnWorkload("kda_b256_h32_k128_L16", 256, 32, 32, 128, 128, 16, 128, 512, "bf16",
                  "f32", 1005, kda=True)

ALL = (TINY, LAYER_2P7B, LARGE_BATCH, GROUPED, GDN)


class Mamba2Inputs:
    """Seeded inputs of one Mamba2 workload."""

    def __init__(self, wl: Mamba2Workload):
        self.wl = wl

    def params(self):
        wl = self.wl
        r = _rng(wl.seed, _TAG_PARAMS)
        H = wl.nheads
        A = -np.exp(r.uniform(0.0, math.log(16.0), H))
        dt_target = r.uniform(1e-3, 1e-1, H)
        dt_bias = np.log(np.expm1(dt_target))
        D = r.standard_normal(H)
        return {"A": _to(A.astype(np.float32), "f32"),
                "D": _to(D.astype(np.float32), "f32"),
                "dt_bias": _to(dt_bias.astype(np.float32), "f32")}

    def slot_idx(self):
        wl = self.wl
        r = _rng(wl.seed, _TAG_LAYOUT, 0)
        if wl.batch > wl.num_slots:
            raise ValueError("batch exceeds the pool")
        return torch.from_numpy(
            r.permutation(wl.num_slots)[:wl.batch].astype(np.int32))

    def start_positions(self):
        """Per-row write position at step 0 (0 unless the workload desyncs)."""
        wl = self.wl
        if not wl.desync:
            return torch.zeros(wl.batch, dtype=torch.int32)
        r = _rng(wl.seed, _TAG_LAYOUT, 1)
        return torch.from_numpy(
            r.integers(0, wl.ring_len, wl.batch).astype(np.int32))

    def slot_state(self, slot, tag_index=None):
        """Initial state of one slot [H, P, N] in the state dtype."""
        wl = self.wl
        idx = slot if tag_index is None else tag_index
        r = _rng(wl.seed, _TAG_STATE, idx)
        a = r.standard_normal((wl.nheads, wl.headdim, wl.dstate),
                              dtype=np.float32) * np.float32(0.1)
        return _to(a, wl.state_dtype)

    def state_pool(self, slots=None):
        """Pool [num_slots, H, P, N]: drawn state in ``slots``, NaN elsewhere."""
        wl = self.wl
        if slots is None:
            slots = self.slot_idx().tolist()
        pool = torch.full((wl.num_slots, wl.nheads, wl.headdim, wl.dstate),
                          float("nan"), dtype=TORCH_DTYPES[wl.state_dtype])
        for s in slots:
            pool[s] = self.slot_state(int(s))
        return pool

    def _step_from(self, r, rows=None):
        wl = self.wl
        nb, H, P, N, G = wl.batch, wl.nheads, wl.headdim, wl.dstate, wl.ngroups
        x = r.standard_normal((nb, H, P), dtype=np.float32)
        z = r.standard_normal((nb, H, P), dtype=np.float32)
        dt = r.standard_normal((nb, H), dtype=np.float32)
        B = r.standard_normal((nb, G, N), dtype=np.float32) * np.float32(0.25)
        C = r.standard_normal((nb, G, N), dtype=np.float32) * np.float32(0.25)
        out = {"x": x, "z": z, "dt": dt, "B": B, "C": C}
        if rows is not None:
            out = {k: v[rows] for k, v in out.items()}
        return {k: _to(v, wl.io_dtype) for k, v in out.items()}

    def step(self, t, rows=None):
        """Inputs of decode step t: x, z [batch,H,P]; dt [batch,H]; B, C [batch,G,N]."""
        return self._step_from(_rng(self.wl.seed, _TAG_STEP, t), rows)

    def warm_step(self, k, rows=None):
        """Inputs of warm-up step k (the steps that desync the rings)."""
        return self._step_from(_rng(self.wl.seed, _TAG_WARM, k), rows)

    def warm_force_flush(self, k):
        """Rows the caller forces to flush at warm-up step k (uint8 [batch]).

        With L warm-up steps from an empty ring, forcing row r to flush at
        step L-1-w0[r] leaves exactly w0[r] ring entries at step 0.
        """
        wl = self.wl
        w0 = self.start_positions().numpy()
        return torch.from_numpy(
            ((wl.ring_len - 1 - w0) == k).astype(np.uint8))

    def resets(self, t):
        """(rows, fresh states [n, H, P, N]) of the slot reuses at step t."""
        wl = self.wl
        if t not in wl.reset_steps:
            return [], None
        r = _rng(wl.seed, _TAG_RESET, t)
        rows = np.nonzero(r.random(wl.batch) < wl.reset_prob)[0].tolist()
        if not rows:
            return [], None
        fresh = torch.stack([self.slot_state(0, tag_index=10_000_000 * (t + 1) + row)
                             for row in rows])
        return rows, fresh


class GdnInputs:
    """Seeded inputs of one GDN workload."""

    def __init__(self, wl: GdnWorkload):
        self.wl = wl

    def slot_idx(self):
        wl = self.wl
        r = _rng(wl.seed, _TAG_LAYOUT, 0)
        return torch.from_numpy(
            r.permutation(wl.num_slots)[:wl.batch].astype(np.int32))

    def start_positions(self):
        wl = self.wl
        if not wl.desync:
            return torch.zeros(wl.batch, dtype=torch.int32)
        r = _rng(wl.seed, _TAG_LAYOUT, 1)
        return torch.from_numpy(
            r.integers(0, wl.ring_len, wl.batch).astype(np.int32))

    def slot_state(self, slot):
        wl = self.wl
        r = _rng(wl.seed, _TAG_STATE, slot)
        a = r.standard_normal((wl.v_heads, wl.dv, wl.dk),
                              dtype=np.float32) * np.float32(0.1)
        return _to(a, wl.state_dtype)

    def state_pool(self, slots=None):
        wl = self.wl
        if slots is None:
            slots = self.slot_idx().tolist()
        pool = torch.full((wl.num_slots, wl.v_heads, wl.dv, wl.dk),
                          float("nan"), dtype=TORCH_DTYPES[wl.state_dtype])
        for s in slots:
            pool[s] = self.slot_state(int(s))
        return pool

    def _step_from(self, r, rows=None):
        wl = self.wl
        nb = wl.batch

        def unit(shape):
            a = r.standard_normal(shape)
            return (a / np.linalg.norm(a, axis=-1, keepdims=True)).astype(np.float32)

        q = unit((nb, wl.k_heads, wl.dk))
        k = unit((nb, wl.k_heads, wl.dk))
        v = r.standard_normal((nb, wl.v_heads, wl.dv), dtype=np.float32)
        beta = (1.0 / (1.0 + np.exp(-r.standard_normal((nb, wl.v_heads))))).astype(np.float32)
        a = r.standard_normal((nb, wl.v_heads, wl.dk) if wl.kda else (nb, wl.v_heads))
        g = np.exp(-(np.maximum(a, 0) + np.log1p(np.exp(-np.abs(a))))).astype(np.float32)
        out = {"q": q, "k": k, "v": v, "beta": beta, "g": g}
        if rows is not None:
            out = {kk: vv[rows] for kk, vv in out.items()}
        res = {kk: _to(out[kk], wl.io_dtype) for kk in ("q", "k", "v")}
        res["beta"] = _to(out["beta"], "f32")
        res["g"] = _to(out["g"], "f32")
        return res

    def step(self, t, rows=None):
        return self._step_from(_rng(self.wl.seed, _TAG_STEP, t), rows)

    def warm_step(self, k, rows=None):
        return self._step_from(_rng(self.wl.seed, _TAG_WARM, k), rows)

    def warm_force_flush(self, k):
        wl = self.wl
        w0 = self.start_positions().numpy()
        return torch.from_numpy(
            ((wl.ring_len - 1 - w0) == k).astype(np.uint8))


def device_normal_(t, std, seed):
    """Fill a device tensor with seeded N(0, std^2) (bench-sized pools)."""
    g = torch.Generator(device=t.device)
    g.manual_seed(seed)
    tmp = torch.empty(t.shape, dtype=torch.float32, device=t.device)
    tmp.normal_(0.0, std, generator=g)
    t.copy_(tmp)
    return t
