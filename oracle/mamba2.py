"""Mamba2 selective state update: recurrence and ReplaySSM replay (float64).

Test infrastructure only; see the package docstring.

Sources (vLLM #48018, "[Kernel] ReplaySSM: cache SSM inputs for faster Mamba2
standard decode"):

* Motivation: decode loads and stores the per-request (nheads, headdim,
  dstate) state every step; ReplaySSM keeps a small ring of the step inputs
  plus a periodic checkpoint, forms most outputs from checkpoint + ring
  without materialising the state, and writes the full state back once every
  L steps.
* Implementation item 1: a per-row ``is_flush`` flag picks the flush path
  (fold and write back) or the snapshot path (output only).
* Implementation items 2-3: the ring holds x, dt and B (``x_cache``,
  ``dt_cache``, ``B_cache``); per-row ``write_pos`` / ``is_flush`` come from
  the metadata builder.
* Key source snippet (``mamba_mixer2.py``): both the baseline and the replay
  op take (state, x, dt, A, B, C, D), ``dt_bias``, ``dt_softplus=True``,
  ``state_batch_indices`` and a preallocated output.

Conventions (the readings taken where the pages are silent):

* Shapes.  state pool ``[num_slots, H, P, N]``; x, z ``[batch, H, P]``;
  dt_raw ``[batch, H]`` (one dt per row and head, Mamba2 form); A, D,
  dt_bias ``[H]``; B, C ``[batch, G, N]``; head h reads group
  ``h // (H // G)``.
* Gate: y <- y * z * sigmoid(z), applied to the whole output including D*x.
* The ring stores x and B as given (input dtype) and dt *after* softplus.
* A flush folds every entry 0..w, the current step included; the current
  step is then not appended and the row's next write position is 0.  A flush
  may be requested before the ring is full (a forced flush).
* Output on a flush row is read from the folded state before rounding.
* Rings here are float64 arrays holding the exact stored values.

Status bits (rows outside the contract; their outputs are unspecified):
bit 0 = write_pos outside [0, L); bit 1 = write_pos == L-1 without flush
(no room left in the ring); bit 2 = slot index outside [0, num_slots).
Rows with bit 0 or 1 are processed as a flush at the clamped position; rows
with bit 2 are skipped (y = NaN, cursors reset).
"""

import numpy as np

from .numerics import store_tiles_sr, silu_gate, softplus, store

ST_BAD_WRITE_POS = 1
ST_RING_OVERFLOW = 2
ST_BAD_SLOT = 4


def head_groups(H, G):
    """Group index of every head: contiguous blocks of H // G heads."""
    if G < 1 or H % G:
        raise ValueError("ngroups must divide nheads")
    return np.arange(H) // (H // G)


def dt_process(dt_raw, dt_bias, dt_softplus):
    """dt = softplus(dt_raw + dt_bias), or dt_raw + dt_bias without softplus."""
    v = np.asarray(dt_raw, dtype=np.float64)
    if dt_bias is not None:
        v = v + np.asarray(dt_bias, dtype=np.float64)[None, :]
    return softplus(v) if dt_softplus else v


def _write_state(state, slots, S, state_dtype, rounding, sr_seed, sr_offset, sr_slots=None):
    """Write state tiles S [k, H, P, N] to pool slots; nearest rounding or,
    for a bf16 pool, stochastic rounding with tile index slot * H + head
    (``sr_slots`` names the slots whose random bits to use when this pool is
    a compact copy of a larger one)."""
    slots = np.asarray(slots).reshape(-1)
    if rounding == "stochastic":
        if state_dtype != "bf16":
            raise ValueError("stochastic rounding applies to a bf16 state")
        H = S.shape[1]
        ts = slots if sr_slots is None else np.asarray(sr_slots).reshape(-1)
        tiles = ts[:, None] * H + np.arange(H)[None, :]
        state[slots] = store_tiles_sr(S, tiles, sr_seed, sr_offset)
    elif rounding == "nearest":
        state[slots] = store(S, state_dtype)
    else:
        raise ValueError(f"unknown rounding {rounding!r}")


def ssu_standard_step(state, slot_idx, x, dt_raw, A, B, C, D=None, z=None,
                      dt_bias=None, dt_softplus=True, state_dtype="f64",
                      rounding="nearest", sr_seed=0, sr_offset=0, sr_slots=None):
    """One step of the standard (read + write) selective state update.

    For each row b (slot s = slot_idx[b]) and head h:
        dt = softplus(dt_raw + dt_bias)
        S  = exp(dt * A[h]) * S + dt * outer(x[b, h], B[b, g(h)])
        y  = S @ C[b, g(h)] + D[h] * x[b, h];   y *= z * sigmoid(z)
    and S is written back to the pool in ``state_dtype`` (bf16 by nearest or
    stochastic rounding, see ``numerics.store_tiles_sr``).
    ``state`` is modified in place; returns y as float64 [batch, H, P].
    """
    x = np.asarray(x, np.float64)
    B = np.asarray(B, np.float64)
    C = np.asarray(C, np.float64)
    A = np.asarray(A, np.float64)
    nb, H, P = x.shape
    grp = head_groups(H, B.shape[1])
    Bh = B[:, grp, :]                                   # [batch, H, N]
    Ch = C[:, grp, :]
    dt = dt_process(dt_raw, dt_bias, dt_softplus)       # [batch, H]
    decay = np.exp(dt * A[None, :])                     # [batch, H]
    S = state[slot_idx]                                 # [batch, H, P, N]
    S = (decay[:, :, None, None] * S
         + (dt[:, :, None] * x)[:, :, :, None] * Bh[:, :, None, :])
    y = np.matmul(S, Ch[:, :, :, None])[..., 0]         # [batch, H, P]
    if D is not None:
        y = y + np.asarray(D, np.float64)[None, :, None] * x
    if z is not None:
        y = silu_gate(y, z)
    _write_state(state, slot_idx, S, state_dtype, rounding, sr_seed, sr_offset, sr_slots)
    return y


def cursor_advance(write_pos, is_flush, L):
    """Next cursors: w' = 0 after a flush, else w + 1; flush' = (w' == L - 1)."""
    w = np.asarray(write_pos, np.int64)
    f = np.asarray(is_flush).astype(bool)
    nxt = np.where(f, 0, w + 1)
    return nxt.astype(np.int32), (nxt == L - 1).astype(np.uint8)


def ring_reset(write_pos, is_flush, rows, L):
    """Rows that received a fresh checkpoint restart with an empty ring."""
    write_pos = np.array(write_pos, np.int32)
    is_flush = np.array(is_flush, np.uint8)
    for r in rows:
        write_pos[r] = 0
        is_flush[r] = 1 if L == 1 else 0
    return write_pos, is_flush


def replay_step(state, x_ring, dt_ring, B_ring, slot_idx, write_pos, is_flush,
                x, dt_raw, A, B, C, D=None, z=None, dt_bias=None,
                dt_softplus=True, state_dtype="f64", rounding="nearest", sr_seed=0,
                sr_offset=0, sr_slots=None):
    """One ReplaySSM output-only decode step over a batch.

    ``state`` (the checkpoint pool S0), ``x_ring`` [slots, H, L, P],
    ``dt_ring`` [slots, H, L] and ``B_ring`` [slots, G, L, N] are float64 and
    are modified in place.  For row b with slot s, position w and flag f the
    entries 0..w-1 come from the ring and entry w is the current step; with
    T = sum_{j<=w} dt_j and r_i = sum_{i<j<=w} dt_j:

        cumdecay = exp(A * T),   wt_i = dt_i * exp(A * r_i)
        y = cumdecay * (S0 @ C) + sum_i wt_i * (B_i . C) * x_i + D * x_w

    (the recurrence unrolled from S0 over the window).  On a flush row
    S_new = cumdecay * S0 + sum_i wt_i * outer(x_i, B_i) is written to the
    pool, y = S_new @ C + D * x_w, and w' = 0; otherwise the current
    (x, dt, B) is written at ring position w and w' = w + 1.

    Returns (y [batch, H, P] float64, next_write_pos int32, next_is_flush
    uint8, status int).
    """
    x = np.asarray(x, np.float64)
    B = np.asarray(B, np.float64)
    C = np.asarray(C, np.float64)
    A = np.asarray(A, np.float64)
    nb, H, P = x.shape
    L = x_ring.shape[2]
    num_slots = state.shape[0]
    grp = head_groups(H, B.shape[1])
    dt = dt_process(dt_raw, dt_bias, dt_softplus)
    Dv = None if D is None else np.asarray(D, np.float64)

    y = np.full((nb, H, P), np.nan)
    nwp = np.zeros(nb, np.int32)
    status = 0
    for b in range(nb):
        s = int(slot_idx[b])
        w = int(write_pos[b])
        f = bool(is_flush[b])
        if s < 0 or s >= num_slots:
            status |= ST_BAD_SLOT
            nwp[b] = 0
            continue
        if w < 0 or w >= L:
            status |= ST_BAD_WRITE_POS
            w = min(max(w, 0), L - 1)
            f = True
        if w == L - 1 and not f:
            status |= ST_RING_OVERFLOW
            f = True

        # entries 0..w: ring then the current step
        xs = np.concatenate([x_ring[s, :, :w, :], x[b][:, None, :]], axis=1)
        dts = np.concatenate([dt_ring[s, :, :w], dt[b][:, None]], axis=1)
        Bs = np.concatenate([B_ring[s][:, :w, :], B[b][:, None, :]], axis=1)
        Bs = Bs[grp]                                    # [H, w+1, N]
        Cb = C[b][grp]                                  # [H, N]

        total = dts.sum(axis=1)                         # [H]
        cumdecay = np.exp(A * total)
        suffix = np.array([[dts[h, i + 1:].sum() for i in range(w + 1)]
                           for h in range(H)])          # [H, w+1]
        wt = dts * np.exp(A[:, None] * suffix)          # [H, w+1]

        S0 = state[s]                                   # [H, P, N]
        if f:
            S_new = (cumdecay[:, None, None] * S0
                     + np.einsum("hi,hip,hin->hpn", wt, xs, Bs))
            yb = np.matmul(S_new, Cb[:, :, None])[..., 0]
            _write_state(state, [s], S_new[None], state_dtype, rounding, sr_seed, sr_offset,
                         None if sr_slots is None else [sr_slots[b]])
            nwp[b] = 0
        else:
            u = np.matmul(S0, Cb[:, :, None])[..., 0]   # [H, P]
            bc = np.einsum("hin,hn->hi", Bs, Cb)        # [H, w+1]
            yb = cumdecay[:, None] * u + np.einsum("hi,hip->hp", wt * bc, xs)
            x_ring[s, :, w, :] = x[b]
            dt_ring[s, :, w] = dt[b]
            B_ring[s, :, w, :] = B[b]
            nwp[b] = w + 1
        if Dv is not None:
            yb = yb + Dv[:, None] * x[b]
        if z is not None:
            yb = silu_gate(yb, np.asarray(z[b], np.float64))
        y[b] = yb
    nfl = (nwp == L - 1).astype(np.uint8)
    return y, nwp, nfl, status


def replay_logical_state(state, x_ring, dt_ring, B_ring, slot, write_pos, A):
    """The state S0 + ring represent for one slot: the fold of entries 0..w-1.

    Used to compare with the recurrence between flushes.
    """
    A = np.asarray(A, np.float64)
    H = state.shape[1]
    G = B_ring.shape[1]
    grp = head_groups(H, G)
    w = int(write_pos)
    S0 = state[slot]
    if w == 0:
        return S0.copy()
    xs = x_ring[slot, :, :w, :]
    dts = dt_ring[slot, :, :w]
    Bs = B_ring[slot][:, :w, :][grp]
    total = dts.sum(axis=1)
    suffix = np.array([[dts[h, i + 1:].sum() for i in range(w)]
                       for h in range(H)])
    wt = dts * np.exp(A[:, None] * suffix)
    return (np.exp(A * total)[:, None, None] * S0
            + np.einsum("hi,hip,hin->hpn", wt, xs, Bs))
