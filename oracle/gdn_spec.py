"""GDN speculative verify from the checkpoint + ring, and the commit with its
exact fold (float64).

Test infrastructure only; see the package docstring.

Source: sglang #28695 "[GDN] Support ReplaySSM Ring Spec-Verify" - Motivation
(the recurrent verify stores a full state snapshot per draft token, the bulk
of spec-decode memory), Implementation items 2-4 (per-slot ring of d, k, g
plus the raw inputs v, k and beta; a verify kernel that rebuilds the outputs
of the draft tokens from the frozen checkpoint and the ring; an exact-fold
kernel that, on flush, replays the raw inputs in order through the recurrent
update; commit after verify advances the cursor instead of copying a
snapshot; linear draft chains only; ring length at least twice the draft
count) and the review notes (the closed-form fold drifted on long outputs;
the exact fold restored parity).

Readings taken here:

* a row at cursor w (ring entries 0..w-1 committed) verifies T draft tokens
  as ring entries w..w+T-1, each formed exactly like a decode step of the
  GDN replay (pred, d, o from S0 and the entries before it); requires
  w + T <= L; the verify writes those entries (d, k, g, v, beta) but neither
  the state nor the cursor;
* commit with a accepted drafts (0 <= a <= T): w' = w + a; if w' + T > L (the
  next verify would not fit) or a flush is forced, the state is rebuilt by
  the recurrence over entries 0..w'-1 from their raw inputs,
      S <- g S;  d = beta (v - S k);  S <- S + outer(d, k),
  stored, and w' = 0 ("exact fold").
"""

import numpy as np

from .gdn import key_head
from .mamba2 import ST_BAD_SLOT, ST_RING_OVERFLOW
from .numerics import store


def gdn_spec_verify(state, d_ring, k_ring, g_ring, v_ring, beta_ring, slot_idx, write_pos,
                    q, k, v, g, beta, scale=None):
    """Verify T drafts per row; rings modified in place at entries w..w+T-1.

    q, k [batch, T, HK, K]; v [batch, T, HV, V]; g, beta [batch, T, HV].
    Returns (o [batch, T, HV, V] float64, status).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    nb, T, HV, V = v.shape
    K = k.shape[3]
    L = d_ring.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(K)
    kh = key_head(HV, k.shape[2])
    o = np.full((nb, T, HV, V), np.nan)
    status = 0
    for b in range(nb):
        s = int(slot_idx[b])
        w = int(write_pos[b])
        if s < 0 or s >= state.shape[0]:
            status |= ST_BAD_SLOT
            continue
        if w < 0 or w + T > L:
            status |= ST_RING_OVERFLOW
            continue
        S0 = state[s]                                        # [HV, V, K]
        for t in range(T):
            p = w + t                                        # this draft's ring entry
            kt, qt = k[b, t][kh], q[b, t][kh]                # [HV, K]
            ks = np.concatenate([k_ring[s][:, :p, :][kh], kt[:, None, :]], axis=1)
            gs = np.concatenate([g_ring[s, :, :p], g[b, t][:, None]], axis=1)
            gam = np.array([[np.prod(gs[h, i + 1:]) for i in range(p + 1)] for h in range(HV)])
            Gam = np.prod(gs, axis=1)
            ds_old = d_ring[s, :, :p, :]
            kdot = np.einsum("hik,hk->hi", ks[:, :p, :], kt)
            pred = (Gam[:, None] * np.matmul(S0, kt[:, :, None])[..., 0]
                    + np.einsum("hi,hiv->hv", gam[:, :p] * kdot, ds_old))
            dt = beta[b, t][:, None] * (v[b, t] - pred)
            ds = np.concatenate([ds_old, dt[:, None, :]], axis=1)
            qdot = np.einsum("hik,hk->hi", ks, qt)
            o[b, t] = scale * (Gam[:, None] * np.matmul(S0, qt[:, :, None])[..., 0]
                               + np.einsum("hi,hiv->hv", gam * qdot, ds))
            d_ring[s, :, p, :] = dt
            k_ring[s, :, p, :] = k[b, t]
            g_ring[s, :, p] = g[b, t]
            v_ring[s, :, p, :] = v[b, t]
            beta_ring[s, :, p] = beta[b, t]
    return o, status


def exact_fold(S0, k_ring, g_ring, v_ring, beta_ring, slot, n, kh):
    """The recurrence over ring entries 0..n-1 of one slot from their raw inputs."""
    S = S0.copy()
    for i in range(n):
        ki = k_ring[slot][:, i, :][kh]                       # [HV, K]
        S = g_ring[slot, :, i][:, None, None] * S
        pred = np.matmul(S, ki[:, :, None])[..., 0]
        d = beta_ring[slot, :, i][:, None] * (v_ring[slot, :, i, :] - pred)
        S = S + d[:, :, None] * ki[:, None, :]
    return S


def gdn_spec_commit(state, k_ring, g_ring, v_ring, beta_ring, slot_idx, write_pos, accepted, T,
                    force_flush=None, state_dtype="f64"):
    """Commit accepted drafts; exact fold when the next verify would not fit.

    Returns (next_write_pos int32 [batch], flushed uint8 [batch], status).
    """
    nb = len(slot_idx)
    L = g_ring.shape[2]
    HV = state.shape[1]
    kh = key_head(HV, k_ring.shape[1])
    nwp = np.zeros(nb, np.int32)
    flushed = np.zeros(nb, np.uint8)
    status = 0
    for b in range(nb):
        s = int(slot_idx[b])
        w = int(write_pos[b]) + int(accepted[b])
        if s < 0 or s >= state.shape[0]:
            status |= ST_BAD_SLOT
            continue
        if w > L or int(accepted[b]) < 0 or int(accepted[b]) > T:
            status |= ST_RING_OVERFLOW
            w = min(max(w, 0), L)
        force = force_flush is not None and bool(force_flush[b])
        if w + T > L or force:
            state[s] = store(exact_fold(state[s], k_ring, g_ring, v_ring, beta_ring, s, w, kh),
                             state_dtype)
            flushed[b] = 1
            w = 0
        nwp[b] = w
    return nwp, flushed, status
