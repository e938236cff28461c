"""Gated delta rule (GDN) decode: recurrence and ReplaySSM ring replay (float64).

Test infrastructure only; see the package docstring.

Sources:

* sglang #28451 (GDN/KDA ReplaySSM decode): Motivation - every GDN decode
  step reads and writes the full [HV, V, K] state; Implementation item 1 -
  non-flush steps rebuild the output from the checkpoint S0 plus the ring,
  and the full state is refreshed once every L steps; Risks - the extra ring
  memory per slot is d: HV*L*V, k: H*L*K and g.
* sglang #28695 "[GDN] Support ReplaySSM Ring Spec-Verify": memory-pool
  snippet - per slot the ring holds d [L, V], k [L, K] and the scalar gate g
  [L].

Recurrence (per row, value head hv, key head hk = hv // (HV // HK)):

    S <- g * S;  pred = S k;  S <- S + beta * outer(v - pred, k);
    o = scale * S q,   scale = 1 / sqrt(K)

S is [V, K] (the product S k contracts K).  Unrolled from a checkpoint S0
over ring entries 0..w (entry w = the current step), with
Gamma = prod_{j<=w} g_j and gamma_i = prod_{i<j<=w} g_j, every entry adds
gamma_i * outer(d_i, k_i), where d_i = beta_i * (v_i - pred_i) is the
delta the step wrote.  So

    pred_w = Gamma * (S0 k_w) + sum_{i<w} gamma_i * d_i * (k_i . k_w)
    d_w    = beta_w * (v_w - pred_w)
    o      = scale * [Gamma * (S0 q) + sum_{i<=w} gamma_i * d_i * (k_i . q)]
    flush:   S0 <- Gamma * S0 + sum_{i<=w} gamma_i * outer(d_i, k_i)

The ring stores (d, k, g).  Readings: g and beta arrive already activated;
q and k are used as given (the caller normalises them); status bits and the
flush rules are those of the Mamba2 replay.
"""

import numpy as np

from .numerics import store
from .mamba2 import ST_BAD_SLOT, ST_BAD_WRITE_POS, ST_RING_OVERFLOW


def key_head(HV, HK):
    if HK < 1 or HV % HK:
        raise ValueError("key heads must divide value heads")
    return np.arange(HV) // (HV // HK)


def gdn_standard_step(state, slot_idx, q, k, v, g, beta, scale=None,
                      state_dtype="f64"):
    """One recurrent gated-delta-rule step; state [slots, HV, V, K] in place.

    q, k [batch, HK, K]; v [batch, HV, V]; g, beta [batch, HV].
    Returns o [batch, HV, V] float64.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    nb, HV, V = v.shape
    K = k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(K)
    kh = key_head(HV, k.shape[1])
    kk = k[:, kh, :]                                    # [batch, HV, K]
    qq = q[:, kh, :]
    S = g[:, :, None, None] * state[slot_idx]           # [batch, HV, V, K]
    pred = np.matmul(S, kk[..., None])[..., 0]          # [batch, HV, V]
    S = S + (beta[:, :, None] * (v - pred))[..., None] * kk[:, :, None, :]
    o = scale * np.matmul(S, qq[..., None])[..., 0]
    state[slot_idx] = store(S, state_dtype)
    return o


def gdn_replay_step(state, d_ring, k_ring, g_ring, slot_idx, write_pos,
                    is_flush, q, k, v, g, beta, scale=None, state_dtype="f64"):
    """One GDN ReplaySSM decode step over a batch (rings modified in place).

    d_ring [slots, HV, L, V], k_ring [slots, HK, L, K], g_ring [slots, HV, L].
    Returns (o, next_write_pos, next_is_flush, status).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    nb, HV, V = v.shape
    K = k.shape[2]
    L = d_ring.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(K)
    kh = key_head(HV, k.shape[1])
    num_slots = state.shape[0]

    o = np.full((nb, HV, V), np.nan)
    nwp = np.zeros(nb, np.int32)
    status = 0
    for b in range(nb):
        s = int(slot_idx[b])
        w = int(write_pos[b])
        f = bool(is_flush[b])
        if s < 0 or s >= num_slots:
            status |= ST_BAD_SLOT
            continue
        if w < 0 or w >= L:
            status |= ST_BAD_WRITE_POS
            w = min(max(w, 0), L - 1)
            f = True
        if w == L - 1 and not f:
            status |= ST_RING_OVERFLOW
            f = True

        kw = k[b][kh]                                   # [HV, K]
        qw = q[b][kh]
        ks = np.concatenate([k_ring[s][:, :w, :][kh], kw[:, None, :]], axis=1)
        gs = np.concatenate([g_ring[s, :, :w], g[b][:, None]], axis=1)
        gamma = np.array([[np.prod(gs[h, i + 1:]) for i in range(w + 1)]
                          for h in range(HV)])          # [HV, w+1]
        Gam = np.prod(gs, axis=1)                       # [HV]
        S0 = state[s]                                   # [HV, V, K]
        ds_old = d_ring[s, :, :w, :]                    # [HV, w, V]

        kdot = np.einsum("hik,hk->hi", ks[:, :w, :], kw)
        pred = (Gam[:, None] * np.matmul(S0, kw[:, :, None])[..., 0]
                + np.einsum("hi,hiv->hv", gamma[:, :w] * kdot, ds_old))
        dw = beta[b][:, None] * (v[b] - pred)           # [HV, V]
        ds = np.concatenate([ds_old, dw[:, None, :]], axis=1)
        qdot = np.einsum("hik,hk->hi", ks, qw)
        ob = (Gam[:, None] * np.matmul(S0, qw[:, :, None])[..., 0]
              + np.einsum("hi,hiv->hv", gamma * qdot, ds))
        o[b] = scale * ob
        if f:
            S_new = (Gam[:, None, None] * S0
                     + np.einsum("hi,hiv,hik->hvk", gamma, ds, ks))
            state[s] = store(S_new, state_dtype)
            nwp[b] = 0
        else:
            d_ring[s, :, w, :] = dw
            g_ring[s, :, w] = g[b]
            k_ring[s, :, w, :] = k[b]
            nwp[b] = w + 1
    nfl = (nwp == L - 1).astype(np.uint8)
    return o, nwp, nfl, status


def gdn_replay_logical_state(state, d_ring, k_ring, g_ring, slot, write_pos):
    """The state S0 + ring represent for one slot (fold of entries 0..w-1)."""
    HV = state.shape[1]
    kh = key_head(HV, k_ring.shape[1])
    w = int(write_pos)
    S0 = state[slot]
    if w == 0:
        return S0.copy()
    ks = k_ring[slot][:, :w, :][kh]
    gs = g_ring[slot, :, :w]
    ds = d_ring[slot, :, :w, :]
    gamma = np.array([[np.prod(gs[h, i + 1:]) for i in range(w)]
                      for h in range(HV)])
    return (np.prod(gs, axis=1)[:, None, None] * S0
            + np.einsum("hi,hiv,hik->hvk", gamma, ds, ks))
