"""KDA (per-key-channel gated delta rule) decode: recurrence and ReplaySSM
ring replay (float64).

Test infrastructure only; see the package docstring.

Sources: sglang #28451 (GDN/KDA ReplaySSM decode) - Implementation item 1
(one decode kernel serves the GDN scalar gate and the KDA per-key-channel
gate, the ring length set by the cache-length option) and the review notes
(the KDA ring keeps a gate row per entry, g_cache [slots, HV, L, K], and the
per-step ring write is larger than GDN's).

Recurrence (per row, value head hv, key head hk = hv // (HV // HK); g is a
vector over the K key channels):

    S <- S diag(g);  pred = S k;  S <- S + beta * outer(v - pred, k);
    o = scale * S q

Unrolled from a checkpoint S0 over ring entries 0..w (entry w = the current
step), with Gamma = prod_{j<=w} g_j and gamma_i = prod_{i<j<=w} g_j taken
per channel, every entry adds outer(d_i, gamma_i * k_i):

    pred_w = S0 (Gamma * k_w) + sum_{i<w} d_i ((gamma_i * k_i) . k_w)
    o      = scale * [S0 (Gamma * q) + sum_{i<=w} d_i ((gamma_i * k_i) . q)]
    flush:   S0 <- S0 diag(Gamma) + sum_{i<=w} outer(d_i, gamma_i * k_i)

The ring stores (d, k, g) with g a [K] row.  Cursor, status and flush rules
are those of the GDN replay.
"""

import numpy as np

from .gdn import key_head
from .mamba2 import ST_BAD_SLOT, ST_BAD_WRITE_POS, ST_RING_OVERFLOW
from .numerics import store


def kda_standard_step(state, slot_idx, q, k, v, g, beta, scale=None, state_dtype="f64"):
    """One recurrent KDA step; state [slots, HV, V, K] in place.

    q, k [batch, HK, K]; v [batch, HV, V]; g [batch, HV, K]; beta [batch, HV].
    """
    q, k, v, g, beta = (np.asarray(a, np.float64) for a in (q, k, v, g, beta))
    nb, HV, V = v.shape
    K = k.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(K)
    kh = key_head(HV, k.shape[1])
    kk, qq = k[:, kh, :], q[:, kh, :]
    S = state[slot_idx] * g[:, :, None, :]               # columns scaled by g
    pred = np.matmul(S, kk[..., None])[..., 0]
    S = S + (beta[:, :, None] * (v - pred))[..., None] * kk[:, :, None, :]
    o = scale * np.matmul(S, qq[..., None])[..., 0]
    state[slot_idx] = store(S, state_dtype)
    return o


def kda_replay_step(state, d_ring, k_ring, g_ring, slot_idx, write_pos, is_flush, q, k, v, g,
                    beta, scale=None, state_dtype="f64"):
    """One KDA ReplaySSM decode step (rings modified in place).

    d_ring [slots, HV, L, V], k_ring [slots, HK, L, K], g_ring [slots, HV, L, K].
    Returns (o, next_write_pos, next_is_flush, status).
    """
    q, k, v, g, beta = (np.asarray(a, np.float64) for a in (q, k, v, g, beta))
    nb, HV, V = v.shape
    K = k.shape[2]
    L = d_ring.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(K)
    kh = key_head(HV, k.shape[1])
    o = np.full((nb, HV, V), np.nan)
    nwp = np.zeros(nb, np.int32)
    status = 0
    for b in range(nb):
        s, w, f = int(slot_idx[b]), int(write_pos[b]), bool(is_flush[b])
        if s < 0 or s >= state.shape[0]:
            status |= ST_BAD_SLOT
            continue
        if w < 0 or w >= L:
            status |= ST_BAD_WRITE_POS
            w = min(max(w, 0), L - 1)
            f = True
        if w == L - 1 and not f:
            status |= ST_RING_OVERFLOW
            f = True
        kw, qw = k[b][kh], q[b][kh]                          # [HV, K]
        ks = np.concatenate([k_ring[s][:, :w, :][kh], kw[:, None, :]], axis=1)   # [HV, w+1, K]
        gs = np.concatenate([g_ring[s, :, :w, :], g[b][:, None, :]], axis=1)     # [HV, w+1, K]
        gam = np.stack([np.prod(gs[:, i + 1:, :], axis=1) for i in range(w + 1)], axis=1)
        Gam = np.prod(gs, axis=1)                            # [HV, K]
        kt = gam * ks                                        # gamma_i * k_i
        S0 = state[s]
        ds_old = d_ring[s, :, :w, :]
        pred = (np.matmul(S0, (Gam * kw)[:, :, None])[..., 0]
                + np.einsum("hi,hiv->hv", np.einsum("hik,hk->hi", kt[:, :w], kw), ds_old))
        dw = beta[b][:, None] * (v[b] - pred)
        ds = np.concatenate([ds_old, dw[:, None, :]], axis=1)
        o[b] = scale * (np.matmul(S0, (Gam * qw)[:, :, None])[..., 0]
                        + np.einsum("hi,hiv->hv", np.einsum("hik,hk->hi", kt, qw), ds))
        if f:
            S_new = S0 * Gam[:, None, :] + np.einsum("hiv,hik->hvk", ds, kt)
            state[s] = store(S_new, state_dtype)
            nwp[b] = 0
        else:
            d_ring[s, :, w, :] = dw
            g_ring[s, :, w, :] = g[b]
            k_ring[s, :, w, :] = k[b]
            nwp[b] = w + 1
    nfl = (nwp == L - 1).astype(np.uint8)
    return o, nwp, nfl, status


def kda_replay_logical_state(state, d_ring, k_ring, g_ring, slot, write_pos):
    """The state S0 + ring represent for one slot (fold of entries 0..w-1)."""
    HV = state.shape[1]
    kh = key_head(HV, k_ring.shape[1])
    w = int(write_pos)
    S0 = state[slot]
    if w == 0:
        return S0.copy()
    ks = k_ring[slot][:, :w, :][kh]
    gs = g_ring[slot, :, :w, :]
    gam = np.stack([np.prod(gs[:, i + 1:, :], axis=1) for i in range(w)], axis=1)
    return (S0 * np.prod(gs, axis=1)[:, None, :]
            + np.einsum("hiv,hik->hvk", d_ring[slot, :, :w, :], gam * ks))
