"""GDN speculative verify and commit on the GPU against the float64 oracle:
rounds of verify -> random acceptance -> commit (with exact folds whenever the
next verify would not fit, and forced folds), checking every draft output,
every cursor and every folded state; and the deferred-fold rounds (verify
with flush -> random acceptance -> advance) against the oracle's rounds on
the same inputs."""

import numpy as np
import pytest
import torch

import linear_recurrence_amd as R
from oracle import gdn_spec as OS

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")


def _unit(rng, shape):
    a = rng.normal(size=shape)
    return a / np.linalg.norm(a, axis=-1, keepdims=True)


def run_spec(nb, HK, HV, K, V, L, T, io, rounds, sample, seed, out=torch.float32, offset=0,
             gates=None, force_p=0.1):
    """offset > 0 places the cursors and accepted counts `offset` int32s off
    a 16-byte boundary.  gates(rng, shape) draws the decays g (default:
    exp(-softplus(N(0, 1)))).  force_p: the chance that a row's commit is
    forced to fold."""
    print(f"case: spec nb={nb} HK={HK} HV={HV} K={K} V={V} L={L} T={T} io={io} "
          f"offset={offset}", flush=True)
    rng = np.random.default_rng(seed)
    dev = torch.device("cuda:0")
    ns = nb + 3
    slots = rng.permutation(ns)[:nb].astype(np.int32)
    pool = rng.normal(0, 0.1, (ns, HV, V, K)).astype(np.float32)
    st = torch.tensor(pool, device=dev)
    dr = torch.full((ns, HV, L, V), float("nan"), device=dev)
    kr = torch.full((ns, HK, L, K), float("nan"), dtype=io, device=dev)
    gr = torch.full((ns, HV, L), float("nan"), device=dev)
    vr = torch.full((ns, HV, L, V), float("nan"), dtype=io, device=dev)
    br = torch.full((ns, HV, L), float("nan"), device=dev)
    wp = torch.zeros(nb + offset, dtype=torch.int32, device=dev)[offset:]
    nwp = torch.zeros(nb + offset, dtype=torch.int32, device=dev)[offset:]
    acc_buf = torch.zeros(nb + offset, dtype=torch.int32, device=dev)
    fl = torch.empty(nb, dtype=torch.uint8, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    sl = torch.tensor(slots, device=dev)
    sample = sorted(set(sample))
    k_ = len(sample)
    o_pool = pool[slots[sample]].astype(np.float64)
    o_rings = [np.full((k_, HV, L, V), np.nan), np.full((k_, HK, L, K), np.nan),
               np.full((k_, HV, L), np.nan), np.full((k_, HV, L, V), np.nan),
               np.full((k_, HV, L), np.nan)]
    o_sl = np.arange(k_)
    o_wp = np.zeros(k_, np.int32)
    fp32 = io == torch.float32
    folds = 0
    for r in range(rounds):
        q = torch.tensor(_unit(rng, (nb, T, HK, K)), dtype=io, device=dev)
        k = torch.tensor(_unit(rng, (nb, T, HK, K)), dtype=io, device=dev)
        v = torch.tensor(rng.normal(size=(nb, T, HV, V)), dtype=io, device=dev)
        gv = (gates(rng, (nb, T, HV)) if gates else
              np.exp(-np.log1p(np.exp(rng.normal(size=(nb, T, HV))))))
        g = torch.tensor(gv, dtype=torch.float32, device=dev)
        beta = torch.tensor(1 / (1 + np.exp(-rng.normal(size=(nb, T, HV)))),
                            dtype=torch.float32, device=dev)
        o = R.replayssm_gdn_spec_verify(st, dr, kr, gr, vr, br, sl, wp, q, k, v, g, beta,
                                        status=status, out_dtype=out)
        npv = lambda t: t[sample].double().cpu().numpy()
        o_ref, ost = OS.gdn_spec_verify(o_pool, *o_rings, o_sl, o_wp, npv(q), npv(k), npv(v),
                                        npv(g), npv(beta))
        assert ost == 0
        got = o[sample].double().cpu().numpy()
        d = np.abs(got - o_ref)
        if fp32 and out == torch.float32:
            err = d.max() / np.abs(o_ref).max()
            assert err <= 2e-5, f"round {r}: o error {err:.2e}"
        else:
            bound = np.maximum(1e-2, np.abs(o_ref) * 2**-7)
            assert (d <= bound).all(), f"round {r}: o error {d.max():.2e}"
        acc = rng.integers(0, T + 1, nb).astype(np.int32)
        force = (rng.random(nb) < force_p).astype(np.uint8)
        acc_t = acc_buf[offset:]
        acc_t.copy_(torch.tensor(acc, device=dev))
        R.replayssm_gdn_spec_commit(st, kr, gr, vr, br, sl, wp, acc_t,
                                    T, nwp, force_flush=torch.tensor(force, device=dev),
                                    flushed=fl, status=status)
        o_wp, o_fl, ost = OS.gdn_spec_commit(o_pool, *o_rings[1:], o_sl, o_wp, acc[sample], T,
                                             force_flush=force[sample], state_dtype="f32")
        assert ost == 0
        # cursors of every row follow the commit rule
        w_all = wp.cpu().numpy() + acc
        fl_ref = ((w_all + T > L) | (force != 0)).astype(np.uint8)
        np.testing.assert_array_equal(fl.cpu().numpy(), fl_ref)
        np.testing.assert_array_equal(nwp.cpu().numpy(), np.where(fl_ref, 0, w_all))
        np.testing.assert_array_equal(nwp.cpu().numpy()[sample], o_wp)
        for j, row in enumerate(sample):
            if o_fl[j]:
                folds += 1
                gs = st[int(slots[row])].double().cpu().numpy()
                e = np.abs(gs - o_pool[j]).max()
                lim = 2e-5 * np.abs(o_pool[j]).max() if fp32 else 1e-2
                assert e <= lim, f"round {r} row {row}: folded state error {e:.2e}"
        wp, nwp = nwp, wp
    torch.cuda.synchronize()
    assert status.item() == 0
    assert folds > 0


@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("K,V", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_spec_small(io, K, V):
    run_spec(5, 2, 4, K, V, 8, 3, io, 14, range(5), seed=K + V + (io == torch.bfloat16))


@pytest.mark.parametrize("L,T", [(2, 1), (16, 8), (64, 8), (20, 5)])
def test_spec_ring_lengths(L, T):
    run_spec(3, 1, 2, 128, 128, L, T, torch.bfloat16, max(6, 3 * L // T), range(3), seed=L * 7 + T)


def test_spec_full_size_bf16_output():
    """256 rows, 16 key / 32 value heads, K = V = 128, L = 16, 4 drafts."""
    run_spec(256, 16, 32, 128, 128, 16, 4, torch.bfloat16, 12, [0, 99, 200, 255], seed=4,
             out=torch.bfloat16)


def _extreme_gates(rng, shape):
    """Decays that drive the fold's running decay product out of its lazy
    range within a few entries: zeros, 1e-9, 1e-30 and ones among the usual
    draws."""
    g = np.exp(-np.log1p(np.exp(rng.normal(size=shape))))
    pick = rng.random(shape)
    g = np.where(pick < 0.1, 0.0, g)
    g = np.where((pick >= 0.1) & (pick < 0.2), 1e-9, g)
    g = np.where((pick >= 0.2) & (pick < 0.25), 1e-30, g)
    return np.where((pick >= 0.25) & (pick < 0.35), 1.0, g)


@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16])
def test_spec_fold_with_extreme_decays(io):
    """Decays of 0, 1e-9 and 1e-30 (and 1) in the folded entries, long rings
    (L = 64 with bf16 inputs, 48 with fp32, whose verify staging would not
    fit one workgroup's LDS at 64) and L = 16: the fold keeps the decay of
    the tile as one running product and applies it to the state whenever
    that product leaves [2^-60, 2^60]."""
    L = 64 if io == torch.bfloat16 else 48
    run_spec(6, 2, 4, 128, 128, L, 8, io, 24, range(6), seed=95, gates=_extreme_gates)
    run_spec(6, 1, 2, 64, 128, 16, 4, io, 16, range(6), seed=96, gates=_extreme_gates)


def test_spec_commit_every_row_folds():
    """Every commit forced: all 256 x 32 (row, value head) tiles fold each
    round, eight fold tasks per workgroup of the commit's 1024-workgroup
    grid."""
    run_spec(256, 16, 32, 128, 128, 16, 4, torch.bfloat16, 4, [0, 77, 200, 255], seed=97,
             force_p=1.0)


def test_spec_commit_large_batch_and_unaligned_cursors():
    """A batch over 512 rows takes the commit's grid of one workgroup per
    (row, value head); cursors and accepted counts off a 16-byte boundary
    (the task-list commit reads them element by element)."""
    run_spec(520, 1, 2, 64, 64, 8, 3, torch.bfloat16, 8, [0, 255, 300, 519], seed=91)
    run_spec(40, 2, 4, 128, 128, 16, 4, torch.bfloat16, 10, range(0, 40, 7), seed=92, offset=1)


def run_spec_deferred(nb, HK, HV, K, V, L, T, io, rounds, sample, seed, out=torch.float32,
                      gates=None, force_p=0.1, drain=False):
    """Deferred-fold rounds (verify with flush, then advance) on the GPU
    against the oracle's eager rounds (verify, then commit with its fold) on
    the same inputs: the drafts' outputs agree every round; a row's fold,
    done by the GPU at its next verify, leaves the state the oracle's commit
    left; the cursors follow the advance rule and agree with the oracle's
    (w' where the oracle kept it, 0 where it folded); a folded row's new
    k rows land at its ring entries 0..T-1; at the end every sampled row's
    checkpoint folded with its ring equals the oracle's.  drain: then fold
    every row's ring at once by the eager commit (no accepted drafts,
    forced) and compare the stored states."""
    print(f"case: deferred spec nb={nb} HK={HK} HV={HV} K={K} V={V} L={L} T={T} io={io}",
          flush=True)
    rng = np.random.default_rng(seed)
    dev = torch.device("cuda:0")
    ns = nb + 3
    slots = rng.permutation(ns)[:nb].astype(np.int32)
    pool = rng.normal(0, 0.1, (ns, HV, V, K)).astype(np.float32)
    st = torch.tensor(pool, device=dev)
    dr = torch.full((ns, HV, L, V), float("nan"), device=dev)
    kr = torch.full((ns, HK, L, K), float("nan"), dtype=io, device=dev)
    gr = torch.full((ns, HV, L), float("nan"), device=dev)
    vr = torch.full((ns, HV, L, V), float("nan"), dtype=io, device=dev)
    br = torch.full((ns, HV, L), float("nan"), device=dev)
    wp = torch.zeros(nb, dtype=torch.int32, device=dev)
    nwp = torch.zeros(nb, dtype=torch.int32, device=dev)
    fl = torch.zeros(nb, dtype=torch.uint8, device=dev)
    nfl = torch.zeros(nb, dtype=torch.uint8, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    sl = torch.tensor(slots, device=dev)
    sample = sorted(set(sample))
    k_ = len(sample)
    o_pool = pool[slots[sample]].astype(np.float64)
    o_rings = [np.full((k_, HV, L, V), np.nan), np.full((k_, HK, L, K), np.nan),
               np.full((k_, HV, L), np.nan), np.full((k_, HV, L, V), np.nan),
               np.full((k_, HV, L), np.nan)]
    o_sl = np.arange(k_)
    o_wp = np.zeros(k_, np.int32)
    fp32 = io == torch.float32
    lim = (lambda ref: 2e-5 * np.abs(ref).max()) if fp32 else (lambda ref: 1e-2)
    folds = 0
    for r in range(rounds):
        q = torch.tensor(_unit(rng, (nb, T, HK, K)), dtype=io, device=dev)
        k = torch.tensor(_unit(rng, (nb, T, HK, K)), dtype=io, device=dev)
        v = torch.tensor(rng.normal(size=(nb, T, HV, V)), dtype=io, device=dev)
        gv = (gates(rng, (nb, T, HV)) if gates else
              np.exp(-np.log1p(np.exp(rng.normal(size=(nb, T, HV))))))
        g = torch.tensor(gv, dtype=torch.float32, device=dev)
        beta = torch.tensor(1 / (1 + np.exp(-rng.normal(size=(nb, T, HV)))),
                            dtype=torch.float32, device=dev)
        fl_now = fl.cpu().numpy().astype(bool)
        wp_now = wp.cpu().numpy()
        o = R.replayssm_gdn_spec_verify_flush(st, dr, kr, gr, vr, br, sl, wp, fl, q, k, v, g,
                                              beta, status=status, out_dtype=out)
        # a folding row's stored state is the oracle's state after its last commit
        for j, row in enumerate(sample):
            if fl_now[row] and wp_now[row] > 0:
                folds += 1
                gs = st[int(slots[row])].double().cpu().numpy()
                e = np.abs(gs - o_pool[j]).max()
                assert e <= lim(o_pool[j]), f"round {r} row {row}: folded state error {e:.2e}"
        npv = lambda t: t[sample].double().cpu().numpy()
        o_ref, ost = OS.gdn_spec_verify(o_pool, *o_rings, o_sl, o_wp, npv(q), npv(k), npv(v),
                                        npv(g), npv(beta))
        assert ost == 0
        got = o[sample].double().cpu().numpy()
        d = np.abs(got - o_ref)
        if fp32 and out == torch.float32:
            err = d.max() / np.abs(o_ref).max()
            assert err <= 2e-5, f"round {r}: o error {err:.2e}"
        else:
            bound = np.maximum(1e-2, np.abs(o_ref) * 2**-7)
            assert (d <= bound).all(), f"round {r}: o error {d.max():.2e}"
        acc = rng.integers(0, T + 1, nb).astype(np.int32)
        force = (rng.random(nb) < force_p).astype(np.uint8)
        R.replayssm_gdn_spec_advance(kr, gr, vr, br, sl, wp, fl, torch.tensor(acc, device=dev),
                                     T, k, v, g, beta, nwp, nfl,
                                     force_flush=torch.tensor(force, device=dev), status=status)
        o_wp, o_fl, ost = OS.gdn_spec_commit(o_pool, *o_rings[1:], o_sl, o_wp, acc[sample], T,
                                             force_flush=force[sample], state_dtype="f32")
        assert ost == 0
        w_all = np.where(fl_now, 0, wp_now) + acc
        nfl_ref = ((w_all + T > L) | (force != 0)).astype(np.uint8)
        np.testing.assert_array_equal(nwp.cpu().numpy(), w_all)
        np.testing.assert_array_equal(nfl.cpu().numpy(), nfl_ref)
        np.testing.assert_array_equal(o_fl, nfl_ref[sample])
        np.testing.assert_array_equal(o_wp, np.where(nfl_ref, 0, w_all)[sample])
        # the kept drafts' k, v, g and beta rows, written by the advance at
        # entries w..w'-1 (bit copies of the inputs)
        bits = (lambda t: t.view(torch.int16)) if io == torch.bfloat16 else (lambda t: t)
        krs, vrs, grs, brs = kr.cpu(), vr.cpu(), gr.cpu(), br.cpu()
        kc, vc, gc, bc = k.cpu(), v.cpu(), g.cpu(), beta.cpu()
        w_eff = np.where(fl_now, 0, wp_now)
        for row in range(nb):
            s_, a_, w_ = int(slots[row]), int(acc[row]), int(w_eff[row])
            if a_ == 0:
                continue
            assert torch.equal(bits(krs[s_, :, w_:w_ + a_, :]),
                               bits(kc[row, :a_].permute(1, 0, 2).contiguous()))
            assert torch.equal(bits(vrs[s_, :, w_:w_ + a_, :]),
                               bits(vc[row, :a_].permute(1, 0, 2).contiguous()))
            assert torch.equal(grs[s_, :, w_:w_ + a_], gc[row, :a_].t())
            assert torch.equal(brs[s_, :, w_:w_ + a_], bc[row, :a_].t())
        wp, nwp = nwp, wp
        fl, nfl = nfl, fl
    torch.cuda.synchronize()
    assert status.item() == 0
    assert folds > 0
    # end: each sampled row's logical state (checkpoint folded with its ring)
    rings = [t.double().cpu().numpy() for t in (kr, gr, vr, br)]
    wpe = wp.cpu().numpy()
    kh = np.arange(HV) // (HV // HK)
    for j, row in enumerate(sample):
        s = int(slots[row])
        got = OS.exact_fold(st[s].double().cpu().numpy(), *rings, s, int(wpe[row]), kh)
        ref = OS.exact_fold(o_pool[j], o_rings[1], o_rings[2], o_rings[3], o_rings[4], j,
                            int(o_wp[j]), kh)
        e = np.abs(got - ref).max()
        assert e <= lim(ref), f"row {row}: end state error {e:.2e}"
        if drain:
            o_pool[j] = ref
    if drain:
        zero = torch.zeros(nb, dtype=torch.int32, device=dev)
        ones = torch.ones(nb, dtype=torch.uint8, device=dev)
        R.replayssm_gdn_spec_commit(st, kr, gr, vr, br, sl, wp, zero, T, nwp, force_flush=ones,
                                    status=status)
        torch.cuda.synchronize()
        assert status.item() == 0
        assert (nwp.cpu().numpy() == 0).all()
        for j, row in enumerate(sample):
            got = st[int(slots[row])].double().cpu().numpy()
            e = np.abs(got - o_pool[j]).max()
            assert e <= lim(o_pool[j]), f"row {row}: drained state error {e:.2e}"


@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("K,V", [(128, 128), (64, 64), (64, 128), (128, 64)])
def test_spec_deferred_small(io, K, V):
    run_spec_deferred(5, 2, 4, K, V, 8, 3, io, 14, range(5), seed=K + V + 7)


@pytest.mark.parametrize("L,T,io", [(2, 1, torch.bfloat16), (16, 8, torch.bfloat16),
                                    (20, 5, torch.bfloat16), (35, 8, torch.bfloat16),
                                    (42, 8, torch.bfloat16), (46, 4, torch.bfloat16),
                                    (24, 8, torch.float32), (27, 4, torch.float32)])
def test_spec_deferred_ring_lengths(L, T, io):
    """Up to the longest rings whose raw rows fit beside the verify's staging
    (42 / 46 entries with bf16 inputs, 24 / 27 with fp32; 35 is the longest
    on the matrix-core path at 8 drafts)."""
    run_spec_deferred(3, 1, 2, 128, 128, L, T, io, max(6, 3 * L // T), range(3), seed=L * 5 + T)


def test_spec_deferred_full_size_bf16_output():
    """256 rows, 16 key / 32 value heads, K = V = 128, L = 16, 4 drafts; at
    the end every ring is folded at once by the eager commit."""
    run_spec_deferred(256, 16, 32, 128, 128, 16, 4, torch.bfloat16, 12, [0, 99, 200, 255],
                      seed=14, out=torch.bfloat16, drain=True)


def test_spec_deferred_many_heads():
    """64 value heads and 8 drafts: the advance copies its kept drafts' rows
    in several batches of vectors and of gates per row."""
    run_spec_deferred(8, 16, 64, 128, 128, 16, 8, torch.bfloat16, 8, range(8), seed=94)


def test_spec_deferred_large_batch():
    """520 rows (one advance workgroup per row; the verify's grid in batch
    order), fp32 inputs, drained at the end."""
    run_spec_deferred(520, 1, 2, 64, 64, 8, 3, torch.float32, 8, [0, 255, 300, 519], seed=93,
                      drain=True)


@pytest.mark.parametrize("io", [torch.float32, torch.bfloat16])
def test_spec_deferred_fold_with_extreme_decays(io):
    L = 32 if io == torch.bfloat16 else 24
    run_spec_deferred(6, 2, 4, 128, 128, L, 8, io, 20, range(6), seed=195, gates=_extreme_gates)
    run_spec_deferred(6, 1, 2, 64, 128, 16, 4, io, 16, range(6), seed=196, gates=_extreme_gates)


def test_spec_deferred_every_row_folds():
    """Every advance forced: every row folds in every verify."""
    run_spec_deferred(256, 16, 32, 128, 128, 16, 4, torch.bfloat16, 4, [0, 77, 200, 255],
                      seed=197, force_p=1.0)


def test_spec_deferred_too_long_ring_is_refused():
    print("case: deferred spec ring too long", flush=True)
    dev = torch.device("cuda:0")
    HK, HV, K, V, L, T = 1, 2, 128, 128, 47, 4
    st = torch.zeros((2, HV, V, K), device=dev)
    rings = (torch.zeros((2, HV, L, V), device=dev),
             torch.zeros((2, HK, L, K), dtype=torch.bfloat16, device=dev),
             torch.zeros((2, HV, L), device=dev),
             torch.zeros((2, HV, L, V), dtype=torch.bfloat16, device=dev),
             torch.zeros((2, HV, L), device=dev))
    sl = torch.tensor([0, 1], dtype=torch.int32, device=dev)
    wp = torch.zeros(2, dtype=torch.int32, device=dev)
    fl = torch.zeros(2, dtype=torch.uint8, device=dev)
    q = torch.ones((2, T, HK, K), dtype=torch.bfloat16, device=dev)
    v = torch.ones((2, T, HV, V), dtype=torch.bfloat16, device=dev)
    gb = torch.full((2, T, HV), 0.5, device=dev)
    with pytest.raises(R.RssmError):
        R.replayssm_gdn_spec_verify_flush(st, *rings, sl, wp, fl, q, q, v, gb, gb)
    # the verify without folds still takes it
    R.replayssm_gdn_spec_verify(st, *rings, sl, wp, q, q, v, gb, gb)
    torch.cuda.synchronize()


def test_spec_deferred_bad_cursor_is_refused():
    """A folding row past the ring (w > L) and an other row whose drafts do
    not fit (w + T > L) are refused with the status bit and NaN outputs;
    the good rows are verified.  The advance with accepted counts out of
    range sets the status bit, clamps the cursor to the ring and copies at
    most the T drafts."""
    print("case: deferred spec bad cursors", flush=True)
    dev = torch.device("cuda:0")
    HK, HV, K, V, L, T = 1, 2, 64, 64, 8, 4
    st = torch.zeros((4, HV, V, K), device=dev)
    rings = tuple(torch.zeros(sh, device=dev) for sh in
                  ((4, HV, L, V), (4, HK, L, K), (4, HV, L), (4, HV, L, V), (4, HV, L)))
    sl = torch.tensor([0, 1, 2, 3], dtype=torch.int32, device=dev)
    wp = torch.tensor([0, 9, 5, 8], dtype=torch.int32, device=dev)
    fl = torch.tensor([0, 1, 0, 1], dtype=torch.uint8, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    q = torch.ones((4, T, HK, K), device=dev) / 8
    v = torch.ones((4, T, HV, V), device=dev)
    gb = torch.full((4, T, HV), 0.5, device=dev)
    o = R.replayssm_gdn_spec_verify_flush(st, *rings, sl, wp, fl, q, q, v, gb, gb,
                                          status=status)
    torch.cuda.synchronize()
    assert status.item() & R.ST_RING_OVERFLOW
    assert torch.isnan(o[1]).all() and torch.isnan(o[2]).all()
    assert torch.isfinite(o[0]).all() and torch.isfinite(o[3]).all()
    # accepted counts out of range: the status bit, the cursor clamped to the
    # ring, at most T kept drafts copied
    status.zero_()
    wp2 = torch.tensor([0, 6, 2, 0], dtype=torch.int32, device=dev)
    fl2 = torch.zeros(4, dtype=torch.uint8, device=dev)
    acc = torch.tensor([T + 1, 4, -1, 2], dtype=torch.int32, device=dev)
    nwp = torch.empty(4, dtype=torch.int32, device=dev)
    nfl = torch.empty(4, dtype=torch.uint8, device=dev)
    kr, gr, vr, br = rings[1], rings[2], rings[3], rings[4]
    R.replayssm_gdn_spec_advance(kr, gr, vr, br, sl, wp2, fl2, acc, T, q, v, gb, gb, nwp, nfl,
                                 status=status)
    torch.cuda.synchronize()
    assert status.item() & R.ST_RING_OVERFLOW
    assert nwp.cpu().tolist() == [T + 1, 8, 1, 2]
    assert nfl.cpu().tolist() == [1, 1, 0, 0]
    assert torch.equal(kr[0, 0, :T], q[0, :, 0]) and (kr[0, 0, T:] == 0).all()


def test_spec_bad_cursor_is_refused():
    print("case: spec bad cursor", flush=True)
    dev = torch.device("cuda:0")
    HK, HV, K, V, L, T = 1, 2, 64, 64, 8, 4
    st = torch.zeros((2, HV, V, K), device=dev)
    rings = (torch.zeros((2, HV, L, V), device=dev), torch.zeros((2, HK, L, K), device=dev),
             torch.zeros((2, HV, L), device=dev), torch.zeros((2, HV, L, V), device=dev),
             torch.zeros((2, HV, L), device=dev))
    sl = torch.tensor([0, 1], dtype=torch.int32, device=dev)
    wp = torch.tensor([0, 5], dtype=torch.int32, device=dev)   # row 1: 5 + 4 > 8
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    q = torch.ones((2, T, HK, K), device=dev) / 8
    v = torch.ones((2, T, HV, V), device=dev)
    gb = torch.full((2, T, HV), 0.5, device=dev)
    o = R.replayssm_gdn_spec_verify(st, *rings, sl, wp, q, q, v, gb, gb, status=status)
    torch.cuda.synchronize()
    assert status.item() & R.ST_RING_OVERFLOW
    assert torch.isnan(o[1]).all() and torch.isfinite(o[0]).all()
