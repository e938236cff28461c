"""Decode steps inside HIP graphs: K steps captured once, the graph replayed
several times with unrelated eager GPU work and synchronisations between
the replays, and every replay's outputs, cursors, rings and state equal, bit
for bit, to the same steps launched one by one on an identical copy.  A
serving loop submits its decode steps this way; the entry points only
launch kernels on the caller's stream (no allocation, fill or
synchronisation), which is what stream capture needs.  The cursor buffers
ping-pong every step, so K is even and a replay leaves them where the
capture found them."""

import dataclasses

import pytest
import torch

import linear_recurrence_amd as R
from workloads import TINY, TORCH_DTYPES, GdnInputs, GdnWorkload, Mamba2Inputs

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    R.load()


def _side_work(dev):
    a = torch.randn(512, 512, device=dev)
    (a @ a).sum().item()


def _same(a, b):
    """Bit-for-bit equal, NaN where the other has NaN (unused pool slots)."""
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    elif a.is_floating_point():
        a, b = a.view(torch.int32), b.view(torch.int32)
    return torch.equal(a, b)


def _check_replays(eager_step, graph_step, k_steps, snapshot, dev):
    """Run R x K eager steps (reference snapshots after each K), then capture
    K graph steps and compare each replay with its reference."""
    refs = []
    for _ in range(REPLAYS):
        for k in range(k_steps):
            eager_step(k)
        torch.cuda.synchronize()
        refs.append(snapshot("eager"))
    # the steps change the state: a replay that did nothing could not match
    assert not _same(refs[0]["state"], refs[1]["state"])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for k in range(k_steps):
            graph_step(k)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        g.replay()
        torch.cuda.synchronize()
        got = snapshot("graph")
        for name, ref in refs[r].items():
            assert _same(got[name], ref), f"replay {r}: {name} differs"
        _side_work(dev)
    del g


def test_mamba2_replay_in_a_graph():
    wl = dataclasses.replace(TINY, name="graph_tiny", desync=True)
    gen = Mamba2Inputs(wl)
    dev = torch.device("cuda:0")
    print("case: mamba2 replay, 8 steps per graph", flush=True)
    H, P, N, G, L, ns, nb = (wl.nheads, wl.headdim, wl.dstate, wl.ngroups, wl.ring_len,
                             wl.num_slots, wl.batch)
    io = TORCH_DTYPES[wl.io_dtype]
    prm = {k: v.to(dev) for k, v in gen.params().items()}
    k_steps = 8
    inps = [{k: v.to(dev) for k, v in gen.step(t).items()} for t in range(k_steps)]
    w0 = gen.start_positions()

    def layer():
        return {"state": gen.state_pool().to(dev),
                "xr": torch.zeros((ns, H, L, P), dtype=io, device=dev),
                "dr": torch.zeros((ns, H, L), device=dev),
                "br": torch.zeros((ns, G, L, N), dtype=io, device=dev),
                "wp": w0.to(dev), "fl": (w0 == L - 1).to(torch.uint8).to(dev),
                "nwp": torch.zeros(nb, dtype=torch.int32, device=dev),
                "nfl": torch.zeros(nb, dtype=torch.uint8, device=dev),
                "y": [torch.empty((nb, H, P), dtype=io, device=dev) for _ in range(k_steps)]}

    slots = gen.slot_idx().to(dev)
    lay = {"eager": layer(), "graph": layer()}

    def step(d, k):
        x = inps[k]
        R.replayssm_decode(d["state"], d["xr"], d["dr"], d["br"], slots, d["wp"], d["fl"],
                           x["x"], x["dt"], prm["A"], x["B"], x["C"], D=prm["D"], z=x["z"],
                           dt_bias=prm["dt_bias"], y=d["y"][k], next_write_pos=d["nwp"],
                           next_is_flush=d["nfl"])
        d["wp"], d["nwp"] = d["nwp"], d["wp"]
        d["fl"], d["nfl"] = d["nfl"], d["fl"]

    def snapshot(which):
        d = lay[which]
        out = {f"y{k}": d["y"][k].clone() for k in range(k_steps)}
        out.update(state=d["state"].clone(), wp=d["wp"].clone(), fl=d["fl"].clone(),
                   xr=d["xr"].clone(), dr=d["dr"].clone(), br=d["br"].clone())
        return out

    _check_replays(lambda k: step(lay["eager"], k), lambda k: step(lay["graph"], k), k_steps,
                   snapshot, dev)


def test_gdn_replay_decode_in_a_graph():
    wl = GdnWorkload("graph_gdn", 4, 2, 4, 64, 64, 8, 16, 8, "bf16", "f32", 4400, desync=True)
    gen = GdnInputs(wl)
    dev = torch.device("cuda:0")
    print("case: gdn replay decode, 16 steps per graph", flush=True)
    HK, HV, K, V, L, ns, nb = (wl.k_heads, wl.v_heads, wl.dk, wl.dv, wl.ring_len, wl.num_slots,
                               wl.batch)
    io = TORCH_DTYPES[wl.io_dtype]
    k_steps = 16
    inps = [{k: v.to(dev) for k, v in gen.step(t).items()} for t in range(k_steps)]
    w0 = gen.start_positions()

    def layer():
        return {"state": gen.state_pool().to(dev),
                "dr": torch.zeros((ns, HV, L, V), device=dev),
                "kr": torch.zeros((ns, HK, L, K), dtype=io, device=dev),
                "gr": torch.zeros((ns, HV, L), device=dev),
                "wp": w0.to(dev), "fl": (w0 == L - 1).to(torch.uint8).to(dev),
                "nwp": torch.zeros(nb, dtype=torch.int32, device=dev),
                "nfl": torch.zeros(nb, dtype=torch.uint8, device=dev),
                "o": [torch.empty((nb, HV, V), dtype=io, device=dev) for _ in range(k_steps)]}

    slots = gen.slot_idx().to(dev)
    lay = {"eager": layer(), "graph": layer()}

    def step(d, k):
        x = inps[k]
        R.replayssm_gdn_decode(d["state"], d["dr"], d["kr"], d["gr"], slots, d["wp"], d["fl"],
                               x["q"], x["k"], x["v"], x["g"], x["beta"], o=d["o"][k],
                               next_write_pos=d["nwp"], next_is_flush=d["nfl"])
        d["wp"], d["nwp"] = d["nwp"], d["wp"]
        d["fl"], d["nfl"] = d["nfl"], d["fl"]

    def snapshot(which):
        d = lay[which]
        out = {f"o{k}": d["o"][k].clone() for k in range(k_steps)}
        out.update(state=d["state"].clone(), wp=d["wp"].clone(), fl=d["fl"].clone(),
                   dr=d["dr"].clone(), kr=d["kr"].clone(), gr=d["gr"].clone())
        return out

    _check_replays(lambda k: step(lay["eager"], k), lambda k: step(lay["graph"], k), k_steps,
                   snapshot, dev)


def test_gdn_spec_rounds_in_a_graph():
    """Verify + commit rounds (4 drafts, L = 16, accepted counts fixed per
    round on the device, some forced folds), 4 rounds per graph."""
    wl = GdnWorkload("graph_spec", 8, 2, 4, 128, 128, 16, 4, 12, "bf16", "f32", 4500)
    gen = GdnInputs(wl)
    dev = torch.device("cuda:0")
    print("case: gdn spec rounds, 4 rounds per graph", flush=True)
    HK, HV, K, V, L, ns, nb = (wl.k_heads, wl.v_heads, wl.dk, wl.dv, wl.ring_len, wl.num_slots,
                               wl.batch)
    T, k_rounds = 4, 4
    io = TORCH_DTYPES[wl.io_dtype]
    g0 = torch.Generator().manual_seed(4500)

    def unit(shape):
        a = torch.randn(shape, generator=g0)
        return (a / a.norm(dim=-1, keepdim=True)).to(io).to(dev)

    def normal(shape):
        return torch.randn(shape, generator=g0).to(io).to(dev)

    inps = []
    for _ in range(k_rounds):
        gate = torch.randn((nb, T, HV), generator=g0)
        inps.append({"q": unit((nb, T, HK, K)), "k": unit((nb, T, HK, K)),
                     "v": normal((nb, T, HV, V)),
                     "g": torch.exp(-torch.nn.functional.softplus(gate)).to(dev),
                     "beta": torch.sigmoid(torch.randn((nb, T, HV), generator=g0)).to(dev),
                     "acc": torch.randint(0, T + 1, (nb,), generator=g0, dtype=torch.int32).to(dev),
                     "force": (torch.rand(nb, generator=g0) < 0.2).to(torch.uint8).to(dev)})

    def layer():
        return {"state": gen.state_pool().to(dev),
                "dr": torch.zeros((ns, HV, L, V), device=dev),
                "kr": torch.zeros((ns, HK, L, K), dtype=io, device=dev),
                "gr": torch.zeros((ns, HV, L), device=dev),
                "vr": torch.zeros((ns, HV, L, V), dtype=io, device=dev),
                "br": torch.zeros((ns, HV, L), device=dev),
                "wp": torch.zeros(nb, dtype=torch.int32, device=dev),
                "nwp": torch.zeros(nb, dtype=torch.int32, device=dev),
                "fl": torch.zeros(nb, dtype=torch.uint8, device=dev),
                "o": [torch.empty((nb, T, HV, V), dtype=io, device=dev) for _ in range(k_rounds)]}

    slots = gen.slot_idx().to(dev)
    lay = {"eager": layer(), "graph": layer()}

    def rnd(d, k):
        x = inps[k]
        R.replayssm_gdn_spec_verify(d["state"], d["dr"], d["kr"], d["gr"], d["vr"], d["br"],
                                    slots, d["wp"], x["q"], x["k"], x["v"], x["g"], x["beta"],
                                    o=d["o"][k])
        R.replayssm_gdn_spec_commit(d["state"], d["kr"], d["gr"], d["vr"], d["br"], slots,
                                    d["wp"], x["acc"], T, d["nwp"], force_flush=x["force"],
                                    flushed=d["fl"])
        d["wp"], d["nwp"] = d["nwp"], d["wp"]

    def snapshot(which):
        d = lay[which]
        out = {f"o{k}": d["o"][k].clone() for k in range(k_rounds)}
        out.update(state=d["state"].clone(), wp=d["wp"].clone(), fl=d["fl"].clone(),
                   dr=d["dr"].clone(), kr=d["kr"].clone(), gr=d["gr"].clone(),
                   vr=d["vr"].clone(), br=d["br"].clone())
        return out

    _check_replays(lambda k: rnd(lay["eager"], k), lambda k: rnd(lay["graph"], k), k_rounds,
                   snapshot, dev)


def test_gdn_spec_deferred_rounds_in_a_graph():
    """Deferred-fold rounds (verify with flush + advance: the fold flags and
    the cursors ping-pong), 4 rounds per graph, some rows forced to fold."""
    wl = GdnWorkload("graph_spec_def", 8, 2, 4, 128, 128, 16, 4, 12, "bf16", "f32", 4600)
    gen = GdnInputs(wl)
    dev = torch.device("cuda:0")
    print("case: gdn deferred spec rounds, 4 rounds per graph", flush=True)
    HK, HV, K, V, L, ns, nb = (wl.k_heads, wl.v_heads, wl.dk, wl.dv, wl.ring_len, wl.num_slots,
                               wl.batch)
    T, k_rounds = 4, 4
    io = TORCH_DTYPES[wl.io_dtype]
    g0 = torch.Generator().manual_seed(4600)

    def unit(shape):
        a = torch.randn(shape, generator=g0)
        return (a / a.norm(dim=-1, keepdim=True)).to(io).to(dev)

    def normal(shape):
        return torch.randn(shape, generator=g0).to(io).to(dev)

    inps = []
    for _ in range(k_rounds):
        gate = torch.randn((nb, T, HV), generator=g0)
        inps.append({"q": unit((nb, T, HK, K)), "k": unit((nb, T, HK, K)),
                     "v": normal((nb, T, HV, V)),
                     "g": torch.exp(-torch.nn.functional.softplus(gate)).to(dev),
                     "beta": torch.sigmoid(torch.randn((nb, T, HV), generator=g0)).to(dev),
                     "acc": torch.randint(0, T + 1, (nb,), generator=g0, dtype=torch.int32).to(dev),
                     "force": (torch.rand(nb, generator=g0) < 0.2).to(torch.uint8).to(dev)})

    def layer():
        return {"state": gen.state_pool().to(dev),
                "dr": torch.zeros((ns, HV, L, V), device=dev),
                "kr": torch.zeros((ns, HK, L, K), dtype=io, device=dev),
                "gr": torch.zeros((ns, HV, L), device=dev),
                "vr": torch.zeros((ns, HV, L, V), dtype=io, device=dev),
                "br": torch.zeros((ns, HV, L), device=dev),
                "wp": torch.zeros(nb, dtype=torch.int32, device=dev),
                "nwp": torch.zeros(nb, dtype=torch.int32, device=dev),
                "fl": torch.zeros(nb, dtype=torch.uint8, device=dev),
                "nfl": torch.zeros(nb, dtype=torch.uint8, device=dev),
                "o": [torch.empty((nb, T, HV, V), dtype=io, device=dev) for _ in range(k_rounds)]}

    slots = gen.slot_idx().to(dev)
    lay = {"eager": layer(), "graph": layer()}

    def rnd(d, k):
        x = inps[k]
        R.replayssm_gdn_spec_verify_flush(d["state"], d["dr"], d["kr"], d["gr"], d["vr"],
                                          d["br"], slots, d["wp"], d["fl"], x["q"], x["k"],
                                          x["v"], x["g"], x["beta"], o=d["o"][k])
        R.replayssm_gdn_spec_advance(d["kr"], d["gr"], d["vr"], d["br"], slots, d["wp"], d["fl"],
                                     x["acc"], T, x["k"], x["v"], x["g"], x["beta"], d["nwp"],
                                     d["nfl"], force_flush=x["force"])
        d["wp"], d["nwp"] = d["nwp"], d["wp"]
        d["fl"], d["nfl"] = d["nfl"], d["fl"]

    def snapshot(which):
        d = lay[which]
        out = {f"o{k}": d["o"][k].clone() for k in range(k_rounds)}
        out.update(state=d["state"].clone(), wp=d["wp"].clone(), fl=d["fl"].clone(),
                   dr=d["dr"].clone(), kr=d["kr"].clone(), gr=d["gr"].clone(),
                   vr=d["vr"].clone(), br=d["br"].clone())
        return out

    _check_replays(lambda k: rnd(lay["eager"], k), lambda k: rnd(lay["graph"], k), k_rounds,
                   snapshot, dev)
