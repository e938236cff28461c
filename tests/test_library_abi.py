"""CPU-side checks of the C-ABI library: it loads and exports every entry
point declared in include/*.h (no compute calls: there is no GPU here)."""

import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?\w+\s*\**\s*(\w+)\s*\(", src, re.M):
            names.add(m.group(1))
    return names


def test_header_declares_the_boundary():
    names = _declared()
    for fn in ("ssu_standard_decode", "replayssm_decode", "replayssm_ring_reset",
               "gdn_standard_decode", "replayssm_gdn_decode", "kda_standard_decode",
               "replayssm_kda_decode"):
        assert fn in names


def test_library_loads_and_exports_every_declared_symbol():
    import linear_recurrence_amd as R
    if not os.path.exists(R.library_path()):
        pytest.fail("libreplayssm.so is not built; run __graft_entry__.build()")
    lib = R.load()
    for fn in sorted(_declared()):
        assert hasattr(lib, fn), f"{fn} is declared but not exported"
    assert set(R.EXPORTS) <= _declared()
    assert lib.replayssm_abi_version() == 102
    assert lib.replayssm_strerror(-4).decode().startswith("shape")


def test_host_validation_rejects_bad_arguments_without_a_gpu():
    """Argument checks happen on the host before any HIP call, so they can be
    exercised here: NULL dims, bad sizes, bad dtypes, unsupported shapes and
    misaligned pointers all return their codes."""
    import linear_recurrence_amd as R
    lib = R.load()
    V = ctypes.c_void_p
    good = dict(batch=2, nheads=4, headdim=64, dstate=16, ngroups=2, ring_len=4,
                num_slots=4, state_dtype=0, io_dtype=0, out_dtype=0, dt_softplus=1)

    def call(**over):
        d = R.Dims(**{**good, **over.pop("dims", {})})
        p = {k: V(0x1000) for k in ("state", "xr", "dr", "br", "slot", "wp", "fl",
                                    "x", "dt", "A", "B", "C", "y")}
        p.update(over)
        return lib.replayssm_decode(
            ctypes.byref(d), p["state"], p["xr"], p["dr"], p["br"], p["slot"],
            p["wp"], p["fl"], None, None, p["x"], p["dt"], p["A"], p["B"], p["C"],
            None, None, None, p["y"], None, None)

    assert lib.replayssm_decode(None, *([None] * 20)) == -1
    assert call(dims=dict(ngroups=3)) == -1
    assert call(dims=dict(batch=-1)) == -1
    assert call(dims=dict(io_dtype=5)) == -2
    assert call(dims=dict(headdim=48)) == -4
    assert call(dims=dict(ring_len=0)) == -4
    assert call(dims=dict(ring_len=65)) == -4
    assert call(x=V(0x1004)) == -1                  # misaligned vector operand
    assert call(y=None) == -1                       # required pointer
    assert call(dims=dict(batch=0)) == 0            # empty batch: nothing to do
    assert call(dims=dict(rounding=2)) == -1        # unknown rounding mode
    assert call(dims=dict(rounding=1)) == -2        # stochastic rounding of an fp32 state
    assert call(dims=dict(rounding=1, state_dtype=1, batch=0)) == 0
    gd = R.GdnDims(2, 1, 2, 128, 128, 4, 4, 1, 1, 1, 0.0)
    assert lib.gdn_standard_decode(ctypes.byref(gd), *([V(0x1000)] * 8), None, None) == -2
    gd = R.GdnDims(2, 1, 2, 128, 128, 8, 4, 0, 1, 1, 0.0)
    sv = [V(0x1000)] * 14                     # state .. o
    assert lib.replayssm_gdn_spec_verify(ctypes.byref(gd), 0, *sv, None, None) == -4   # T < 1
    assert lib.replayssm_gdn_spec_verify(ctypes.byref(gd), 5, *sv, None, None) == -4   # 2T > L
    assert lib.replayssm_gdn_spec_verify(ctypes.byref(gd), 4, *sv[:13], None, None, None) == -1
    cm = [V(0x1000)] * 6                      # state .. slot_idx
    assert lib.replayssm_gdn_spec_commit(ctypes.byref(gd), 4, *cm, V(0x1000), None, None,
                                         V(0x2000), None, None, None) == -1        # no accepted
    assert lib.replayssm_gdn_spec_commit(ctypes.byref(gd), 4, *cm, V(0x3000), V(0x1000), None,
                                         V(0x3000), None, None, None) == -1        # aliasing
    # deferred-fold rounds: is_flush is required; a folding row's raw ring
    # rows must fit beside the verify's staging (46 entries at T = 4, bf16)
    P = V(0x1000)
    fv = [P] * 8                              # state .. write_pos
    gd = R.GdnDims(2, 1, 2, 128, 128, 16, 4, 0, 1, 1, 0.0)
    assert lib.replayssm_gdn_spec_verify_flush(ctypes.byref(gd), 4, *fv, None, *[P] * 6,
                                               None, None) == -1
    for L, io in ((47, 1), (28, 0)):         # past 46 (bf16) / 27 (fp32) entries
        gd = R.GdnDims(2, 1, 2, 128, 128, L, 4, 0, io, 1, 0.0)
        assert lib.replayssm_gdn_spec_verify_flush(ctypes.byref(gd), 4, *fv, P, *[P] * 6,
                                                   None, None) == -4
    gd = R.GdnDims(2, 1, 2, 128, 128, 16, 4, 0, 1, 1, 0.0)
    A, B = V(0x2000), V(0x3000)
    rk = [P] * 8                              # k_ring .. beta
    assert lib.replayssm_gdn_spec_advance(ctypes.byref(gd), 4, *rk, P, P, A, P, None, B, A,
                                          None, None) == -1        # next_is_flush aliases is_flush
    assert lib.replayssm_gdn_spec_advance(ctypes.byref(gd), 4, *rk, P, B, A, P, None, B, P,
                                          None, None) == -1        # next_write_pos aliases write_pos
    assert lib.replayssm_gdn_spec_advance(ctypes.byref(gd), 4, *rk, P, P, A, None, None, B, P,
                                          None, None) == -1        # no accepted
    assert lib.replayssm_gdn_spec_advance(ctypes.byref(gd), 4, P, P, P, P, P, V(0x1008), P, P,
                                          P, P, A, P, None, B, P, None, None) == -1  # misaligned v
    # KDA: the gate rows are vector operands (16-byte alignment) and take LDS
    # of their own (at K = V = 128 a ring fits 48 entries with bf16 inputs)
    P = V(0x1000)
    for L, io in ((49, 1), (41, 0), (64, 1)):  # past 48 (bf16) / 40 (fp32) entries
        kd = R.GdnDims(2, 2, 2, 128, 128, L, 4, 0, io, 1, 0.0)
        assert lib.replayssm_kda_decode(ctypes.byref(kd), *[P] * 7, None, None,
                                        *[P] * 6, None, None) == -4
    kd = R.GdnDims(2, 2, 2, 128, 128, 16, 4, 0, 1, 1, 0.0)
    assert lib.replayssm_kda_decode(ctypes.byref(kd), P, P, P, V(0x1004), *[P] * 3, None,
                                    None, *[P] * 6, None, None) == -1   # misaligned g_ring
    assert lib.replayssm_kda_decode(ctypes.byref(kd), *[P] * 7, None, None, P, P, P,
                                    V(0x1004), P, P, None, None) == -1  # misaligned g
    assert lib.kda_standard_decode(ctypes.byref(kd), P, P, P, P, P, V(0x1004), P, P,
                                   None, None) == -1
    kd = R.GdnDims(2, 2, 2, 128, 128, 16, 4, 1, 1, 1, 0.0)               # bf16 state
    assert lib.kda_standard_decode(ctypes.byref(kd), *[P] * 8, None, None) == -2
    d = R.Dims(**good)
    assert lib.replayssm_ring_reset(ctypes.byref(d), None, None, None, 0, None, None) == 0
    assert lib.replayssm_ring_reset(ctypes.byref(d), None, None, None, -1, None, None) == -1
