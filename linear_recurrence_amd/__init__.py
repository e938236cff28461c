"""Python binding of libreplayssm (the MI355X ReplaySSM decode library).

Argument marshalling only: every function infers the dimensions from the
tensors, checks devices, dtypes, shapes and contiguity, and passes raw
device pointers plus the current HIP stream to the C ABI declared in
``include/replayssm.h``.  All arithmetic runs in the library's HIP kernels.
PyTorch supplies device memory and streams.

The library must have been built (``python -m linear_recurrence_amd._build``
or ``__graft_entry__.build()``); importing the binding without it, or calling
it on tensors that are not on a GPU, raises instead of computing anything
elsewhere.
"""

import ctypes
import os

import torch  # loads the HIP runtime the library then binds to

__all__ = [
    "ssu_standard_decode", "replayssm_decode", "replayssm_ring_reset",
    "gdn_standard_decode", "replayssm_gdn_decode", "replayssm_gdn_spec_verify",
    "replayssm_gdn_spec_commit", "replayssm_gdn_spec_verify_flush", "replayssm_gdn_spec_advance",
    "kda_standard_decode", "replayssm_kda_decode", "build_metadata", "flush_first_order",
    "check_copy_sources", "library_path", "load",
    "RssmError", "ST_BAD_WRITE_POS", "ST_RING_OVERFLOW", "ST_BAD_SLOT",
    "ST_BAD_ROW", "EXPORTS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libreplayssm.so")

F32, BF16 = 0, 1
ST_BAD_WRITE_POS, ST_RING_OVERFLOW, ST_BAD_SLOT, ST_BAD_ROW = 1, 2, 4, 8
EXPORTS = ("ssu_standard_decode", "replayssm_decode", "replayssm_ring_reset",
           "gdn_standard_decode", "replayssm_gdn_decode", "replayssm_gdn_spec_verify",
           "replayssm_gdn_spec_commit", "replayssm_gdn_spec_verify_flush",
           "replayssm_gdn_spec_advance", "kda_standard_decode", "replayssm_kda_decode",
           "replayssm_build_metadata", "replayssm_decode_ordered", "replayssm_flush_first_order",
           "replayssm_check_copy_sources", "replayssm_strerror", "replayssm_abi_version")

_DT = {torch.float32: F32, torch.bfloat16: BF16}


class RssmError(RuntimeError):
    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} failed with code {code}: {msg}")
        self.code = code


ROUND_NEAREST, ROUND_STOCHASTIC = 0, 1


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "nheads", "headdim", "dstate", "ngroups", "ring_len",
        "num_slots", "state_dtype", "io_dtype", "out_dtype", "dt_softplus",
        "rounding")] + [("sr_seed", ctypes.c_uint64), ("sr_offset", ctypes.c_uint64)]


class GdnDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "k_heads", "v_heads", "dk", "dv", "ring_len", "num_slots",
        "state_dtype", "io_dtype", "out_dtype")] + [("scale", ctypes.c_float)]


_lib = None


def library_path():
    return LIB_PATH


def load():
    """Load libreplayssm.so (once); raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m linear_recurrence_amd._build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int32
    lib.ssu_standard_decode.argtypes = [ctypes.POINTER(Dims)] + [P] * 13
    lib.replayssm_decode.argtypes = [ctypes.POINTER(Dims)] + [P] * 20
    lib.replayssm_decode_ordered.argtypes = [ctypes.POINTER(Dims)] + [P] * 21
    lib.replayssm_decode_ordered.restype = ctypes.c_int
    lib.replayssm_flush_first_order.argtypes = [I, P, P]
    lib.replayssm_flush_first_order.restype = ctypes.c_int
    lib.replayssm_ring_reset.argtypes = [ctypes.POINTER(Dims), P, P, P, I, P, P]
    lib.gdn_standard_decode.argtypes = [ctypes.POINTER(GdnDims)] + [P] * 10
    lib.replayssm_gdn_decode.argtypes = [ctypes.POINTER(GdnDims)] + [P] * 17
    lib.replayssm_gdn_spec_verify.argtypes = [ctypes.POINTER(GdnDims), I] + [P] * 16
    lib.replayssm_gdn_spec_commit.argtypes = [ctypes.POINTER(GdnDims), I] + [P] * 13
    lib.replayssm_gdn_spec_verify_flush.argtypes = [ctypes.POINTER(GdnDims), I] + [P] * 17
    lib.replayssm_gdn_spec_advance.argtypes = [ctypes.POINTER(GdnDims), I] + [P] * 17
    lib.kda_standard_decode.argtypes = [ctypes.POINTER(GdnDims)] + [P] * 10
    lib.replayssm_kda_decode.argtypes = [ctypes.POINTER(GdnDims)] + [P] * 17
    for fn in ("ssu_standard_decode", "replayssm_decode", "replayssm_ring_reset",
               "gdn_standard_decode", "replayssm_gdn_decode", "replayssm_gdn_spec_verify",
               "replayssm_gdn_spec_commit", "replayssm_gdn_spec_verify_flush",
               "replayssm_gdn_spec_advance", "kda_standard_decode", "replayssm_kda_decode"):
        getattr(lib, fn).restype = ctypes.c_int
    lib.replayssm_build_metadata.argtypes = [I, I, I, P, P, P, P, P]
    lib.replayssm_build_metadata.restype = ctypes.c_int
    lib.replayssm_check_copy_sources.argtypes = [I, P]
    lib.replayssm_check_copy_sources.restype = ctypes.c_int
    lib.replayssm_strerror.argtypes = [ctypes.c_int]
    lib.replayssm_strerror.restype = ctypes.c_char_p
    lib.replayssm_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn, rc):
    if rc != 0:
        raise RssmError(fn, rc, load().replayssm_strerror(rc).decode())


def _need(t, name, dtype=None, shape=None, dev=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name} is on {t.device}, expected {dev}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _opt(t, *a, **k):
    return None if t is None else _need(t, *a, **k)


def _rounding(rounding):
    if rounding in ("nearest", None):
        return ROUND_NEAREST
    if rounding == "stochastic":
        return ROUND_STOCHASTIC
    raise ValueError("rounding must be 'nearest' or 'stochastic'")


def _mamba2_dims(state, x, B, ring_len, y_dtype, dt_softplus, rounding=None, sr_seed=0,
                 sr_offset=0):
    ns, H, P, N = state.shape
    nb = x.shape[0]
    G = B.shape[1]
    if state.dtype not in _DT or x.dtype not in _DT or y_dtype not in _DT:
        raise ValueError("dtypes must be float32 or bfloat16")
    return Dims(nb, H, P, N, G, ring_len, ns, _DT[state.dtype], _DT[x.dtype],
                _DT[y_dtype], 1 if dt_softplus else 0, _rounding(rounding),
                sr_seed & (2**64 - 1), sr_offset & (2**64 - 1))


def ssu_standard_decode(state, slot_idx, x, dt, A, B, C, D=None, z=None,
                        dt_bias=None, y=None, dt_softplus=True, status=None,
                        rounding="nearest", sr_seed=0, sr_offset=0,
                        out_dtype=None, stream=None):
    """Standard selective state update (reads and writes ``state``); returns y."""
    dev = _need(state, "state").device
    ns, H, P, N = state.shape
    _need(x, "x", (torch.float32, torch.bfloat16), dev=dev)
    nb = x.shape[0]
    io = x.dtype
    _need(x, "x", io, (nb, H, P))
    _need(B, "B", io, dev=dev)
    G = B.shape[1]
    _need(B, "B", io, (nb, G, N))
    _need(C, "C", io, (nb, G, N))
    _need(dt, "dt", io, (nb, H))
    _need(A, "A", torch.float32, (H,))
    _need(slot_idx, "slot_idx", torch.int32, (nb,))
    _opt(D, "D", torch.float32, (H,))
    _opt(z, "z", io, (nb, H, P))
    _opt(dt_bias, "dt_bias", torch.float32, (H,))
    _opt(status, "status", torch.int32, (1,))
    if y is None:
        y = torch.empty((nb, H, P), dtype=out_dtype or io, device=dev)
    _need(y, "y", (torch.float32, torch.bfloat16), (nb, H, P), dev=dev)
    d = _mamba2_dims(state, x, B, 1, y.dtype, dt_softplus, rounding, sr_seed, sr_offset)
    rc = load().ssu_standard_decode(
        ctypes.byref(d), _ptr(state), _ptr(slot_idx), _ptr(x), _ptr(dt), _ptr(A),
        _ptr(B), _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias), _ptr(y), _ptr(status),
        _stream(stream))
    _check("ssu_standard_decode", rc)
    return y


def replayssm_decode(state, x_ring, dt_ring, B_ring, slot_idx, write_pos,
                     is_flush, x, dt, A, B, C, D=None, z=None, dt_bias=None,
                     y=None, next_write_pos=None, next_is_flush=None,
                     dt_softplus=True, status=None, out_dtype=None, rounding="nearest",
                     sr_seed=0, sr_offset=0, stream=None, row_order=None):
    """One ReplaySSM output-only decode step; returns y.

    Rings: x_ring [slots, H, L, P] (io dtype), dt_ring [slots, H, L] float32,
    B_ring [slots, G, L, N] (io dtype).  Cursors: write_pos int32 [batch],
    is_flush uint8 [batch]; the next cursors are written to next_write_pos /
    next_is_flush when given.  row_order (int32 [batch] on the device, a
    permutation of the rows, flush rows first: see flush_first_order) selects
    replayssm_decode_ordered, which gives the same results with the flush
    rows spread evenly over the GPU's dies.
    """
    dev = _need(state, "state").device
    ns, H, P, N = state.shape
    _need(x, "x", (torch.float32, torch.bfloat16), dev=dev)
    nb = x.shape[0]
    io = x.dtype
    _need(x, "x", io, (nb, H, P))
    _need(B, "B", io, dev=dev)
    G = B.shape[1]
    _need(x_ring, "x_ring", io, dev=dev)
    L = x_ring.shape[2]
    _need(x_ring, "x_ring", io, (ns, H, L, P))
    _need(dt_ring, "dt_ring", torch.float32, (ns, H, L), dev=dev)
    _need(B_ring, "B_ring", io, (ns, G, L, N), dev=dev)
    _need(B, "B", io, (nb, G, N))
    _need(C, "C", io, (nb, G, N))
    _need(dt, "dt", io, (nb, H))
    _need(A, "A", torch.float32, (H,))
    _need(slot_idx, "slot_idx", torch.int32, (nb,))
    _need(write_pos, "write_pos", torch.int32, (nb,))
    _need(is_flush, "is_flush", torch.uint8, (nb,))
    _opt(next_write_pos, "next_write_pos", torch.int32, (nb,))
    _opt(next_is_flush, "next_is_flush", torch.uint8, (nb,))
    _opt(D, "D", torch.float32, (H,))
    _opt(z, "z", io, (nb, H, P))
    _opt(dt_bias, "dt_bias", torch.float32, (H,))
    _opt(status, "status", torch.int32, (1,))
    if y is None:
        y = torch.empty((nb, H, P), dtype=out_dtype or io, device=dev)
    _need(y, "y", (torch.float32, torch.bfloat16), (nb, H, P), dev=dev)
    d = _mamba2_dims(state, x, B, L, y.dtype, dt_softplus, rounding, sr_seed, sr_offset)
    args = [ctypes.byref(d), _ptr(state), _ptr(x_ring), _ptr(dt_ring), _ptr(B_ring),
            _ptr(slot_idx), _ptr(write_pos), _ptr(is_flush), _ptr(next_write_pos),
            _ptr(next_is_flush), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
            _ptr(D), _ptr(z), _ptr(dt_bias), _ptr(y)]
    if row_order is None:
        rc = load().replayssm_decode(*args, _ptr(status), _stream(stream))
        _check("replayssm_decode", rc)
    else:
        _need(row_order, "row_order", torch.int32, (nb,), dev=dev)
        rc = load().replayssm_decode_ordered(*args, _ptr(row_order), _ptr(status),
                                             _stream(stream))
        _check("replayssm_decode_ordered", rc)
    return y


def replayssm_ring_reset(write_pos, is_flush, rows, ring_len, status=None,
                         stream=None):
    """Restart the rings of ``rows`` (int32 device tensor of batch rows)."""
    dev = _need(write_pos, "write_pos", torch.int32).device
    nb = write_pos.shape[0]
    _need(is_flush, "is_flush", torch.uint8, (nb,), dev=dev)
    _need(rows, "rows", torch.int32, dev=dev)
    _opt(status, "status", torch.int32, (1,))
    d = Dims(nb, 1, 0, 0, 1, ring_len, 1, 0, 0, 0, 0, 0, 0, 0)
    rc = load().replayssm_ring_reset(
        ctypes.byref(d), _ptr(write_pos), _ptr(is_flush), _ptr(rows),
        ctypes.c_int32(rows.numel()), _ptr(status), _stream(stream))
    _check("replayssm_ring_reset", rc)


def _host(a, name, dtype, n=None):
    import numpy as np
    if not isinstance(a, np.ndarray) or a.dtype != dtype or a.ndim != 1 or \
            not a.flags.c_contiguous:
        raise TypeError(f"{name} must be a contiguous 1-D numpy {np.dtype(dtype)} array")
    if n is not None and a.shape[0] != n:
        raise ValueError(f"{name} must have {n} entries")
    return ctypes.c_void_p(a.ctypes.data) if a.size else None


def build_metadata(pos, decode_base, ring_len, force_flush=None, align_block=0):
    """Host-side cursors of one decode step (numpy arrays, see the header).

    pos, decode_base: int64 [n] (decode_base is updated in place on flush
    rows); force_flush: optional uint8 [n].  Returns (write_pos int32 [n],
    is_flush uint8 [n]) as numpy arrays.
    """
    import numpy as np
    n = pos.shape[0] if hasattr(pos, "shape") else 0
    pp = _host(pos, "pos", np.int64)
    bp = _host(decode_base, "decode_base", np.int64, n)
    fp = None if force_flush is None else _host(force_flush, "force_flush", np.uint8, n)
    wp = np.zeros(n, np.int32)
    fl = np.zeros(n, np.uint8)
    rc = load().replayssm_build_metadata(
        ctypes.c_int32(n), ctypes.c_int32(ring_len), ctypes.c_int32(align_block), pp, bp, fp,
        ctypes.c_void_p(wp.ctypes.data) if n else None,
        ctypes.c_void_p(fl.ctypes.data) if n else None)
    _check("replayssm_build_metadata", rc)
    return wp, fl


def flush_first_order(is_flush):
    """Row order for replayssm_decode(row_order=...): the flush rows, then the
    others, each in increasing row index.  is_flush: uint8 numpy [n] (host);
    returns an int32 numpy [n]."""
    import numpy as np
    n = is_flush.shape[0] if hasattr(is_flush, "shape") else 0
    fp = _host(is_flush, "is_flush", np.uint8)
    order = np.zeros(n, np.int32)
    rc = load().replayssm_flush_first_order(
        ctypes.c_int32(n), fp, ctypes.c_void_p(order.ctypes.data) if n else None)
    _check("replayssm_flush_first_order", rc)
    return order


def check_copy_sources(src_write_pos):
    """Raise unless every source row's ring is empty (write position 0)."""
    import numpy as np
    n = src_write_pos.shape[0]
    rc = load().replayssm_check_copy_sources(
        ctypes.c_int32(n), _host(src_write_pos, "src_write_pos", np.int32))
    _check("replayssm_check_copy_sources", rc)


def _gdn_dims(state, q, v, ring_len, o_dtype, scale):
    ns, HV, V, K = state.shape
    return GdnDims(v.shape[0], q.shape[1], HV, K, V, ring_len, ns,
                   _DT[state.dtype], _DT[q.dtype], _DT[o_dtype],
                   0.0 if scale is None else float(scale))


def _gdn_inputs(state, q, k, v, g, beta, o, out_dtype, dev, kda=False):
    ns, HV, V, K = state.shape
    _need(state, "state", torch.float32)
    _need(q, "q", (torch.float32, torch.bfloat16), dev=dev)
    nb, HK = q.shape[0], q.shape[1]
    io = q.dtype
    _need(q, "q", io, (nb, HK, K))
    _need(k, "k", io, (nb, HK, K), dev=dev)
    _need(v, "v", io, (nb, HV, V), dev=dev)
    _need(g, "g", torch.float32, (nb, HV, K) if kda else (nb, HV), dev=dev)
    _need(beta, "beta", torch.float32, (nb, HV), dev=dev)
    if o is None:
        o = torch.empty((nb, HV, V), dtype=out_dtype or io, device=dev)
    _need(o, "o", (torch.float32, torch.bfloat16), (nb, HV, V), dev=dev)
    return nb, HK, o


def _gated_standard(fn, kda, state, slot_idx, q, k, v, g, beta, o, scale, status,
                    out_dtype, stream):
    dev = _need(state, "state").device
    nb, HK, o = _gdn_inputs(state, q, k, v, g, beta, o, out_dtype, dev, kda)
    _need(slot_idx, "slot_idx", torch.int32, (nb,), dev=dev)
    _opt(status, "status", torch.int32, (1,))
    d = _gdn_dims(state, q, v, 1, o.dtype, scale)
    rc = getattr(load(), fn)(
        ctypes.byref(d), _ptr(state), _ptr(slot_idx), _ptr(q), _ptr(k), _ptr(v),
        _ptr(g), _ptr(beta), _ptr(o), _ptr(status), _stream(stream))
    _check(fn, rc)
    return o


def _gated_replay(fn, kda, state, d_ring, k_ring, g_ring, slot_idx, write_pos, is_flush,
                  q, k, v, g, beta, o, next_write_pos, next_is_flush, scale, status,
                  out_dtype, stream):
    dev = _need(state, "state").device
    ns, HV, V, K = state.shape
    nb, HK, o = _gdn_inputs(state, q, k, v, g, beta, o, out_dtype, dev, kda)
    _need(d_ring, "d_ring", torch.float32, dev=dev)
    L = d_ring.shape[2]
    _need(d_ring, "d_ring", torch.float32, (ns, HV, L, V))
    _need(k_ring, "k_ring", q.dtype, (ns, HK, L, K), dev=dev)
    _need(g_ring, "g_ring", torch.float32, (ns, HV, L, K) if kda else (ns, HV, L), dev=dev)
    _need(slot_idx, "slot_idx", torch.int32, (nb,), dev=dev)
    _need(write_pos, "write_pos", torch.int32, (nb,), dev=dev)
    _need(is_flush, "is_flush", torch.uint8, (nb,), dev=dev)
    _opt(next_write_pos, "next_write_pos", torch.int32, (nb,), dev=dev)
    _opt(next_is_flush, "next_is_flush", torch.uint8, (nb,), dev=dev)
    _opt(status, "status", torch.int32, (1,))
    d = _gdn_dims(state, q, v, L, o.dtype, scale)
    rc = getattr(load(), fn)(
        ctypes.byref(d), _ptr(state), _ptr(d_ring), _ptr(k_ring), _ptr(g_ring),
        _ptr(slot_idx), _ptr(write_pos), _ptr(is_flush), _ptr(next_write_pos),
        _ptr(next_is_flush), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
        _ptr(o), _ptr(status), _stream(stream))
    _check(fn, rc)
    return o


def gdn_standard_decode(state, slot_idx, q, k, v, g, beta, o=None, scale=None,
                        status=None, out_dtype=None, stream=None):
    """Recurrent gated-delta-rule step (reads and writes ``state``); returns o.
    g, beta [batch, HV] float32."""
    return _gated_standard("gdn_standard_decode", False, state, slot_idx, q, k, v, g, beta,
                           o, scale, status, out_dtype, stream)


def replayssm_gdn_decode(state, d_ring, k_ring, g_ring, slot_idx, write_pos,
                         is_flush, q, k, v, g, beta, o=None, next_write_pos=None,
                         next_is_flush=None, scale=None, status=None,
                         out_dtype=None, stream=None):
    """One GDN ReplaySSM decode step; returns o.

    Rings: d_ring [slots, HV, L, V] float32, k_ring [slots, HK, L, K] (io
    dtype), g_ring [slots, HV, L] float32.
    """
    return _gated_replay("replayssm_gdn_decode", False, state, d_ring, k_ring, g_ring,
                         slot_idx, write_pos, is_flush, q, k, v, g, beta, o, next_write_pos,
                         next_is_flush, scale, status, out_dtype, stream)


def kda_standard_decode(state, slot_idx, q, k, v, g, beta, o=None, scale=None,
                        status=None, out_dtype=None, stream=None):
    """Recurrent KDA step (per-key-channel gate g [batch, HV, K] float32);
    reads and writes ``state``; returns o."""
    return _gated_standard("kda_standard_decode", True, state, slot_idx, q, k, v, g, beta,
                           o, scale, status, out_dtype, stream)


def replayssm_kda_decode(state, d_ring, k_ring, g_ring, slot_idx, write_pos,
                         is_flush, q, k, v, g, beta, o=None, next_write_pos=None,
                         next_is_flush=None, scale=None, status=None,
                         out_dtype=None, stream=None):
    """One KDA ReplaySSM decode step; returns o.

    g [batch, HV, K] float32; rings as for replayssm_gdn_decode except
    g_ring [slots, HV, L, K] float32.
    """
    return _gated_replay("replayssm_kda_decode", True, state, d_ring, k_ring, g_ring,
                         slot_idx, write_pos, is_flush, q, k, v, g, beta, o, next_write_pos,
                         next_is_flush, scale, status, out_dtype, stream)


def _spec_rings(state, d_ring, k_ring, g_ring, v_ring, beta_ring, io, dev):
    ns, HV, V, K = state.shape
    _need(k_ring, "k_ring", io, dev=dev)
    HK, L = k_ring.shape[1], k_ring.shape[2]
    _need(k_ring, "k_ring", io, (ns, HK, L, K))
    if d_ring is not None:
        _need(d_ring, "d_ring", torch.float32, (ns, HV, L, V), dev=dev)
    _need(g_ring, "g_ring", torch.float32, (ns, HV, L), dev=dev)
    _need(v_ring, "v_ring", io, (ns, HV, L, V), dev=dev)
    _need(beta_ring, "beta_ring", torch.float32, (ns, HV, L), dev=dev)
    return HK, L


def replayssm_gdn_spec_verify(state, d_ring, k_ring, g_ring, v_ring, beta_ring, slot_idx,
                              write_pos, q, k, v, g, beta, o=None, scale=None, status=None,
                              out_dtype=None, stream=None):
    """Verify T draft tokens per row from the checkpoint and the ring; returns o.

    q, k [batch, T, HK, K]; v [batch, T, HV, V] (io dtype); g, beta
    [batch, T, HV] float32; o [batch, T, HV, V].  Writes ring entries
    w..w+T-1; leaves the state and the cursors alone.
    """
    return _spec_verify("replayssm_gdn_spec_verify", state, d_ring, k_ring, g_ring, v_ring,
                        beta_ring, slot_idx, write_pos, None, q, k, v, g, beta, o, scale, status,
                        out_dtype, stream)


def replayssm_gdn_spec_verify_flush(state, d_ring, k_ring, g_ring, v_ring, beta_ring, slot_idx,
                                    write_pos, is_flush, q, k, v, g, beta, o=None, scale=None,
                                    status=None, out_dtype=None, stream=None):
    """The verify of the deferred-fold rounds: rows with is_flush [batch]
    (uint8) set first fold ring entries 0..w-1 into the state by the exact
    recurrence, then verify their drafts at entries 0..T-1 (their k rows are
    written by replayssm_gdn_spec_advance); the other rows as in
    replayssm_gdn_spec_verify.  Returns o."""
    return _spec_verify("replayssm_gdn_spec_verify_flush", state, d_ring, k_ring, g_ring,
                        v_ring, beta_ring, slot_idx, write_pos, is_flush, q, k, v, g, beta, o,
                        scale, status, out_dtype, stream)


def _spec_verify(fn, state, d_ring, k_ring, g_ring, v_ring, beta_ring, slot_idx, write_pos,
                 is_flush, q, k, v, g, beta, o, scale, status, out_dtype, stream):
    dev = _need(state, "state", torch.float32).device
    ns, HV, V, K = state.shape
    _need(q, "q", (torch.float32, torch.bfloat16), dev=dev)
    nb, T, HK = q.shape[0], q.shape[1], q.shape[2]
    io = q.dtype
    _need(q, "q", io, (nb, T, HK, K))
    _need(k, "k", io, (nb, T, HK, K), dev=dev)
    _need(v, "v", io, (nb, T, HV, V), dev=dev)
    _need(g, "g", torch.float32, (nb, T, HV), dev=dev)
    _need(beta, "beta", torch.float32, (nb, T, HV), dev=dev)
    _, L = _spec_rings(state, d_ring, k_ring, g_ring, v_ring, beta_ring, io, dev)
    _need(slot_idx, "slot_idx", torch.int32, (nb,), dev=dev)
    _need(write_pos, "write_pos", torch.int32, (nb,), dev=dev)
    if is_flush is not None:
        _need(is_flush, "is_flush", torch.uint8, (nb,), dev=dev)
    _opt(status, "status", torch.int32, (1,))
    if o is None:
        o = torch.empty((nb, T, HV, V), dtype=out_dtype or io, device=dev)
    _need(o, "o", (torch.float32, torch.bfloat16), (nb, T, HV, V), dev=dev)
    d = GdnDims(nb, HK, HV, K, V, L, ns, F32, _DT[io], _DT[o.dtype],
                0.0 if scale is None else float(scale))
    head = [ctypes.byref(d), ctypes.c_int32(T), _ptr(state), _ptr(d_ring), _ptr(k_ring),
            _ptr(g_ring), _ptr(v_ring), _ptr(beta_ring), _ptr(slot_idx), _ptr(write_pos)]
    if is_flush is not None:
        head.append(_ptr(is_flush))
    rc = getattr(load(), fn)(*head, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(o),
                             _ptr(status), _stream(stream))
    _check(fn, rc)
    return o


def replayssm_gdn_spec_commit(state, k_ring, g_ring, v_ring, beta_ring, slot_idx, write_pos,
                              accepted, n_draft, next_write_pos, force_flush=None,
                              flushed=None, status=None, stream=None):
    """Keep the accepted drafts; rows whose next verify would not fit (or
    forced) fold their ring into the state by the exact recurrence."""
    dev = _need(state, "state", torch.float32).device
    ns, HV, V, K = state.shape
    io = k_ring.dtype
    HK, L = _spec_rings(state, None, k_ring, g_ring, v_ring, beta_ring, io, dev)
    nb = slot_idx.shape[0]
    _need(slot_idx, "slot_idx", torch.int32, (nb,), dev=dev)
    _need(write_pos, "write_pos", torch.int32, (nb,), dev=dev)
    _need(accepted, "accepted", torch.int32, (nb,), dev=dev)
    _need(next_write_pos, "next_write_pos", torch.int32, (nb,), dev=dev)
    _opt(force_flush, "force_flush", torch.uint8, (nb,), dev=dev)
    _opt(flushed, "flushed", torch.uint8, (nb,), dev=dev)
    _opt(status, "status", torch.int32, (1,))
    d = GdnDims(nb, HK, HV, K, V, L, ns, F32, _DT[io], _DT[io], 0.0)
    rc = load().replayssm_gdn_spec_commit(
        ctypes.byref(d), ctypes.c_int32(n_draft), _ptr(state), _ptr(k_ring), _ptr(g_ring),
        _ptr(v_ring), _ptr(beta_ring), _ptr(slot_idx), _ptr(write_pos), _ptr(accepted),
        _ptr(force_flush), _ptr(next_write_pos), _ptr(flushed), _ptr(status), _stream(stream))
    _check("replayssm_gdn_spec_commit", rc)


def replayssm_gdn_spec_advance(k_ring, g_ring, v_ring, beta_ring, slot_idx, write_pos, is_flush,
                               accepted, n_draft, k, v, g, beta, next_write_pos, next_is_flush,
                               force_flush=None, status=None, stream=None):
    """Cursor advance of the deferred-fold rounds (no fold here): a row that
    folded in this round's verify (is_flush set) restarts from entry 0; the
    kept drafts' v, k, g, beta rows (this round's inputs: k [batch, T, HK,
    K], v [batch, T, HV, V], g, beta [batch, T, HV]) go to their ring
    entries; w' = w + accepted and next_is_flush = (w' + T > L) or
    force_flush."""
    dev = k_ring.device
    io = k_ring.dtype
    _need(k_ring, "k_ring", (torch.float32, torch.bfloat16), dev=dev)
    ns, HK, L, K = k_ring.shape
    _need(v_ring, "v_ring", io, dev=dev)
    HV, V = v_ring.shape[1], v_ring.shape[3]
    _need(v_ring, "v_ring", io, (ns, HV, L, V))
    _need(g_ring, "g_ring", torch.float32, (ns, HV, L), dev=dev)
    _need(beta_ring, "beta_ring", torch.float32, (ns, HV, L), dev=dev)
    nb = slot_idx.shape[0]
    T = n_draft
    _need(k, "k", io, (nb, T, HK, K), dev=dev)
    _need(v, "v", io, (nb, T, HV, V), dev=dev)
    _need(g, "g", torch.float32, (nb, T, HV), dev=dev)
    _need(beta, "beta", torch.float32, (nb, T, HV), dev=dev)
    _need(slot_idx, "slot_idx", torch.int32, (nb,), dev=dev)
    _need(write_pos, "write_pos", torch.int32, (nb,), dev=dev)
    _need(is_flush, "is_flush", torch.uint8, (nb,), dev=dev)
    _need(accepted, "accepted", torch.int32, (nb,), dev=dev)
    _need(next_write_pos, "next_write_pos", torch.int32, (nb,), dev=dev)
    _need(next_is_flush, "next_is_flush", torch.uint8, (nb,), dev=dev)
    _opt(force_flush, "force_flush", torch.uint8, (nb,), dev=dev)
    _opt(status, "status", torch.int32, (1,))
    d = GdnDims(nb, HK, HV, K, V, L, ns, F32, _DT[io], _DT[io], 0.0)
    rc = load().replayssm_gdn_spec_advance(
        ctypes.byref(d), ctypes.c_int32(T), _ptr(k_ring), _ptr(g_ring), _ptr(v_ring),
        _ptr(beta_ring), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(slot_idx), _ptr(write_pos),
        _ptr(is_flush), _ptr(accepted), _ptr(force_flush), _ptr(next_write_pos),
        _ptr(next_is_flush), _ptr(status), _stream(stream))
    _check("replayssm_gdn_spec_advance", rc)