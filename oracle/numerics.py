"""Storage rounding and elementwise helpers for the oracle (float64).

Test infrastructure only; see the package docstring.

The state pool may be stored in bf16 while all arithmetic runs in fp32 on the
device.  vLLM #48018 ("ReplaySSM: cache SSM inputs for faster Mamba2 standard
decode", Risks item 2) explains that the standard update rounds its fp32
result to bf16 on every step, while ReplaySSM accumulates in fp32 and writes
the state once per ring period.  The oracle mirrors that storage step with
``store``: a float64 value is rounded to fp32 (round to nearest even, what an
fp32 accumulator holds) and then, for a bf16 pool, from fp32 to bf16 (round to
nearest even).
"""

import numpy as np

STATE_DTYPES = ("f64", "f32", "bf16")


def softplus(v):
    """softplus(v) = log(1 + e^v), evaluated as max(v, 0) + log1p(e^-|v|).

    The two forms are equal for every real v; the second never overflows.
    Mamba2 applies it to dt_raw + dt_bias when ``dt_softplus`` is set (the
    ``dt_softplus=True`` argument in the ``mamba_mixer2.py`` snippet of
    vLLM #48018).
    """
    v = np.asarray(v, dtype=np.float64)
    return np.maximum(v, 0.0) + np.log1p(np.exp(-np.abs(v)))


def silu_gate(y, z):
    """y * z * sigmoid(z), the Mamba2 output gate, with sigmoid = 1/(1+e^-z)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-z))
    return y * z * sig


def round_f32(a):
    """Round float64 values to the nearest fp32 (ties to even), as float64."""
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_bf16_from_f32(a32):
    """Round fp32 values to bf16 with round-to-nearest-even; return float32.

    bf16 keeps the top 16 bits of the fp32 pattern.  Rounding adds half an
    ulp of the kept part, plus one when the kept part is odd (ties to even),
    then truncates.  NaN is kept NaN (quiet); +-inf and overflow to +-inf
    follow from the same addition.
    """
    a32 = np.ascontiguousarray(a32, dtype=np.float32)
    bits = a32.view(np.uint32).astype(np.uint64)
    keep_lsb = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = (bits + np.uint64(0x7FFF) + keep_lsb) & np.uint64(0xFFFF0000)
    out = (rounded & np.uint64(0xFFFFFFFF)).astype(np.uint32).view(np.float32)
    nan = np.isnan(a32)
    if nan.any():
        out = out.copy()
        out[nan] = np.float32("nan")
    return out


def round_bf16(a):
    """float64 -> fp32 (RNE) -> bf16 (RNE), returned as float64."""
    a32 = np.asarray(a, dtype=np.float64).astype(np.float32)
    return round_bf16_from_f32(a32).astype(np.float64)


# ---- stochastic rounding (vLLM #48018, review notes: SR of the bf16 state
# write-back for quantised models).  Random bits: Philox4x64-10 (Salmon,
# Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011),
# written from its round function; pinned against numpy's Philox bit
# generator in the tests.

_M32 = np.uint64(0xFFFFFFFF)
PHILOX_MUL = (0xD2E7470EE14C6C93, 0xCA5A826395121157)
PHILOX_WEYL = (0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)


def _mulhilo64(a, m):
    """(high, low) 64-bit halves of the 128-bit product a * m (a uint64 array)."""
    a0, a1 = a & _M32, a >> np.uint64(32)
    m0, m1 = np.uint64(m & 0xFFFFFFFF), np.uint64(m >> 32)
    p00, p01, p10, p11 = a0 * m0, a0 * m1, a1 * m0, a1 * m1
    mid = (p00 >> np.uint64(32)) + (p01 & _M32) + (p10 & _M32)
    lo = (p00 & _M32) | ((mid & _M32) << np.uint64(32))
    hi = p11 + (p01 >> np.uint64(32)) + (p10 >> np.uint64(32)) + (mid >> np.uint64(32))
    return hi, lo


def philox4x64_10(ctr, key):
    """Philox4x64 with 10 rounds.  ctr: uint64 [..., 4]; key: (k0, k1) ints.

    Round: (c0, c1, c2, c3) -> (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2),
    hi(M0*c0) ^ c3 ^ k1, lo(M0*c0)); then the key advances by the Weyl
    constants (mod 2^64).
    """
    c = [np.asarray(ctr, np.uint64)[..., i].copy() for i in range(4)]
    k0, k1 = int(key[0]) % 2**64, int(key[1]) % 2**64
    with np.errstate(over="ignore"):
        for _ in range(10):
            hi0, lo0 = _mulhilo64(c[0], PHILOX_MUL[0])
            hi1, lo1 = _mulhilo64(c[2], PHILOX_MUL[1])
            c = [hi1 ^ c[1] ^ np.uint64(k0), lo1, hi0 ^ c[3] ^ np.uint64(k1), lo0]
            k0 = (k0 + PHILOX_WEYL[0]) % 2**64
            k1 = (k1 + PHILOX_WEYL[1]) % 2**64
    return np.stack(c, axis=-1)


def sr_bits(tile, n_elems, seed, offset):
    """16 random bits for each element e of a state tile: Philox4x64-10 with
    key (seed, offset) and counter (tile * n_elems/16 + e // 16, 0, 0, 0);
    element e takes bits 16*(e % 4).. of output word (e % 16) // 4."""
    nblk = n_elems // 16
    ctr = np.zeros((nblk, 4), np.uint64)
    ctr[:, 0] = np.uint64(tile * nblk) + np.arange(nblk, dtype=np.uint64)
    out = philox4x64_10(ctr, (seed, offset))                     # [nblk, 4]
    e = np.arange(16)
    bits = (out[:, e // 4] >> (np.uint64(16) * (e % 4).astype(np.uint64))) & np.uint64(0xFFFF)
    return bits.reshape(n_elems).astype(np.uint32)


def round_bf16_sr_from_f32(a32, r16):
    """fp32 -> bf16 by stochastic rounding with 16 random bits per element:
    the bf16 pattern is (fp32 bits + r) >> 16, so the value rounds away from
    zero with probability (dropped 16 bits) / 2^16; Inf and NaN round to
    nearest.  Returns float32 values."""
    a32 = np.ascontiguousarray(a32, dtype=np.float32)
    u = a32.view(np.uint32).astype(np.uint64)
    out = (((u + np.asarray(r16, np.uint64)) >> np.uint64(16)) << np.uint64(16)).astype(np.uint32)
    res = out.view(np.float32).copy()
    special = (a32.view(np.uint32) & np.uint32(0x7F800000)) == np.uint32(0x7F800000)
    if special.any():
        res[special] = round_bf16_from_f32(a32[special])
    return res


def store_tiles_sr(S, tiles, seed, offset):
    """Stochastic-rounding bf16 store of state tiles S [..., P, N] (float64)
    whose pool tile indices (slot * nheads + head) are ``tiles`` [...]."""
    S = np.asarray(S, np.float64)
    P, N = S.shape[-2:]
    flat = S.reshape(-1, P * N)
    tl = np.asarray(tiles).reshape(-1)
    out = np.empty_like(flat)
    for i in range(flat.shape[0]):
        a32 = flat[i].astype(np.float32)
        out[i] = round_bf16_sr_from_f32(a32, sr_bits(int(tl[i]), P * N, seed, offset))
    return out.reshape(S.shape)


def store(a, state_dtype):
    """Value a float64 state takes once written to a pool of ``state_dtype``."""
    if state_dtype == "f64":
        return np.asarray(a, dtype=np.float64)
    if state_dtype == "f32":
        return round_f32(a)
    if state_dtype == "bf16":
        return round_bf16(a)
    raise ValueError(f"unknown state dtype {state_dtype!r}")
