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


def store(a, state_dtype):
    """Value a float64 state takes once written to a pool of ``state_dtype``."""
    if state_dtype == "f64":
        return np.asarray(a, dtype=np.float64)
    if state_dtype == "f32":
        return round_f32(a)
    if state_dtype == "bf16":
        return round_bf16(a)
    raise ValueError(f"unknown state dtype {state_dtype!r}")
