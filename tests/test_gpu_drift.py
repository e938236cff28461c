"""Long runs against the float64 oracle: thousands of decode steps, so that
an error which grows slowly (a state that drifts from the recurrence over
many flushes, a bf16 checkpoint whose rounding accumulates) shows up.

The pages name this risk twice: bf16-state outputs of the replay differ from
the baseline because the baseline rounds the state to bf16 every step while
the replay keeps fp32 between flushes (vLLM #48018, Risks), and long outputs
drifted with bf16 until the ring was folded by the exact recurrence (sglang
#28695, review notes).  Here the GPU runs are compared, every step, with the
oracle that rounds at the same points, at the stated tolerances: normwise
relative 2e-5 for fp32 paths, 1e-2 absolute with bf16 inputs or state; and
at the end the state that the GPU's checkpoint + ring represent is compared
with the recurrence.
"""

import pytest
import torch

from harness import run_gdn, run_mamba2
from workloads import GdnWorkload, Mamba2Workload

pytestmark = pytest.mark.gpu

STEPS = 2048


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    import linear_recurrence_amd as R
    R.load()


@pytest.mark.parametrize("io,state_dt", [("f32", "f32"), ("bf16", "bf16"), ("bf16", "f32")])
def test_mamba2_long_run(io, state_dt):
    """4 rows, 8 heads, headdim 64, dstate 16, L = 16, 2048 steps (128 flushes
    per row) with start positions uniform in [0, L); y of every row and step,
    every flushed checkpoint, every cursor, and the end state."""
    print(f"case: mamba2 drift io={io} state={state_dt} steps={STEPS}", flush=True)
    wl = Mamba2Workload(f"drift_{io}_{state_dt}", 4, 8, 64, 16, 1, 16, STEPS, 8, io, state_dt,
                        4100 + len(io) + len(state_dt), desync=True)
    worst = run_mamba2(wl, sample=range(4), y_dtype=torch.float32)
    print(f"worst errors over {STEPS} steps: {worst}", flush=True)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_gdn_long_run(io):
    """GDN decode, 4 rows, 2 key / 4 value heads, K = V = 128, L = 16, 2048
    steps, start positions uniform; outputs every step, checkpoints at every
    flush, and the end state."""
    print(f"case: gdn drift io={io} steps={STEPS}", flush=True)
    wl = GdnWorkload(f"gdn_drift_{io}", 4, 2, 4, 128, 128, 16, STEPS, 8, io, "f32",
                     4200 + len(io), desync=True)
    worst = run_gdn(wl, sample=range(4))
    print(f"worst errors over {STEPS} steps: {worst}", flush=True)


def test_gdn_spec_long_run_through_exact_folds():
    """GDN speculative decoding with bf16 q/k/v: 400 rounds of verify (4
    drafts) and commit, each row folding its ring by the exact recurrence
    every few rounds (about 60 folds per row); every draft output and every
    folded state against the oracle."""
    from test_gpu_gdn_spec import run_spec
    run_spec(4, 2, 4, 128, 128, 16, 4, torch.bfloat16, 400, range(4), seed=4300)


def test_gdn_spec_deferred_long_run_through_exact_folds():
    """The deferred-fold rounds over the same 400-round schedule: each fold
    runs in the next verify, on the tile it loads; draft outputs every round
    and the folded states against the oracle's eager rounds."""
    from test_gpu_gdn_spec import run_spec_deferred
    run_spec_deferred(4, 2, 4, 128, 128, 16, 4, torch.bfloat16, 400, range(4), seed=4300)
