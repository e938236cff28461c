"""Host metadata of a ReplaySSM decode step (float-free, plain Python).

Test infrastructure only; see the package docstring.

Source: vLLM #48018 "[Kernel] ReplaySSM: cache SSM inputs for faster Mamba2
standard decode" - Implementation item 3 (the metadata builder gives every
row its write_pos and is_flush from a per-request decode base, and re-anchors
in the prefix-caching "align" mode) and the review notes (flush boundary,
one-token prefill, and the preemption fix: the base is re-anchored whenever a
request resumes, since its checkpoint is then no longer at the prompt end).
Copy rule: sglang #28451 / #28695 (a slot is copied only once flushed).

Reading taken here (the pages give no formula):

* decode_base = number of tokens folded into the row's checkpoint S0;
  pos = index of the token decoded in this step;
* the step's ring position is w = pos - decode_base, which must be in [0, L);
* the step flushes when its entry fills the ring (w = L-1), when the caller
  forces it, or, in align mode with block size A, when the token completes a
  block ((pos + 1) % A == 0) so that the checkpoint lands on a block boundary;
* after a flush the checkpoint holds the token: decode_base = pos + 1.
"""


def build_metadata(pos, decode_base, L, force_flush=None, align_block=0):
    """Returns (write_pos, is_flush, next_decode_base) as Python lists."""
    n = len(pos)
    wp, fl, nb = [], [], []
    for r in range(n):
        p, b = int(pos[r]), int(decode_base[r])
        w = p - b
        if p < 0 or b < 0 or not 0 <= w < L:
            raise ValueError(f"row {r}: position {p} is outside the ring of base {b}")
        f = w == L - 1
        if force_flush is not None and force_flush[r]:
            f = True
        if align_block > 0 and (p + 1) % align_block == 0:
            f = True
        wp.append(w)
        fl.append(1 if f else 0)
        nb.append(p + 1 if f else b)
    return wp, fl, nb


def copy_sources_flushed(src_write_pos):
    """A slot may be copied only when its ring is empty (write position 0)."""
    return all(int(w) == 0 for w in src_write_pos)


def flush_first_order(is_flush):
    """The rows whose flush flag is nonzero in increasing index, then the
    others in increasing index (a scheduling order for the decode launch,
    not part of the method: the decode gives the same results for any
    permutation of the rows)."""
    n = len(is_flush)
    return ([r for r in range(n) if int(is_flush[r]) != 0]
            + [r for r in range(n) if int(is_flush[r]) == 0])
