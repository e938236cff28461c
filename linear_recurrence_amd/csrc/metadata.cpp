// Host-side ReplaySSM cursors: per-row write position and flush flag for one
// decode step, computed from token positions (plain C++, no device code).
//
// Method: vLLM #48018 "[Kernel] ReplaySSM: cache SSM inputs for faster Mamba2
// standard decode" - Implementation item 3 (the metadata builder derives each
// row's write_pos and is_flush from a per-request decode base, with
// re-anchoring in the prefix-caching "align" mode) and the review notes (the
// flush boundary and the one-token prefill are the risky cases; a preempted
// request resumes from a checkpoint that is no longer at the prompt end, so
// the base is re-anchored on every resume).  Copy rule: sglang #28451 /
// sglang #28695 - a slot may only be copied once its ring is empty (the
// source has flushed).  The formulas are in replayssm.h.
#include <stdint.h>

#include "replayssm.h"

extern "C" int replayssm_build_metadata(int32_t n_rows, int32_t ring_len, int32_t align_block,
                                        const int64_t* pos, int64_t* decode_base,
                                        const uint8_t* force_flush, int32_t* write_pos,
                                        uint8_t* is_flush) {
  if (n_rows < 0 || ring_len < 1 || align_block < 0) return RSSM_EINVAL;
  if (n_rows == 0) return RSSM_OK;
  if (!pos || !decode_base || !write_pos || !is_flush) return RSSM_EINVAL;
  // validate every row before writing anything
  for (int32_t r = 0; r < n_rows; ++r) {
    const int64_t w = pos[r] - decode_base[r];
    if (pos[r] < 0 || decode_base[r] < 0 || w < 0 || w >= ring_len) return RSSM_EINVAL;
  }
  for (int32_t r = 0; r < n_rows; ++r) {
    const int64_t w = pos[r] - decode_base[r];
    const bool f = w == ring_len - 1 || (force_flush && force_flush[r]) ||
                   (align_block > 0 && (pos[r] + 1) % align_block == 0);
    write_pos[r] = (int32_t)w;
    is_flush[r] = f ? 1 : 0;
    if (f) decode_base[r] = pos[r] + 1;  // the checkpoint now holds this token
  }
  return RSSM_OK;
}

extern "C" int replayssm_check_copy_sources(int32_t n, const int32_t* src_write_pos) {
  if (n < 0) return RSSM_EINVAL;
  if (n == 0) return RSSM_OK;
  if (!src_write_pos) return RSSM_EINVAL;
  for (int32_t i = 0; i < n; ++i)
    if (src_write_pos[i] != 0) return RSSM_EINVAL;  // ring not empty: its entries would be lost
  return RSSM_OK;
}

extern "C" int replayssm_flush_first_order(int32_t n_rows, const uint8_t* is_flush,
                                           int32_t* row_order) {
  if (n_rows < 0) return RSSM_EINVAL;
  if (n_rows == 0) return RSSM_OK;
  if (!is_flush || !row_order) return RSSM_EINVAL;
  int32_t k = 0;
  for (int32_t r = 0; r < n_rows; ++r)
    if (is_flush[r]) row_order[k++] = r;  // flush rows first, in row order
  for (int32_t r = 0; r < n_rows; ++r)
    if (!is_flush[r]) row_order[k++] = r;  // then the others, in row order
  return RSSM_OK;
}
