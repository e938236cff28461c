// Mamba2 decode entry points of the C ABI (standard update, ReplaySSM step,
// ring reset): argument checks and dispatch to the kernels of
// mamba2_kernel.hpp.  Stochastic-rounding instances live in mamba2_sr.hip.
#include <stddef.h>

#include "mamba2_kernel.hpp"

// the Python binding mirrors this layout
static_assert(sizeof(rssm_dims) == 64 && offsetof(rssm_dims, sr_seed) == 48 &&
                  offsetof(rssm_dims, sr_offset) == 56,
              "rssm_dims layout");

namespace rssm {

static bool shape_supported(int P, int N) {
  const bool p_ok = P == 32 || P == 64 || P == 128;
  const bool n_ok = N == 16 || N == 32 || N == 64 || N == 128 || N == 256;
  return p_ok && n_ok;
}

static int check_dims(const rssm_dims* d, bool replay) {
  if (!d) return RSSM_EINVAL;
  if (d->batch < 0 || d->nheads < 1 || d->ngroups < 1 || d->nheads % d->ngroups ||
      d->num_slots < 1)
    return RSSM_EINVAL;
  if ((long)d->batch * d->nheads > 0x7fffffffL) return RSSM_EINVAL;
  if (!valid_dtype(d->state_dtype) || !valid_dtype(d->io_dtype) || !valid_dtype(d->out_dtype))
    return RSSM_EDTYPE;
  if (!shape_supported(d->headdim, d->dstate)) return RSSM_ESHAPE;
  if (replay && (d->ring_len < 1 || d->ring_len > 64)) return RSSM_ESHAPE;
  if (d->rounding != RSSM_ROUND_NEAREST && d->rounding != RSSM_ROUND_STOCHASTIC)
    return RSSM_EINVAL;
  if (d->rounding == RSSM_ROUND_STOCHASTIC && d->state_dtype != RSSM_BF16) return RSSM_EDTYPE;
  return RSSM_OK;
}

// Waves the replay grid has with 16 vectors per lane (each wave streams
// 16 KB of state); below kSmallGrid the tiles are split over 4x more waves.
// 4 waves per SIMD x 1024 SIMDs is one round of resident waves: a grid of
// about one round is bound by its slowest waves (the flush tiles), which
// four waves per tile shorten.  Measured on the batch-512 bf16 layer with
// 10 / 20 / 40 heads (5120 / 10240 / 20480 one-wave tiles): 4 vectors per
// lane +5% at 10 heads, -12% at 20, equal at 40.
constexpr long kSmallGrid = 8192;

static int dispatch(bool replay, const Mamba2Args& a, const rssm_dims& d, hipStream_t s) {
  if (d.rounding == RSSM_ROUND_STOCHASTIC) return dispatch_mamba2_sr(replay, a, d, s);
  if (!replay) return dispatch_mamba2<false, false, 4>(a, d, s);
  const long tile_bytes = (long)d.headdim * d.dstate * (d.state_dtype == RSSM_BF16 ? 2 : 4);
  const long waves = (long)d.batch * d.nheads * (tile_bytes > 16384 ? tile_bytes / 16384 : 1);
  if (waves < kSmallGrid) return dispatch_mamba2_small(a, d, s);
  return dispatch_mamba2<true, false, 16>(a, d, s);
}

}  // namespace rssm

using namespace rssm;

extern "C" int ssu_standard_decode(const rssm_dims* dims, void* state, const int32_t* slot_idx,
                                   const void* x, const void* dt, const float* A, const void* B,
                                   const void* C, const float* D, const void* z,
                                   const float* dt_bias, void* y, int32_t* status,
                                   hipStream_t stream) {
  int rc = check_dims(dims, false);
  if (rc) return rc;
  if (dims->batch == 0) return RSSM_OK;  // empty batch: nothing to read or write
  if (!state || !slot_idx || !x || !dt || !A || !B || !C || !y) return RSSM_EINVAL;
  if (!aligned16(state) || !aligned16(x) || !aligned16(B) || !aligned16(C) ||
      (z && !aligned16(z)))
    return RSSM_EINVAL;
  Mamba2Args a{};
  a.state = state;
  a.slot_idx = slot_idx;
  a.x = x;
  a.dt = dt;
  a.A = A;
  a.B = B;
  a.C = C;
  a.D = D;
  a.z = z;
  a.dt_bias = dt_bias;
  a.y = y;
  a.status = status;
  a.nheads = dims->nheads;
  a.ngroups = dims->ngroups;
  a.hpg = dims->nheads / dims->ngroups;
  a.ring_len = 1;
  a.num_slots = dims->num_slots;
  a.dt_softplus = dims->dt_softplus;
  a.sr_seed = dims->sr_seed;
  a.sr_offset = dims->sr_offset;
  return dispatch(false, a, *dims, stream);
}

static int replay_entry(const rssm_dims* dims, void* state, void* x_ring, float* dt_ring,
                        void* B_ring, const int32_t* slot_idx, const int32_t* write_pos,
                        const uint8_t* is_flush, int32_t* next_write_pos, uint8_t* next_is_flush,
                        const void* x, const void* dt, const float* A, const void* B,
                        const void* C, const float* D, const void* z, const float* dt_bias,
                        void* y, const int32_t* row_order, int32_t* status, hipStream_t stream) {
  int rc = check_dims(dims, true);
  if (rc) return rc;
  if (dims->batch == 0) return RSSM_OK;  // empty batch: nothing to read or write
  if (!state || !x_ring || !dt_ring || !B_ring || !slot_idx || !write_pos || !is_flush || !x ||
      !dt || !A || !B || !C || !y)
    return RSSM_EINVAL;
  if (!aligned16(state) || !aligned16(x_ring) || !aligned16(B_ring) || !aligned16(x) ||
      !aligned16(B) || !aligned16(C) || (z && !aligned16(z)))
    return RSSM_EINVAL;
  if ((const void*)next_write_pos == (const void*)write_pos && next_write_pos) return RSSM_EINVAL;
  if ((const void*)next_is_flush == (const void*)is_flush && next_is_flush) return RSSM_EINVAL;
  Mamba2Args a{};
  a.state = state;
  a.x_ring = x_ring;
  a.dt_ring = dt_ring;
  a.B_ring = B_ring;
  a.slot_idx = slot_idx;
  a.write_pos = write_pos;
  a.is_flush = is_flush;
  a.next_write_pos = next_write_pos;
  a.next_is_flush = next_is_flush;
  a.x = x;
  a.dt = dt;
  a.A = A;
  a.B = B;
  a.C = C;
  a.D = D;
  a.z = z;
  a.dt_bias = dt_bias;
  a.y = y;
  a.status = status;
  a.nheads = dims->nheads;
  a.ngroups = dims->ngroups;
  a.hpg = dims->nheads / dims->ngroups;
  a.ring_len = dims->ring_len;
  a.num_slots = dims->num_slots;
  a.dt_softplus = dims->dt_softplus;
  a.sr_seed = dims->sr_seed;
  a.sr_offset = dims->sr_offset;
  a.row_order = row_order;
  // batches of up to 512 rows with 8-byte aligned flags: the full-grid
  // kernel deals the flush rows over the XCDs itself
  a.batch_dealt = dims->batch <= 512 && (reinterpret_cast<uintptr_t>(is_flush) & 7) == 0;
  return dispatch(true, a, *dims, stream);
}

extern "C" int replayssm_decode(const rssm_dims* dims, void* state, void* x_ring, float* dt_ring,
                                void* B_ring, const int32_t* slot_idx, const int32_t* write_pos,
                                const uint8_t* is_flush, int32_t* next_write_pos,
                                uint8_t* next_is_flush, const void* x, const void* dt,
                                const float* A, const void* B, const void* C, const float* D,
                                const void* z, const float* dt_bias, void* y, int32_t* status,
                                hipStream_t stream) {
  return replay_entry(dims, state, x_ring, dt_ring, B_ring, slot_idx, write_pos, is_flush,
                      next_write_pos, next_is_flush, x, dt, A, B, C, D, z, dt_bias, y, nullptr,
                      status, stream);
}

extern "C" int replayssm_decode_ordered(const rssm_dims* dims, void* state, void* x_ring,
                                        float* dt_ring, void* B_ring, const int32_t* slot_idx,
                                        const int32_t* write_pos, const uint8_t* is_flush,
                                        int32_t* next_write_pos, uint8_t* next_is_flush,
                                        const void* x, const void* dt, const float* A,
                                        const void* B, const void* C, const float* D,
                                        const void* z, const float* dt_bias, void* y,
                                        const int32_t* row_order, int32_t* status,
                                        hipStream_t stream) {
  if (!row_order) return RSSM_EINVAL;
  return replay_entry(dims, state, x_ring, dt_ring, B_ring, slot_idx, write_pos, is_flush,
                      next_write_pos, next_is_flush, x, dt, A, B, C, D, z, dt_bias, y, row_order,
                      status, stream);
}

namespace rssm {

struct ResetArgs {
  int32_t* write_pos;
  uint8_t* is_flush;
  const int32_t* rows;
  int32_t* status;
  int32_t n_rows;
  int32_t batch;
  int32_t ring_len;
};

__global__ void __launch_bounds__(256) ring_reset_kernel(const ResetArgs a) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= a.n_rows) return;
  const int r = a.rows[i];
  if (r < 0 || r >= a.batch) {
    if (a.status) atomicOr(a.status, RSSM_ST_BAD_ROW);
    return;
  }
  a.write_pos[r] = 0;
  a.is_flush[r] = a.ring_len == 1 ? 1 : 0;
}

}  // namespace rssm

extern "C" int replayssm_ring_reset(const rssm_dims* dims, int32_t* write_pos, uint8_t* is_flush,
                                    const int32_t* rows, int32_t n_rows, int32_t* status,
                                    hipStream_t stream) {
  if (!dims || dims->batch < 0 || dims->ring_len < 1 || dims->ring_len > 64 || n_rows < 0)
    return RSSM_EINVAL;
  if (n_rows == 0) return RSSM_OK;
  if (!write_pos || !is_flush || !rows) return RSSM_EINVAL;
  ResetArgs a{write_pos, is_flush, rows, status, n_rows, dims->batch, dims->ring_len};
  return launch_kernel(reinterpret_cast<const void*>(&ring_reset_kernel),
                       (unsigned)((n_rows + 255) / 256), 256, 0, stream, a);
}

extern "C" const char* replayssm_strerror(int code) {
  switch (code) {
    case RSSM_OK: return "ok";
    case RSSM_EINVAL: return "invalid argument (null pointer, size, alignment or aliasing)";
    case RSSM_EDTYPE: return "unsupported dtype combination";
    case RSSM_ELAUNCH: return "kernel launch failed";
    case RSSM_ESHAPE: return "shape not supported by the compiled kernels";
  }
  return "unknown error";
}

extern "C" int replayssm_abi_version(void) { return 102; }
