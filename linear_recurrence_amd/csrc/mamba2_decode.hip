// Mamba2 decode kernels for gfx950: the standard selective state update and
// the ReplaySSM output-only step (checkpoint S0 + per-slot input ring, fold
// on flush rows only), plus the cursor reset used on slot reuse.
//
// Method: vLLM #48018 "[Kernel] ReplaySSM: cache SSM inputs for faster Mamba2
// standard decode" - Motivation (the per-step state load+store dominates HBM
// traffic; a ring of inputs plus a periodic checkpoint lets most steps read
// the output without materialising the state; full write-back once every L
// steps) and Implementation item 1 (per-row is_flush picks fold+write-back or
// output only).  The output formula is the recurrence unrolled over the ring
// window; see the contract in replayssm.h.
//
// Mapping: one workgroup per (row, head) tile of the [P, N] state, sized so
// that every lane streams 16 vectors of 16 bytes (a 16 KB bf16 tile is one
// wave).  The work is one memory round trip followed by arithmetic:
//  * row metadata arrives through scalar loads; then every global read of
//    the step is issued at once: the tile into registers (non-temporal), and
//    C, z and the w+1 ring rows of x and B straight into LDS with
//    global_load_lds (no registers, no conversion pass), and dt;
//  * decay weights come from a wave-wide suffix scan of dt; B_i.C from
//    16-lane dot products; both stay in lanes and are broadcast with
//    readlane, so there are no serial LDS loops;
//  * LPR = N / (elements per vector) adjacent lanes hold one state row; a
//    butterfly transpose leaves each lane with whole row sums;
//  * the flush branch depends only on the row, so it is uniform across the
//    workgroup: flush tiles fold the ring into their registers and store the
//    new state, the others only read;
//  * blockIdx is remapped so each XCD works on a contiguous range of rows.
#include "rssm_device.hpp"
#include "rssm_host.hpp"

namespace rssm {

struct Mamba2Args {
  void* state;
  void* x_ring;
  float* dt_ring;
  void* B_ring;
  const int32_t* slot_idx;
  const int32_t* write_pos;
  const uint8_t* is_flush;
  int32_t* next_write_pos;
  uint8_t* next_is_flush;
  const void* x;
  const void* dt;
  const float* A;
  const void* B;
  const void* C;
  const float* D;
  const void* z;
  const float* dt_bias;
  void* y;
  int32_t* status;
  int32_t nheads;
  int32_t ngroups;
  int32_t hpg;  // heads per group
  int32_t ring_len;
  int32_t num_slots;
  int32_t dt_softplus;
};

// Tile geometry: 16 state vectors per lane where the tile allows it.
template <typename ST, int P, int N>
struct TileShape {
  static constexpr int SV = Elt<ST>::kPer16;  // state elements per vector
  static constexpr int LPR = N / SV;          // lanes per state row
  static constexpr int NVEC = P * N / SV;     // vectors per tile
  static constexpr int NT =
      NVEC / 16 < 64 ? 64 : (NVEC / 16 > 512 ? 512 : NVEC / 16);  // threads
  static constexpr int ITEMS = NVEC / NT;     // vectors per lane
  static constexpr int RPI = NT / LPR;        // state rows per item
  static_assert(LPR >= 1 && LPR <= 64 && 64 % LPR == 0, "a state row must fit one wave");
  static_assert(NT % 64 == 0 && NVEC % NT == 0, "whole waves, whole tile");
};

// LDS staging: 16-byte chunks [C | z | x rows 0..w | B rows 0..w], raw.
template <typename IT, int P, int N>
struct Stage {
  static constexpr int IV = Elt<IT>::kPer16;
  static constexpr int XV = P / IV;  // chunks per x row
  static constexpr int BV = N / IV;  // chunks per B / C row
  static_assert(P % IV == 0 && N % IV == 0, "rows are whole chunks");
  // ring rows are allocated in multiples of 8 (the dot-product passes)
  static constexpr int chunks(int L) { return BV + XV + ((L + 7) & ~7) * (XV + BV); }
};

template <typename ST, typename IT, typename OT, int P, int N, bool REPLAY>
__global__ void __launch_bounds__((TileShape<ST, P, N>::NT))
    mamba2_decode_kernel(const Mamba2Args a) {
  using TS = TileShape<ST, P, N>;
  using SG = Stage<IT, P, N>;
  constexpr int SV = TS::SV, LPR = TS::LPR, NT = TS::NT, ITEMS = TS::ITEMS, RPI = TS::RPI;
  constexpr int XV = SG::XV, BV = SG::BV;
  constexpr long kSt = sizeof(ST);
  constexpr long kIo = sizeof(IT);

  extern __shared__ __attribute__((aligned(16))) char lds[];

  const int L = REPLAY ? a.ring_len : 1;
  const int H = a.nheads;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int b = tile / H;
  const int h = tile - b * H;
  const int g = h / a.hpg;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ---- row metadata (uniform across the workgroup)
  const int s = a.slot_idx[b];
  int w = 0;
  bool f = true;
  int st = 0;
  if (REPLAY) {
    w = a.write_pos[b];
    f = a.is_flush[b] != 0;
    if (w < 0 || w >= L) {
      st |= RSSM_ST_BAD_WRITE_POS;
      w = w < 0 ? 0 : L - 1;
      f = true;
    }
    if (w == L - 1 && !f) {
      st |= RSSM_ST_RING_OVERFLOW;
      f = true;
    }
  }
  const bool bad_slot = s < 0 || s >= a.num_slots;
  if (bad_slot) st |= RSSM_ST_BAD_SLOT;
  if (h == 0 && tid == 0) {
    if (REPLAY) {
      const int nw = (f || bad_slot) ? 0 : w + 1;
      if (a.next_write_pos) a.next_write_pos[b] = nw;
      if (a.next_is_flush) a.next_is_flush[b] = (nw == L - 1) ? 1 : 0;
    }
    if (st && a.status) atomicOr(a.status, st);
  }
  const long yoff = ((long)b * H + h) * P;
  if (bad_slot) {
    for (int p = tid; p < P; p += NT) Elt<OT>::store1(a.y, yoff + p, __builtin_nanf(""));
    return;
  }

  // ---- 1. issue every global read of the step
  const long tile_byte = ((long)s * H + h) * (long)P * N * kSt;
  u32x4 sv[ITEMS];
#pragma unroll
  for (int it = 0; it < ITEMS; ++it)
    sv[it] = ld16_stream(a.state, tile_byte + ((long)it * NT + tid) * 16);

  const long xcur = yoff;                                // x[b, h, :]
  const long bccur = ((long)b * a.ngroups + g) * N;      // B, C[b, g, :]
  const long xring0 = ((long)s * H + h) * (long)L * P;   // x_ring[s, h, 0, :]
  const long bring0 = ((long)s * a.ngroups + g) * (long)L * N;
  const int nZ = a.z ? XV : 0;
  const int oX = BV + nZ;                // first chunk of the x rows
  const int oB = oX + (w + 1) * XV;      // first chunk of the B rows
  const int nAll = oB + (w + 1) * BV;
  for (int k = 0; k * NT < nAll; ++k) {
    const int u = k * NT + tid;
    if (u < nAll) {
      const char* src;
      if (u < BV) {
        src = (const char*)a.C + (bccur * kIo + (long)u * 16);
      } else if (u < oX) {
        src = (const char*)a.z + (xcur * kIo + (long)(u - BV) * 16);
      } else if (u < oB) {
        const int i = (u - oX) / XV, c = (u - oX) - i * XV;
        src = (REPLAY && i < w) ? (const char*)a.x_ring + ((xring0 + (long)i * P) * kIo + c * 16)
                                : (const char*)a.x + (xcur * kIo + c * 16);
      } else {
        const int i = (u - oB) / BV, c = (u - oB) - i * BV;
        src = (REPLAY && i < w) ? (const char*)a.B_ring + ((bring0 + (long)i * N) * kIo + c * 16)
                                : (const char*)a.B + (bccur * kIo + c * 16);
      }
      dma16(src, lds + ((long)k * NT + wave * 64) * 16);
    }
  }
  // dt of entries 0..w: lane i < w from the ring, lane w the current step
  const long dtring0 = ((long)s * H + h) * L;
  float dti = 0.f;
  if (REPLAY && lane < w) dti = a.dt_ring[dtring0 + lane];
  const float Ah = a.A[h];
  const float Dh = a.D ? a.D[h] : 0.f;
  {
    const float v = Elt<IT>::load1(a.dt, (long)b * H + h) + (a.dt_bias ? a.dt_bias[h] : 0.f);
    const float dcur = a.dt_softplus ? softplus_f32(v) : v;
    if (lane == w) dti = dcur;
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const char* Cs = lds;
  const char* zs = lds + BV * 16;
  const char* xs = lds + oX * 16;
  const char* Bs = lds + (long)oB * 16;

  // ---- 2. append the current step to the ring (output-only rows)
  const bool append = REPLAY && !f;
  if (append && wave == 0) {
    const bool b_writer = (h % a.hpg) == 0;  // one writer per group
    for (int k = lane; k < XV + BV; k += 64) {
      if (k < XV) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(xs + ((long)w * XV + k) * 16);
        st16(a.x_ring, ((xring0 + (long)w * P) * kIo) + k * 16, v);
      } else if (b_writer) {
        const int cb = k - XV;
        const u32x4 v = *reinterpret_cast<const u32x4*>(Bs + ((long)w * BV + cb) * 16);
        st16(a.B_ring, ((bring0 + (long)w * N) * kIo) + cb * 16, v);
      }
    }
    if (lane == w) a.dt_ring[dtring0 + w] = dti;
  }

  // ---- 3. decay weights: wt_i = dt_i * exp(A * sum_{i<j<=w} dt_j)
  const float rsuf = L <= 16 ? row16_suffix_exclusive(dti) : wave_suffix_exclusive(dti, lane);
  const float cumdecay = expf(Ah * lane_value(dti + rsuf, 0));
  const float wt = lane <= w ? dti * expf(Ah * rsuf) : 0.f;

  // C segment of this lane's state columns
  const int c = tid % LPR;
  float cseg[SV];
  LdsRead<IT>::template seg<SV>(Cs, c * SV, cseg);

  float part[ITEMS];
  float coef = 0.f;  // lane i: wt_i * (B_i . C) on output-only rows
  if (!f) {
    // ---- 4a. B_i . C: 8 lanes per dot, 8 dots per pass
    constexpr int EPL = N / 8;
    const int q8 = lane & 7;
    float cpart[EPL];
    LdsRead<IT>::template seg<EPL>(Cs, q8 * EPL, cpart);
    float bc = 0.f;
#pragma unroll 2
    for (int q = 0; q * 8 <= w; ++q) {
      const int i = q * 8 + (lane >> 3);
      float bv[EPL];
      LdsRead<IT>::template seg<EPL>(Bs, i * N + q8 * EPL, bv);
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc = fmaf(bv[e], cpart[e], acc);
      acc = group_sum<8>(acc);
      const float t = __shfl(acc, (lane & 7) * 8, 64);
      if ((lane >> 3) == q) bc = t;
    }
    coef = lane <= w ? wt * bc : 0.f;
    // ---- 5a. S0 @ C per state row
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      float sf[SV];
      Elt<ST>::unpack(sv[it], sf);
      float d = 0.f;
#pragma unroll
      for (int j = 0; j < SV; ++j) d = fmaf(sf[j], cseg[j], d);
      part[it] = d;
    }
  } else {
    // ---- 5b. fold: S_new = cumdecay * S0 + sum_i wt_i * outer(x_i, B_i)
    constexpr int IC = ITEMS < 4 ? ITEMS : 4;  // items folded together
    const int prow = tid / LPR;
#pragma unroll
    for (int i0 = 0; i0 < ITEMS; i0 += IC) {
      float sf[IC][SV];
#pragma unroll
      for (int q = 0; q < IC; ++q) {
        Elt<ST>::unpack(sv[i0 + q], sf[q]);
#pragma unroll
        for (int j = 0; j < SV; ++j) sf[q][j] *= cumdecay;
      }
      // entries in groups of 4; past w the weight is 0 and the row index is
      // clamped to w, so the extra terms add exact zeros
      for (int ib = 0; ib <= w; ib += 4) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int i = ib + k;
          const int ic = i <= w ? i : w;
          const float wi = lane_value(wt, i);
          float bseg[SV];
          LdsRead<IT>::template seg<SV>(Bs, ic * N + c * SV, bseg);
#pragma unroll
          for (int q = 0; q < IC; ++q) {
            const int p = (i0 + q) * RPI + prow;
            const float cf = wi * LdsRead<IT>::one(xs, ic * P + p);
#pragma unroll
            for (int j = 0; j < SV; ++j) sf[q][j] = fmaf(cf, bseg[j], sf[q][j]);
          }
        }
      }
#pragma unroll
      for (int q = 0; q < IC; ++q) {
        float d = 0.f;
#pragma unroll
        for (int j = 0; j < SV; ++j) d = fmaf(sf[q][j], cseg[j], d);
        part[i0 + q] = d;
        st16_stream(a.state, tile_byte + ((long)(i0 + q) * NT + tid) * 16, Elt<ST>::pack(sf[q]));
      }
    }
  }

  // ---- 6. whole rows per lane; reconstruction, D*x, gate, store
  using RR = RowReduce<ITEMS, LPR>;
  RR::run(part, tid);
  const bool writer = (c % RR::DUP) == 0;
  const int prow = tid / LPR;
#pragma unroll
  for (int j = 0; j < RR::NF; ++j) {
    const int p = RR::item(j, tid) * RPI + prow;
    float yv = part[j];
    if (!f) {
      // coef is 0 past w; row indexes are clamped to w
      yv *= cumdecay;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        yv = fmaf(lane_value(coef, i), LdsRead<IT>::one(xs, (i <= w ? i : w) * P + p), yv);
      for (int i = 16; i <= w; ++i)
        yv = fmaf(lane_value(coef, i), LdsRead<IT>::one(xs, i * P + p), yv);
    }
    yv = fmaf(Dh, LdsRead<IT>::one(xs, w * P + p), yv);
    if (a.z) yv = silu_gate(yv, LdsRead<IT>::one(zs, p));
    if (writer) Elt<OT>::store1(a.y, yoff + p, yv);
  }
}

template <typename ST, typename IT, typename OT, int P, int N, bool REPLAY>
static int launch_mamba2(const Mamba2Args& a, int batch, hipStream_t stream) {
  using TS = TileShape<ST, P, N>;
  const int L = REPLAY ? a.ring_len : 1;  // L <= 64: one dt per lane of a wave
  const size_t lds = (size_t)Stage<IT, P, N>::chunks(L) * 16;
  if (lds > kMaxLds) return RSSM_ESHAPE;  // ring rows must fit one workgroup's LDS
  const long grid = (long)batch * a.nheads;
  return launch_kernel(
      reinterpret_cast<const void*>(&mamba2_decode_kernel<ST, IT, OT, P, N, REPLAY>),
      (unsigned)grid, TS::NT, lds, stream, a);
}

template <bool REPLAY, typename ST, typename IT, typename OT>
static int dispatch_shape(const Mamba2Args& a, const rssm_dims& d, hipStream_t s) {
#define RSSM_SHAPE(PP, NN) \
  if (d.headdim == PP && d.dstate == NN) return launch_mamba2<ST, IT, OT, PP, NN, REPLAY>(a, d.batch, s);
  RSSM_SHAPE(64, 128)
  RSSM_SHAPE(64, 16)
  RSSM_SHAPE(64, 32)
  RSSM_SHAPE(64, 64)
  RSSM_SHAPE(64, 256)
  RSSM_SHAPE(32, 16)
  RSSM_SHAPE(32, 32)
  RSSM_SHAPE(32, 64)
  RSSM_SHAPE(32, 128)
  RSSM_SHAPE(32, 256)
  RSSM_SHAPE(128, 16)
  RSSM_SHAPE(128, 32)
  RSSM_SHAPE(128, 64)
  RSSM_SHAPE(128, 128)
  RSSM_SHAPE(128, 256)
#undef RSSM_SHAPE
  return RSSM_ESHAPE;
}

template <bool REPLAY>
static int dispatch_mamba2(const Mamba2Args& a, const rssm_dims& d, hipStream_t s) {
  const int key = d.state_dtype * 4 + d.io_dtype * 2 + d.out_dtype;
  switch (key) {
    case 0: return dispatch_shape<REPLAY, float, float, float>(a, d, s);
    case 1: return dispatch_shape<REPLAY, float, float, bf16>(a, d, s);
    case 2: return dispatch_shape<REPLAY, float, bf16, float>(a, d, s);
    case 3: return dispatch_shape<REPLAY, float, bf16, bf16>(a, d, s);
    case 4: return dispatch_shape<REPLAY, bf16, float, float>(a, d, s);
    case 5: return dispatch_shape<REPLAY, bf16, float, bf16>(a, d, s);
    case 6: return dispatch_shape<REPLAY, bf16, bf16, float>(a, d, s);
    case 7: return dispatch_shape<REPLAY, bf16, bf16, bf16>(a, d, s);
  }
  return RSSM_EDTYPE;
}

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
  return RSSM_OK;
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
  return dispatch_mamba2<false>(a, *dims, stream);
}

extern "C" int replayssm_decode(const rssm_dims* dims, void* state, void* x_ring, float* dt_ring,
                                void* B_ring, const int32_t* slot_idx, const int32_t* write_pos,
                                const uint8_t* is_flush, int32_t* next_write_pos,
                                uint8_t* next_is_flush, const void* x, const void* dt,
                                const float* A, const void* B, const void* C, const float* D,
                                const void* z, const float* dt_bias, void* y, int32_t* status,
                                hipStream_t stream) {
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
  return dispatch_mamba2<true>(a, *dims, stream);
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

extern "C" int replayssm_abi_version(void) { return 100; }
