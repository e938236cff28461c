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
//  * row metadata in one round trip (replay: the tile's rank picks a row,
//    flush rows first: for batches of up to 512 rows the batch's flush rows
//    are dealt evenly over the eight XCDs, otherwise each 64-row group's
//    flush rows come first); then every global read of
//    the step is issued at once: the tile into registers (non-temporal), and
//    C, z and the w+1 ring rows of x and B straight into LDS with
//    global_load_lds (no registers, no conversion pass), and dt;
//  * decay weights come from a suffix scan of dt across lanes (DPP within a
//    16-lane row, shuffles past 16 entries); B_i.C from 8-lane dot products;
//    the per-entry weights stay in lanes (readlane in the fold) or go
//    through a 64-float LDS array (output rows);
//  * LPR = N / (elements per vector) adjacent lanes hold one state row; a
//    butterfly transpose leaves each lane with whole row sums;
//  * the flush branch depends only on the row, so it is uniform across the
//    workgroup: flush tiles fold the ring into their registers in
//    double-buffered chunks and store the new state, the others only read;
//  * ring appends (x, B, dt of the current step) are not written by each
//    tile: the tiles of the first row of every 64-row group each append one
//    head for all rows of the group before their own work (group_appends);
//  * blockIdx is remapped so each XCD works on a contiguous range of rows.
#pragma once

#include "rssm_device.hpp"
#include "rssm_host.hpp"

namespace rssm {

// Row metadata of a replay tile when the host supplies the rows in
// flush-first order (row_order: a permutation of 0..nb-1 listing the flush
// rows first).  The positions of that list are dealt to the eight XCD rank
// ranges in turn, so each XCD receives an equal share of the flush rows and
// takes them first; with each aligned 64-row group taking only its own
// flush rows, the XCDs' shares vary from step to step and the launch waits
// for the one with the most.  The map rank -> position is a bijection for
// any batch, so any permutation gives the same results.  An entry outside
// [0, nb) is reported as RSSM_ST_BAD_ROW and returned as row -1: the tiles
// at that position then write nothing (no y, cursor or state), so a bad
// entry cannot make two workgroups fold the same checkpoint.  The row
// order and the row's metadata arrive by scalar loads.
typedef __attribute__((address_space(4))) const int32_t kconst_i32;

// Position in a flush-first row list dealt to the eight XCD rank ranges:
// ranks fill the residue classes of the positions mod 8 in turn, class x
// holding ranks [x*q + min(x, m), +q + (x < m)) and positions x, x+8, ...
// (a bijection between ranks and positions for any batch).
__device__ static inline int dealt_position(int rank, int nb) {
  const int q = nb >> 3, m = nb & 7;
  int x = 0;
#pragma unroll
  for (int c = 1; c < 8; ++c)
    if (rank >= c * q + (c < m ? c : m)) x = c;
  return (rank - (x * q + (x < m ? x : m))) * 8 + x;
}

__device__ static inline RowPick dealt_order_pick(int rank, int nb, const int32_t* row_order,
                                                  const int32_t* slot_idx,
                                                  const int32_t* write_pos,
                                                  const uint8_t* is_flush, int& st) {
  const int pos = dealt_position(rank, nb);
  const int b = *(kconst_i32*)(row_order + pos);
  if (b < 0 || b >= nb) {
    st |= RSSM_ST_BAD_ROW;
    return {-1, 0, 0, false};
  }
  return {b, *(kconst_i32*)(slot_idx + b), *(kconst_i32*)(write_pos + b), is_flush[b] != 0};
}

// The same dealing without a host list, for batches of at most 512 rows:
// every wave reads all the flush flags in one load (lane l holds rows
// 8l..8l+7, is_flush 8-byte aligned), ballots them into eight 64-bit masks
// and takes the row at its dealt position of the list "flush rows, then the
// others", each enumerated by (row % 8, row / 8); the row's slot and cursor
// follow by scalar loads.  Results do not depend on the order, so any
// enumeration serves; this one needs no cross-lane prefix sum.
__device__ static inline RowPick batch_dealt_pick(int rank, int nb, const int32_t* slot_idx,
                                                  const int32_t* write_pos,
                                                  const uint8_t* is_flush, int lane) {
  const int pos = dealt_position(rank, nb);
  const int r0 = 8 * lane;
  uint64_t f8 = 0;
  if (r0 + 8 <= nb) {
    f8 = *reinterpret_cast<const uint64_t*>(is_flush + r0);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (r0 + k < nb && is_flush[r0 + k]) f8 |= 1ull << (8 * k);
  }
  uint64_t fm[8], om[8];
  int nf = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const bool fk = ((f8 >> (8 * k)) & 0xff) != 0;
    fm[k] = __ballot(fk);
    om[k] = __ballot(!fk && r0 + k < nb);
    nf += __popcll(fm[k]);
  }
  const bool want_flush = pos < nf;
  int r = want_flush ? pos : pos - nf;  // rank among the rows of that kind
  int kk = 0;
  uint64_t msk = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint64_t mk = want_flush ? fm[k] : om[k];
    const int c = __popcll(mk);
    if (msk == 0) {
      if (r < c) {
        msk = mk;
        kk = k;
      } else {
        r -= c;
      }
    }
  }
  // the lane holding the r-th set bit of msk
  const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(msk >> 32),
                                              __builtin_amdgcn_mbcnt_lo((uint32_t)msk, 0));
  const uint64_t hit = __ballot(((msk >> lane) & 1) && below == r);
  const int b = 8 * __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit)) + kk;
  return {b, *(kconst_i32*)(slot_idx + b), *(kconst_i32*)(write_pos + b), want_flush};
}

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
  uint64_t sr_seed;    // stochastic rounding: Philox key (seed, offset)
  uint64_t sr_offset;
  const int32_t* row_order;  // flush-first row order from the host, or NULL
  int32_t batch_dealt;       // deal the batch's flush rows in the kernel (batch_dealt_pick)
};

// Tile geometry: PER target state vectors per lane.  The replay kernel
// streams 16 per lane where the tile allows it (its per-tile staging is
// amortised over more bytes) and 4 when the grid is too small to fill the
// GPU that way; the standard update, which also writes every tile, runs 4
// per lane (more waves in flight).
template <typename ST, int P, int N, int PER_>
struct TileShape {
  static constexpr int SV = Elt<ST>::kPer16;  // state elements per vector
  static constexpr int LPR = N / SV;          // lanes per state row
  static constexpr int NVEC = P * N / SV;     // vectors per tile
  static constexpr int PER = PER_;            // target vectors per lane
  static constexpr int NT0 = NVEC / PER;
  static constexpr int NT = NT0 < 64 ? 64 : (NT0 > 512 ? 512 : NT0);  // threads
  static constexpr int ITEMS = NVEC / NT;     // vectors per lane
  static constexpr int RPI = NT / LPR;        // state rows per item
  // vectors per fold chunk: 32 fp32 accumulators per lane at most (the small
  // replay grid halves this in the kernel, see kMinWaves)
  static constexpr int ICMAX = 32 / SV;
  static constexpr int IC = ITEMS < ICMAX ? ITEMS : ICMAX;
  static constexpr int NCH = ITEMS / IC;            // fold chunks
  static_assert(LPR >= 1 && LPR <= 64 && 64 % LPR == 0, "a state row must fit one wave");
  static_assert(NT % 64 == 0 && NVEC % NT == 0, "whole waves, whole tile");
  static_assert(ITEMS % IC == 0, "fold chunking");
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

// Dot product of SV state elements (one 16-byte vector) with the matching C
// elements held by the lane.  bf16 x bf16 uses the packed dot2 instruction
// (exact products, fp32 accumulation); otherwise unpack and fma.
template <typename ST, typename IT, int SV>
struct RowDot {
  static constexpr bool kPacked = std::is_same<ST, bf16>::value && std::is_same<IT, bf16>::value;
  // C held as fp32 (generic) or as packed bf16 pairs
  float cf[kPacked ? 1 : SV];
  uint32_t cp[kPacked ? SV / 2 : 1];
  __device__ inline void load(const char* Cs, int c) {
    if constexpr (kPacked) {
      const uint32_t* q = reinterpret_cast<const uint32_t*>(Cs + 2 * c * SV);
#pragma unroll
      for (int k = 0; k < SV / 2; ++k) cp[k] = q[k];
    } else {
      LdsRead<IT>::template seg<SV>(Cs, c * SV, cf);
    }
  }
  __device__ inline float dot(const u32x4& v) const {
    float d = 0.f;
    if constexpr (kPacked) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        // copy the element out first: a bit cast of an ext-vector element
        // expression reads element 0 whatever the index
        const uint32_t sk = v[k];
        const uint32_t ck = cp[k];
        d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, sk),
                                            __builtin_bit_cast(bf16x2_t, ck), d, false);
      }
    } else {
      float f[SV];
      Elt<ST>::unpack(v, f);
#pragma unroll
      for (int j = 0; j < SV; ++j) d = fmaf(f[j], cf[j], d);
    }
    return d;
  }
  // C as fp32, for the fold's dot with the new state
  __device__ inline void cvals(float* out) const {
    if constexpr (kPacked) {
#pragma unroll
      for (int k = 0; k < SV / 2; ++k) {
        out[2 * k] = __uint_as_float(cp[k] << 16);
        out[2 * k + 1] = __uint_as_float(cp[k] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int j = 0; j < SV; ++j) out[j] = cf[j];
    }
  }
};

// Fold one chunk of IC state vectors: S_new = cumdecay*S0 + sum_i wt_i x_i B_i
// for the rows and columns this lane holds; store it; write the row partial
// sums of S_new . C into part[I0 .. I0+IC).
// Stochastic rounding of the bf16 write-back.  The random bits of element
// e of a tile come from Philox4x64-10 with key (seed, offset) and counter
// (tile * (P*N/16) + e/16, 0, 0, 0), where tile = slot * nheads + head:
// element e uses bits 16*(e%4) .. of output word (e%16)/4.  One call covers
// 16 consecutive elements, i.e. the 16-byte vectors of two adjacent lanes.
struct SrCtx {
  uint64_t k0, k1;   // key
  uint64_t blk0;     // counter of the tile's first 16 elements
};

template <typename ST, int NT, int IC, int I0, bool SR>
__device__ __forceinline__ void store_chunk(float (&sf)[IC][Elt<ST>::kPer16], char* tile,
                                            uint32_t lane_off, const SrCtx& sr) {
  if constexpr (!SR) {
#pragma unroll
    for (int q = 0; q < IC; ++q)
      st16_stream(tile, (long)lane_off + (I0 + q) * NT * 16, Elt<ST>::pack(sf[q]));
  } else {
    static_assert(std::is_same<ST, bf16>::value, "stochastic rounding targets bf16 state");
    const int tid = threadIdx.x;
    const int par = tid & 1;  // vector v = item*NT + tid is half v%2 of block v/2
    if constexpr (IC % 2 == 0) {
      // lanes of a pair each draw one block: the even lane the block of item
      // q, the odd lane that of item q+1, and trade the halves they lack
#pragma unroll
      for (int q = 0; q < IC; q += 2) {
        uint64_t c[4] = {sr.blk0 + (uint64_t)((((I0 + q + par) * NT) + tid) >> 1), 0, 0, 0};
        philox4x64_10(c, sr.k0, sr.k1);
        const uint64_t keep0 = par ? c[2] : c[0], keep1 = par ? c[3] : c[1];
        const uint64_t got0 = swap_lane_pair(par ? c[0] : c[2]);
        const uint64_t got1 = swap_lane_pair(par ? c[1] : c[3]);
        const u32x4 va = par ? bf16_pack_sr(sf[q], got0, got1) : bf16_pack_sr(sf[q], keep0, keep1);
        const u32x4 vb =
            par ? bf16_pack_sr(sf[q + 1], keep0, keep1) : bf16_pack_sr(sf[q + 1], got0, got1);
        st16_stream(tile, (long)lane_off + (I0 + q) * NT * 16, va);
        st16_stream(tile, (long)lane_off + (I0 + q + 1) * NT * 16, vb);
      }
    } else {
#pragma unroll
      for (int q = 0; q < IC; ++q) {
        uint64_t c[4] = {sr.blk0 + (uint64_t)((((I0 + q) * NT) + tid) >> 1), 0, 0, 0};
        philox4x64_10(c, sr.k0, sr.k1);
        const u32x4 v = par ? bf16_pack_sr(sf[q], c[2], c[3]) : bf16_pack_sr(sf[q], c[0], c[1]);
        st16_stream(tile, (long)lane_off + (I0 + q) * NT * 16, v);
      }
    }
  }
}

template <typename ST, typename IT, int P, int N, int NT, int SV, int IC, int RPI, int ITEMS, int I0,
          bool SR>
__device__ __forceinline__ void fold_chunk(const u32x4 (&raw)[IC], float (&part)[ITEMS], int w,
                                           float wt, float cumdecay, const char* Bs,
                                           const char* xs, int c, int prow, const float* cv,
                                           char* tile, uint32_t lane_off, const SrCtx& sr) {
  float sf[IC][SV];
#pragma unroll
  for (int q = 0; q < IC; ++q)
#pragma unroll
    for (int j = 0; j < SV; ++j) sf[q][j] = 0.f;
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
        const int p = (I0 + q) * RPI + prow;
        const float cf = wi * LdsRead<IT>::one(xs, ic * P + p);
#pragma unroll
        for (int j = 0; j < SV; ++j) sf[q][j] = fmaf(cf, bseg[j], sf[q][j]);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < IC; ++q) {
    float s0[SV];
    Elt<ST>::unpack(raw[q], s0);
    float d = 0.f;
#pragma unroll
    for (int j = 0; j < SV; ++j) {
      sf[q][j] = fmaf(cumdecay, s0[j], sf[q][j]);
      d = fmaf(sf[q][j], cv[j], d);
    }
    // keep the row sum here: left alone, the compiler sinks it past the
    // later chunks and keeps every chunk's accumulators alive until the end
    asm volatile("" : "+v"(d));
    part[I0 + q] = d;
  }
  // Global (not buffer) stores: a buffer store with an SGPR offset whose
  // data registers are rewritten by the next VALU instruction can send the
  // new value on gfx950, and the compiler only guards the global form.
  store_chunk<ST, NT, IC, I0, SR>(sf, tile, lane_off, sr);
}

struct FoldCtx {
  int w;
  float wt, cumdecay;
  const char* Bs;
  const char* xs;
  int c, prow;
  rsrc_t trs;    // state tile, for the chunk loads
  char* tile;    // state tile, for the stores
  uint32_t lane_off;
  SrCtx sr;
};

// Fold chunks CH, CH+1, ... of the tile.  Chunks alternate between the two
// register buffers; once chunk CH is folded its buffer receives chunk CH+2,
// so one chunk is always in flight while another is folded.
template <typename ST, typename IT, int P, int N, int NT, int SV, int IC, int RPI, int ITEMS, int CH,
          bool SR>
__device__ __forceinline__ void fold_from(u32x4 (&ra)[IC], u32x4 (&rb)[IC], float (&part)[ITEMS],
                                          const float* cv, const FoldCtx& fc) {
  constexpr int NCH = ITEMS / IC;
  if constexpr (CH < NCH) {
    u32x4 (&buf)[IC] = (CH % 2 == 0) ? ra : rb;
    fold_chunk<ST, IT, P, N, NT, SV, IC, RPI, ITEMS, CH * IC, SR>(
        buf, part, fc.w, fc.wt, fc.cumdecay, fc.Bs, fc.xs, fc.c, fc.prow, cv, fc.tile,
        fc.lane_off, fc.sr);
    if constexpr (CH + 2 < NCH) {
#pragma unroll
      for (int q = 0; q < IC; ++q)
        buf[q] = bload16_nt(fc.trs, fc.lane_off, ((CH + 2) * IC + q) * NT * 16);
    }
    fold_from<ST, IT, P, N, NT, SV, IC, RPI, ITEMS, CH + 1, SR>(ra, rb, part, cv, fc);
  }
}

// Ring appends of head hh for every row of the 64-row group starting at g0
// (n rows): x[b, hh, :] and the step's dt go to ring position w of the row's
// slot, and B[b, g, :] too when hh is the first head of its group g.  A row
// appends only when it will not flush: is_flush = 0, 0 <= w <= L-2 and a
// slot in range, the rule the row's own tiles apply.  The tiles of each
// group's first row run this before their own work, so the launch issues its
// ring writes together near its start instead of one small write per tile
// spread through the read stream, where each costs far more than its bytes;
// the stores are non-temporal (measured: a third less cost inside the tile
// read stream than write-back stores).
template <typename IT, int P, int N, int NT>
__device__ __forceinline__ void group_appends(const Mamba2Args& a, int g0, int n, int hh, int L,
                                              int tid) {
  constexpr int XV = P / Elt<IT>::kPer16, BV = N / Elt<IT>::kPer16;
  constexpr int DEPTH = 8;  // vectors in flight per thread
  constexpr long kIo = sizeof(IT);
  const int lane = tid & 63;
  const int H = a.nheads;
  int sl = 0, wl = 0;
  bool app = false;
  if (lane < n) {
    sl = a.slot_idx[g0 + lane];
    wl = a.write_pos[g0 + lane];
    app = a.is_flush[g0 + lane] == 0 && wl >= 0 && wl <= L - 2 && sl >= 0 && sl < a.num_slots;
  }
  const uint64_t am = __ballot(app);  // every wave holds the whole group
  // copy rows of RV vectors: vector v of the batch is (row v / RV, chunk v % RV)
  auto copy_rows = [&](int RV, const char* src, long src_row, long src_off, char* dst,
                       long slot_mul, long dst_off, long row_bytes) {
    for (int v0 = 0; v0 < 64 * RV; v0 += NT * DEPTH) {
      u32x4 buf[DEPTH];
      long dofs[DEPTH];
      bool on[DEPTH];
#pragma unroll
      for (int q = 0; q < DEPTH; ++q) {
        const int v = v0 + q * NT + tid;
        const int r = (v / RV) & 63;
        const int sr = __shfl(sl, r, 64);
        const int wr = __shfl(wl, r, 64);
        on[q] = v < 64 * RV && ((am >> r) & 1);
        dofs[q] = ((long)sr * slot_mul + dst_off + wr) * row_bytes + (long)(v % RV) * 16;
        if (on[q]) buf[q] = ld16(src, (long)(g0 + r) * src_row + src_off + (long)(v % RV) * 16);
      }
#pragma unroll
      for (int q = 0; q < DEPTH; ++q)
        if (on[q]) st16_stream(dst, dofs[q], buf[q]);
    }
  };
  // x_ring[s, hh, w, :] <- x[b, hh, :]
  copy_rows(XV, (const char*)a.x, (long)H * P * kIo, (long)hh * P * kIo, (char*)a.x_ring,
            (long)H * L, (long)hh * L, P * kIo);
  if (hh % a.hpg == 0) {
    // B_ring[s, g, w, :] <- B[b, g, :]
    const int gg = hh / a.hpg;
    copy_rows(BV, (const char*)a.B, (long)a.ngroups * N * kIo, (long)gg * N * kIo,
              (char*)a.B_ring, (long)a.ngroups * L, (long)gg * L, N * kIo);
  }
  if (tid < 64 && app) {
    const float v = Elt<IT>::load1(a.dt, (long)(g0 + lane) * H + hh) + (a.dt_bias ? a.dt_bias[hh] : 0.f);
    __builtin_nontemporal_store(a.dt_softplus ? softplus_f32(v) : v,
                                &a.dt_ring[((long)sl * H + hh) * L + wl]);
  }
}

// Minimum waves per SIMD the compiler must fit.  A small replay grid (4
// vectors per lane) is about one round of resident waves, so occupancy, not
// bandwidth, bounds it: eight waves per SIMD where the registers allow it
// without spills (bf16 state and inputs, dstate <= 128); elsewhere the
// compiler's own choice.
template <typename ST, typename IT, int N, bool REPLAY, int PER>
constexpr int kMinWaves = (REPLAY && PER <= 4 && std::is_same<ST, bf16>::value &&
                           std::is_same<IT, bf16>::value && N <= 128)
                              ? 8
                              : 1;

template <typename ST, typename IT, typename OT, int P, int N, bool REPLAY, bool SR, int PER>
__global__ void __launch_bounds__((TileShape<ST, P, N, PER>::NT), (kMinWaves<ST, IT, N, REPLAY, PER>))
    mamba2_decode_kernel(const Mamba2Args a) {
  using TS = TileShape<ST, P, N, PER>;
  using SG = Stage<IT, P, N>;
  constexpr int SV = TS::SV, LPR = TS::LPR, NT = TS::NT, ITEMS = TS::ITEMS, RPI = TS::RPI;
  // the small replay grid folds in chunks of 16 accumulators per lane, which
  // fits its eight-waves register budget
  constexpr int ICK = (REPLAY && PER <= 4 ? 16 : 32) / SV;
  constexpr int IC = ITEMS < ICK ? ITEMS : ICK, NCH = ITEMS / IC;
  static_assert(ITEMS % IC == 0, "fold chunking");
  constexpr int XV = SG::XV, BV = SG::BV;
  constexpr long kSt = sizeof(ST);
  constexpr long kIo = sizeof(IT);

  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ __attribute__((aligned(16))) float coef_lds[NT];  // ring-term weights per wave

  const int L = REPLAY ? a.ring_len : 1;
  const int H = a.nheads;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rank = tile / H;  // row rank; replay visits flush rows first
  const int h = tile - rank * H;
  const int g = h / a.hpg;

  // ---- row metadata (uniform across the workgroup)
  int st = 0;
  RowPick pick{rank, 0, 0, true};
  if constexpr (REPLAY) {
    if (a.row_order)
      pick = dealt_order_pick(rank, gridDim.x / H, a.row_order, a.slot_idx, a.write_pos,
                              a.is_flush, st);
    else if (PER > 4 && a.batch_dealt)
      pick = batch_dealt_pick(rank, gridDim.x / H, a.slot_idx, a.write_pos, a.is_flush, lane);
    else
      pick = flush_first_pick(rank, gridDim.x / H, a.slot_idx, a.write_pos, a.is_flush, lane);
  } else {
    pick.s = a.slot_idx[rank];
  }
  const bool bad_row = pick.b < 0;  // a row order entry outside the batch
  const int b = pick.b;
  const int s = pick.s;
  int w = 0;
  bool f = true;
  if (REPLAY && !bad_row) {
    w = pick.w;
    f = pick.f;
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
  const bool bad_slot = !bad_row && (s < 0 || s >= a.num_slots);
  if (bad_slot) st |= RSSM_ST_BAD_SLOT;
  if (h == 0 && tid == 0) {
    if (REPLAY && !bad_row) {
      const int nw = (f || bad_slot) ? 0 : w + 1;
      if (a.next_write_pos) a.next_write_pos[b] = nw;
      if (a.next_is_flush) a.next_is_flush[b] = (nw == L - 1) ? 1 : 0;
    }
    if (st && a.status) atomicOr(a.status, st);
  }
  if (REPLAY && L > 1 && (rank & 63) == 0) {
    const int nb = gridDim.x / H;
    group_appends<IT, P, N, NT>(a, rank, nb - rank < 64 ? nb - rank : 64, h, L, tid);
  }
  if (bad_row) return;  // the group appends above are keyed by rank, not by row
  const long yoff = ((long)b * H + h) * P;
  if (bad_slot) {
    for (int p = tid; p < P; p += NT) Elt<OT>::store1(a.y, yoff + p, __builtin_nanf(""));
    return;
  }

  char* const tptr = (char*)a.state + ((long)s * H + h) * (long)P * N * kSt;
  const rsrc_t trs = tile_rsrc(tptr, (uint32_t)(P * N * kSt));
  const uint32_t lane_off = tid * 16;
  const long xcur = yoff;                                // x[b, h, :]
  const long bccur = ((long)b * a.ngroups + g) * N;      // B, C[b, g, :]
  const long xring0 = ((long)s * H + h) * (long)L * P;   // x_ring[s, h, 0, :]
  const long bring0 = ((long)s * a.ngroups + g) * (long)L * N;
  const long dtring0 = ((long)s * H + h) * L;
  const int nZ = a.z ? XV : 0;
  const int oX = BV + nZ;                // first chunk of the x rows
  const int oB = oX + (w + 1) * XV;      // first chunk of the B rows
  const int nAll = oB + (w + 1) * BV;

  // Stage C, z, x_0..x_w, B_0..B_w (entry w = the current step) into LDS
  // with direct-to-LDS loads, one contiguous global span at a time (the w
  // ring rows of a slot are contiguous), and load dt of entries 0..w (lane i).
  // span: LDS chunks [c0, c0+n); the first nring from `ring`, then `cur`.
  auto dma_span = [&](int c0, int n, const char* ring, int nring, const char* cur) {
    for (int j = wave * 64; j < n; j += NT) {
      const int u = j + lane;
      if (u < n) {
        const char* src = u < nring ? ring + (long)u * 16 : cur + (long)(u - nring) * 16;
        dma16<REPLAY>(src, lds + (long)(c0 + j) * 16);
      }
    }
  };
  auto stage = [&]() {
    if constexpr (!REPLAY) {
      // no ring: C, z, x, B are at most a few dozen chunks, one per lane
      for (int u = tid; u < nAll; u += NT) {
        const char* src;
        if (u < BV) src = (const char*)a.C + (bccur * kIo + (long)u * 16);
        else if (u < oX) src = (const char*)a.z + (xcur * kIo + (long)(u - BV) * 16);
        else if (u < oB) src = (const char*)a.x + (xcur * kIo + (long)(u - oX) * 16);
        else src = (const char*)a.B + (bccur * kIo + (long)(u - oB) * 16);
        dma16(src, lds + (long)(u - lane) * 16);
      }
      return;
    }
    const char* cg = (const char*)a.C + bccur * kIo;
    dma_span(0, BV, cg, BV, cg);
    if (a.z) {
      const char* zg = (const char*)a.z + xcur * kIo;
      dma_span(BV, XV, zg, XV, zg);
    }
    dma_span(oX, (w + 1) * XV, REPLAY ? (const char*)a.x_ring + xring0 * kIo : nullptr,
             REPLAY ? w * XV : 0, (const char*)a.x + xcur * kIo);
    dma_span(oB, (w + 1) * BV, REPLAY ? (const char*)a.B_ring + bring0 * kIo : nullptr,
             REPLAY ? w * BV : 0, (const char*)a.B + bccur * kIo);
  };
  // dt of entries 0..w (lane i): the loads are issued after the tile reads
  // (load_dt), the bias and softplus applied after the wait (finish_dt), so
  // no scalar round trip sits in front of the tile stream.
  float dti = 0.f, dtr = 0.f, dtb = 0.f;
  auto load_dt = [&]() {
    if (REPLAY && lane < w) dti = a.dt_ring[dtring0 + lane];
    dtr = Elt<IT>::load1(a.dt, (long)b * H + h);
    if (a.dt_bias) dtb = a.dt_bias[h];
  };
  auto finish_dt = [&]() {
    const float v = dtr + dtb;
    const float dcur = a.dt_softplus ? softplus_f32(v) : v;
    if (lane == w) dti = dcur;
  };
  const float Ah = a.A[h];
  const float Dh = a.D ? a.D[h] : 0.f;

  const char* Cs = lds;
  const char* zs = lds + BV * 16;
  const char* xs = lds + oX * 16;
  const char* Bs = lds + (long)oB * 16;
  const int c = tid % LPR;
  const int prow = tid / LPR;

  float part[ITEMS];
  float cumdecay, coef = 0.f;  // coef (lane i): wt_i * (B_i . C), output-only rows
  if (!f) {
    // ================= output-only tile: the whole tile in flight at once
    u32x4 sv[ITEMS];
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) sv[it] = bload16_nt(trs, lane_off, it * NT * 16);
    stage();
    load_dt();
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    finish_dt();
    // decay weights: wt_i = dt_i * exp(A * sum_{i<j<=w} dt_j)
    const float rsuf = L <= 16 ? row16_suffix_exclusive(dti) : wave_suffix_exclusive(dti, lane);
    cumdecay = expf(Ah * lane_value(dti + rsuf, 0));
    const float wt = lane <= w ? dti * expf(Ah * rsuf) : 0.f;
    // B_i . C: 8 lanes per dot, 8 dots per pass
    {
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
      coef_lds[wave * 64 + lane] = coef;  // broadcast to the wave through LDS
      __builtin_amdgcn_wave_barrier();
    }
    // S0 . C per state row
    RowDot<ST, IT, SV> rd;
    rd.load(Cs, c);
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) part[it] = rd.dot(sv[it]);
  } else {
    // ================= flush tile: stream the tile in chunks, fold, store
    u32x4 ra[IC], rb[IC];
#pragma unroll
    for (int q = 0; q < IC; ++q) ra[q] = bload16_nt(trs, lane_off, q * NT * 16);
    if constexpr (NCH > 1) {
#pragma unroll
      for (int q = 0; q < IC; ++q) rb[q] = bload16_nt(trs, lane_off, (IC + q) * NT * 16);
    }
    stage();
    load_dt();
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    finish_dt();
    const float rsuf = L <= 16 ? row16_suffix_exclusive(dti) : wave_suffix_exclusive(dti, lane);
    cumdecay = expf(Ah * lane_value(dti + rsuf, 0));
    const float wt = lane <= w ? dti * expf(Ah * rsuf) : 0.f;
    RowDot<ST, IT, SV> rd;
    rd.load(Cs, c);
    float cv[SV];
    rd.cvals(cv);
    SrCtx sr{a.sr_seed, a.sr_offset, ((uint64_t)s * H + h) * (uint64_t)(P * N / 16)};
    FoldCtx fc{w, wt, cumdecay, Bs, xs, c, prow, trs, tptr, lane_off, sr};
    fold_from<ST, IT, P, N, NT, SV, IC, RPI, ITEMS, 0, SR>(ra, rb, part, cv, fc);
  }

  // ---- whole rows per lane; ring term, D*x, gate, store
  using RR = RowReduce<ITEMS, LPR>;
  RR::run(part, tid);
  const bool writer = (c % RR::DUP) == 0;
#pragma unroll
  for (int j = 0; j < RR::NF; ++j) {
    const int p = RR::item(j, tid) * RPI + prow;
    float yv = part[j];
    if (!f) {
      // coef is 0 past w; row indexes are clamped to w
      yv *= cumdecay;
      const float* cw = coef_lds + wave * 64;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        yv = fmaf(cw[i], LdsRead<IT>::one(xs, (i <= w ? i : w) * P + p), yv);
      for (int i = 16; i <= w; ++i) yv = fmaf(cw[i], LdsRead<IT>::one(xs, i * P + p), yv);
    }
    yv = fmaf(Dh, LdsRead<IT>::one(xs, w * P + p), yv);
    if (a.z) yv = silu_gate(yv, LdsRead<IT>::one(zs, p));
    if (writer) Elt<OT>::store1(a.y, yoff + p, yv);
  }
}

template <typename ST, typename IT, typename OT, int P, int N, bool REPLAY, bool SR, int PER>
static int launch_mamba2(const Mamba2Args& a, int batch, hipStream_t stream) {
  using TS = TileShape<ST, P, N, PER>;
  const int L = REPLAY ? a.ring_len : 1;  // L <= 64: one dt per lane of a wave
  const size_t lds = (size_t)Stage<IT, P, N>::chunks(L) * 16;
  if (lds > kMaxLds) return RSSM_ESHAPE;  // ring rows must fit one workgroup's LDS
  const long grid = (long)batch * a.nheads;
  return launch_kernel(
      reinterpret_cast<const void*>(&mamba2_decode_kernel<ST, IT, OT, P, N, REPLAY, SR, PER>),
      (unsigned)grid, TS::NT, lds, stream, a);
}

template <bool REPLAY, bool SR, int PER, typename ST, typename IT, typename OT>
static int dispatch_shape(const Mamba2Args& a, const rssm_dims& d, hipStream_t s) {
#define RSSM_SHAPE(PP, NN) \
  if (d.headdim == PP && d.dstate == NN)    \
    return launch_mamba2<ST, IT, OT, PP, NN, REPLAY, SR, PER>(a, d.batch, s);
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

// Dispatch on the dtypes: all eight combinations with nearest rounding;
// stochastic rounding exists for the bf16 state pool only.
template <bool REPLAY, bool SR, int PER>
static int dispatch_mamba2(const Mamba2Args& a, const rssm_dims& d, hipStream_t s) {
  const int key = d.state_dtype * 4 + d.io_dtype * 2 + d.out_dtype;
  if constexpr (SR) {
    switch (key) {
      case 4: return dispatch_shape<REPLAY, true, PER, bf16, float, float>(a, d, s);
      case 5: return dispatch_shape<REPLAY, true, PER, bf16, float, bf16>(a, d, s);
      case 6: return dispatch_shape<REPLAY, true, PER, bf16, bf16, float>(a, d, s);
      case 7: return dispatch_shape<REPLAY, true, PER, bf16, bf16, bf16>(a, d, s);
    }
  } else {
    switch (key) {
      case 0: return dispatch_shape<REPLAY, false, PER, float, float, float>(a, d, s);
      case 1: return dispatch_shape<REPLAY, false, PER, float, float, bf16>(a, d, s);
      case 2: return dispatch_shape<REPLAY, false, PER, float, bf16, float>(a, d, s);
      case 3: return dispatch_shape<REPLAY, false, PER, float, bf16, bf16>(a, d, s);
      case 4: return dispatch_shape<REPLAY, false, PER, bf16, float, float>(a, d, s);
      case 5: return dispatch_shape<REPLAY, false, PER, bf16, float, bf16>(a, d, s);
      case 6: return dispatch_shape<REPLAY, false, PER, bf16, bf16, float>(a, d, s);
      case 7: return dispatch_shape<REPLAY, false, PER, bf16, bf16, bf16>(a, d, s);
    }
  }
  return RSSM_EDTYPE;
}

// Stochastic-rounding instances (mamba2_sr.hip).
int dispatch_mamba2_sr(bool replay, const Mamba2Args& a, const rssm_dims& d, hipStream_t s);
// Replay instances with 4 vectors per lane, for grids too small to fill the
// GPU with 16 (mamba2_small.hip).
int dispatch_mamba2_small(const Mamba2Args& a, const rssm_dims& d, hipStream_t s);

}  // namespace rssm
