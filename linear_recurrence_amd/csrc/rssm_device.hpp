// Device helpers shared by the decode kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rssm {

// Raw 16-byte vector: the unit of every coalesced global load and store.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// bf16 storage is carried as its 16-bit pattern.
struct bf16 {
  uint16_t bits;
};
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <typename T> struct Elt;

template <> struct Elt<float> {
  static constexpr int kPer16 = 4;  // elements per 16-byte vector
  __device__ static inline void unpack(const u32x4& v, float* f) {
#pragma unroll
    for (int k = 0; k < 4; ++k) f[k] = __uint_as_float(v[k]);
  }
  __device__ static inline u32x4 pack(const float* f) {
    u32x4 v;
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = __float_as_uint(f[k]);
    return v;
  }
  __device__ static inline float load1(const void* p, long i) {
    return static_cast<const float*>(p)[i];
  }
  __device__ static inline void store1(void* p, long i, float f) {
    static_cast<float*>(p)[i] = f;
  }
};

// fp32 -> bf16 rounds to nearest even: clang lowers the __bf16 conversion to
// the gfx950 hardware convert, which rounds per the default (RNE) mode.
__device__ static inline uint32_t bf16_pair(float lo, float hi) {
  const __bf16 a = static_cast<__bf16>(lo);
  const __bf16 b = static_cast<__bf16>(hi);
  return uint32_t(__builtin_bit_cast(uint16_t, a)) |
         (uint32_t(__builtin_bit_cast(uint16_t, b)) << 16);
}

template <> struct Elt<bf16> {
  static constexpr int kPer16 = 8;
  __device__ static inline void unpack(const u32x4& v, float* f) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      f[2 * k] = __uint_as_float(v[k] << 16);
      f[2 * k + 1] = __uint_as_float(v[k] & 0xffff0000u);
    }
  }
  __device__ static inline u32x4 pack(const float* f) {
    u32x4 v;
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = bf16_pair(f[2 * k], f[2 * k + 1]);
    return v;
  }
  __device__ static inline float load1(const void* p, long i) {
    return __uint_as_float(uint32_t(static_cast<const uint16_t*>(p)[i]) << 16);
  }
  __device__ static inline void store1(void* p, long i, float f) {
    const __bf16 b = static_cast<__bf16>(f);
    static_cast<uint16_t*>(p)[i] = __builtin_bit_cast(uint16_t, b);
  }
};

__device__ static inline u32x4 ld16(const void* base, long byte_off) {
  return *reinterpret_cast<const u32x4*>(static_cast<const char*>(base) + byte_off);
}

// Streamed once per step (no reuse within the step): non-temporal hint.
__device__ static inline u32x4 ld16_stream(const void* base, long byte_off) {
  return __builtin_nontemporal_load(
      reinterpret_cast<const u32x4*>(static_cast<const char*>(base) + byte_off));
}

__device__ static inline void st16(void* base, long byte_off, const u32x4& v) {
  *reinterpret_cast<u32x4*>(static_cast<char*>(base) + byte_off) = v;
}

__device__ static inline void st16_stream(void* base, long byte_off, const u32x4& v) {
  __builtin_nontemporal_store(
      v, reinterpret_cast<u32x4*>(static_cast<char*>(base) + byte_off));
}

// Raw buffer loads from one state tile: the descriptor (uniform base, size
// in bytes) lives in SGPRs, a lane needs one VGPR offset for all of its
// vectors and the per-vector offset goes in an SGPR.  Loads at or past
// `bytes` read 0 (hardware range check).  Word 3 is the gfx9-family value
// for raw (unformatted) buffers; aux 2 = non-temporal.  Stores stay global:
// with an SGPR offset, a buffer store's data registers must not be
// rewritten by the next VALU instruction, a hazard the compiler does not
// guard for that form.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ static inline rsrc_t tile_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ static inline u32x4 bload16_nt(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2);
}

// Sum over aligned groups of W consecutive lanes (W a power of two <= 64);
// every lane of the group receives the total.
template <int W>
__device__ static inline float group_sum(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Workgroups are handed to the 8 XCDs round-robin by workgroup id.  Remap so
// that each XCD receives one contiguous range of logical tiles: all heads of
// a batch row then share one XCD's L2 for the row's inputs and ring.
__device__ static inline int xcd_tile(int bid, int nblocks) {
  constexpr int kXcd = 8;
  const int xcd = bid % kXcd;
  const int local = bid / kXcd;
  const int q = nblocks / kXcd;
  const int r = nblocks % kXcd;
  return xcd * q + (xcd < r ? xcd : r) + local;
}

// Row metadata of a replay tile, its rows visited flush rows first.  Tiles of
// flush rows (state read, fold, state write) take several times longer than
// output-only tiles and are the only ones that write the state; within each
// aligned group of 64 batch rows the flush rows take the lowest ranks, so they
// are dispatched first (longest jobs first) and the state writes of a launch
// are issued together instead of spread through its read stream.  The map
// rank -> row is a bijection for any batch.  One round trip: every lane
// loads one row's (slot, write_pos, is_flush) and the wave picks its row by
// ballots; the result is uniform.
struct RowPick {
  int b, s, w;
  bool f;
};
__device__ static inline RowPick flush_first_pick(int rank, int nb, const int32_t* slot_idx,
                                                  const int32_t* write_pos,
                                                  const uint8_t* is_flush, int lane) {
  const int g0 = rank & ~63;
  const int n = nb - g0 < 64 ? nb - g0 : 64;
  const int rloc = rank - g0;  // < n
  const bool valid = lane < n;
  int sl = 0, wl = 0;
  bool fl = false;
  if (valid) {
    sl = slot_idx[g0 + lane];
    wl = write_pos[g0 + lane];
    fl = is_flush[g0 + lane] != 0;
  }
  const uint64_t fm = __ballot(fl);
  const uint64_t om = __ballot(valid && !fl);
  const int nf = __popcll(fm);
  const uint64_t m = rloc < nf ? fm : om;        // rows of the wanted kind
  const int r = rloc < nf ? rloc : rloc - nf;  // < popcount(m): exactly one lane matches
  const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                              __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
  const uint64_t hit = __ballot(((m >> lane) & 1) && below == r);
  const int j = __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit));
  return {g0 + j, __builtin_amdgcn_readlane(sl, j), __builtin_amdgcn_readlane(wl, j),
          ((fm >> j) & 1) != 0};
}

// Value of v held by lane `lane` (uniform index), broadcast to the wave.
__device__ static inline float lane_value(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Exclusive suffix sum across the wave: lane i receives sum_{j>i} v_j.
__device__ static inline float wave_suffix_exclusive(float v, int lane) {
  float r = __shfl_down(v, 1, 64);
  if (lane == 63) r = 0.f;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float t = __shfl_down(r, o, 64);
    if (lane + o < 64) r += t;
  }
  return r;
}

// Row shift within rows of 16 lanes (DPP): lane i receives lane i+K of its
// row, 0 past the end of the row.
template <int K>
__device__ static inline float row_shl(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x100 + K, 0xF, 0xF, true));
}

// Exclusive suffix sum over lanes 0..15 (values in lanes > 15 ignored):
// lane i < 16 receives sum_{i<j<16} v_j.  Five DPP adds.
__device__ static inline float row16_suffix_exclusive(float v) {
  float r = row_shl<1>(v);
  r += row_shl<1>(r);
  r += row_shl<2>(r);
  r += row_shl<4>(r);
  r += row_shl<8>(r);
  return r;
}

// Row shift within rows of 16 lanes (DPP) where lanes past the end of the
// row keep `fill`.
template <int K>
__device__ static inline float row_shl_fill(float v, float fill) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(fill), __float_as_int(v),
                                                    0x100 + K, 0xF, 0xF, false));
}

// Exclusive suffix product over lanes 0..15: lane i < 16 receives
// prod_{i<j<16} v_j (1 for lane 15).
__device__ static inline float row16_suffix_product_exclusive(float v) {
  float r = row_shl_fill<1>(v, 1.f);
  r *= row_shl_fill<1>(r, 1.f);
  r *= row_shl_fill<2>(r, 1.f);
  r *= row_shl_fill<4>(r, 1.f);
  r *= row_shl_fill<8>(r, 1.f);
  return r;
}

// Exclusive suffix product across the wave: lane i receives prod_{j>i} v_j.
__device__ static inline float wave_suffix_product_exclusive(float v, int lane) {
  float r = __shfl_down(v, 1, 64);
  if (lane == 63) r = 1.f;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float t = __shfl_down(r, o, 64);
    if (lane + o < 64) r *= t;
  }
  return r;
}

// Row reduction of ITEMS partial sums spread over LPR adjacent lanes, as a
// butterfly transpose: at each level a lane keeps half of its values and
// trades the other half with its partner, so log2(LPR) levels move
// ITEMS-1 values per lane instead of ITEMS*log2(LPR).  Afterwards a lane
// holds NF = ITEMS >> LV complete row sums (value j is item item(j, lane));
// when LPR > ITEMS, DUP adjacent lanes hold the same sums.
template <int ITEMS, int LPR>
struct RowReduce {
  static constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }
  static constexpr int K = ilog2(LPR);
  static constexpr int M = ilog2(ITEMS);
  static constexpr int LV = K < M ? K : M;
  static constexpr int NF = ITEMS >> LV;
  static constexpr int DUP = 1 << (K - LV);
  static_assert((1 << K) == LPR && (1 << M) == ITEMS, "powers of two");

  // One level per template instance, so every array index is a constant.
  template <int L>
  __device__ static inline void level(float (&v)[ITEMS], int lane) {
    if constexpr (L < LV) {
      constexpr int o = LPR >> (L + 1);
      constexpr int h = (ITEMS >> L) >> 1;
      const bool up = (lane & o) != 0;
#pragma unroll
      for (int j = 0; j < h; ++j) {
        const float send = up ? v[j] : v[j + h];
        const float keep = up ? v[j + h] : v[j];
        v[j] = keep + __shfl_xor(send, o, 64);
      }
      level<L + 1>(v, lane);
    } else if constexpr (L < K) {
      constexpr int o = LPR >> (L + 1);
#pragma unroll
      for (int j = 0; j < NF; ++j) v[j] += __shfl_xor(v[j], o, 64);
      level<L + 1>(v, lane);
    }
  }
  __device__ static inline void run(float (&v)[ITEMS], int lane) { level<0>(v, lane); }
  __device__ static inline int item(int j, int lane) {
    int it = j;
#pragma unroll
    for (int l = 0; l < LV; ++l)
      if (lane & (LPR >> (l + 1))) it += ITEMS >> (l + 1);
    return it;
  }
};

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from global memory straight into LDS (no VGPRs): lane l
// of the issuing wave writes lds_wave_base + 16*l.  The base must be uniform
// across the wave.  NT: the non-temporal policy (aux 2), for rows read once
// per step beside the state tile (the ring decode kernels' staging: measured
// faster there; rows that other workgroups of the launch read too stay
// temporal).
template <bool NT = false>
__device__ static inline void dma16(const void* gsrc, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (lds_void*)lds_wave_base, 16, 0, NT ? 2 : 0);
}

// Raw element reads from LDS, converted to fp32.
template <typename T> struct LdsRead;
template <> struct LdsRead<float> {
  __device__ static inline float one(const char* base, int i) {
    return reinterpret_cast<const float*>(base)[i];
  }
  // CNT consecutive elements starting at element i (i*4 bytes, 16B aligned
  // when CNT >= 4)
  template <int CNT>
  __device__ static inline void seg(const char* base, int i, float* out) {
    const float* p = reinterpret_cast<const float*>(base) + i;
#pragma unroll
    for (int k = 0; k < CNT; ++k) out[k] = p[k];
  }
};
template <> struct LdsRead<bf16> {
  __device__ static inline float one(const char* base, int i) {
    return __uint_as_float(uint32_t(reinterpret_cast<const uint16_t*>(base)[i]) << 16);
  }
  // CNT consecutive elements from element i; pairs are read as 32-bit words
  // (i even), a single element as 16 bits.
  template <int CNT>
  __device__ static inline void seg(const char* base, int i, float* out) {
    if constexpr (CNT % 2) {
#pragma unroll
      for (int k = 0; k < CNT; ++k) out[k] = one(base, i + k);
    } else {
      const uint32_t* p = reinterpret_cast<const uint32_t*>(base + 2 * i);
#pragma unroll
      for (int k = 0; k < CNT / 2; ++k) {
        out[2 * k] = __uint_as_float(p[k] << 16);
        out[2 * k + 1] = __uint_as_float(p[k] & 0xffff0000u);
      }
    }
  }
};

// Matrix-core product D = A*B + C, 16x16 outputs, K = 32 bf16 (gfx950).
// Lane l holds A[l%16][8*(l/16) + e] and B[8*(l/16) + e][l%16] (e = 0..7),
// and receives D[4*(l/16) + r][l%16] (r = 0..3).
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ static inline f32x4 mfma16x16x32_bf16(const u32x4& a, const u32x4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011): a counter-based generator.  Each of the ten
// rounds multiplies counter words 0 and 2 by the two round multipliers,
// permutes the words as the 4x64 variant prescribes (high halves xored with
// the other words and the key), and advances the key by the two Weyl
// constants.  c holds the counter on entry and the 256 random bits on exit.
__device__ static inline void philox4x64_10(uint64_t (&c)[4], uint64_t k0, uint64_t k1) {
  constexpr uint64_t kM0 = 0xD2E7470EE14C6C93ull, kM1 = 0xCA5A826395121157ull;
  constexpr uint64_t kW0 = 0x9E3779B97F4A7C15ull, kW1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t hi0 = __umul64hi(kM0, c[0]), lo0 = kM0 * c[0];
    const uint64_t hi1 = __umul64hi(kM1, c[2]), lo1 = kM1 * c[2];
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
    k0 += kW0;
    k1 += kW1;
  }
}

// fp32 -> bf16 by stochastic rounding with 16 random bits r: adding r below
// the kept 16 bits of the pattern carries into them with probability
// (dropped part) / 2^16, so the result rounds away from zero with exactly
// that probability (exact values are kept).  Inf and NaN keep the nearest
// (bit-preserving) conversion.
__device__ static inline uint32_t bf16_bits_sr(float f, uint32_t r) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u)
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
  return (u + (r & 0xffffu)) >> 16;
}

// Eight fp32 values -> one 16-byte bf16 vector, element j using bits
// 16*(j%4) .. of word j/4 of (w0, w1).
__device__ static inline u32x4 bf16_pack_sr(const float* f, uint64_t w0, uint64_t w1) {
  u32x4 v;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint64_t w = k < 2 ? w0 : w1;
    const uint32_t lo = bf16_bits_sr(f[2 * k], (uint32_t)(w >> (32 * (k & 1))));
    const uint32_t hi = bf16_bits_sr(f[2 * k + 1], (uint32_t)(w >> (32 * (k & 1) + 16)));
    v[k] = lo | (hi << 16);
  }
  return v;
}

// Value of a 64-bit register in the other lane of an adjacent pair
// (lane ^ 1), by DPP quad permutation [1, 0, 3, 2].
__device__ static inline uint64_t swap_lane_pair(uint64_t x) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)x, 0xB1, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(x >> 32), 0xB1, 0xF, 0xF, false);
  return (uint64_t)(uint32_t)lo | ((uint64_t)(uint32_t)hi << 32);
}

// softplus(v) = log(1 + e^v): v itself above 20 (exact in fp32).  log1p(e)
// uses Kahan's compensated form, as given in D. Goldberg, "What Every
// Computer Scientist Should Know About Floating-Point Arithmetic" (ACM
// Computing Surveys, 1991, Theorem 4): with u = 1 + e rounded, log1p(e) =
// log(u) * e / (u - 1), which cancels the rounding of u (u - 1 is exact;
// accurate to a few ulp with the hardware log and reciprocal), and e itself
// when u rounds to 1.
__device__ static inline float softplus_f32(float v) {
  if (v > 20.f) return v;
  const float e = expf(v);
  const float u = 1.f + e;
  return u == 1.f ? e : __logf(u) * (e * __builtin_amdgcn_rcpf(u - 1.f));
}

// y * z * sigmoid(z) with the hardware exp and reciprocal (about 2 ulp).
__device__ static inline float silu_gate(float y, float z) {
  return y * (z * __builtin_amdgcn_rcpf(1.f + __expf(-z)));
}

}  // namespace rssm
