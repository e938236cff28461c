// Pieces shared by the GDN kernels (decode and speculative verify): tile
// geometry of the [V, K] fp32 state and 16-lane dot products of staged rows.
#pragma once

#include "rssm_device.hpp"

namespace rssm {

template <int V, int K, bool REPLAY>
struct GdnShape {
  static constexpr int SV = 4;               // fp32 state elements per vector
  static constexpr int LPR = K / SV;         // lanes per state row
  static constexpr int NVEC = V * K / SV;
  static constexpr int PER = REPLAY ? 16 : 8;
  static constexpr int NT0 = NVEC / PER;
  static constexpr int NT = NT0 < 64 ? 64 : (NT0 > 1024 ? 1024 : NT0);
  static constexpr int ITEMS = NVEC / NT;
  static constexpr int RPI = NT / LPR;
  static constexpr int IC = ITEMS < 8 ? ITEMS : 8;  // fold chunk: 32 accumulators
  static_assert(LPR <= 64 && 64 % LPR == 0, "a state row must fit one wave");
  static_assert(NT % 64 == 0 && NVEC % NT == 0 && ITEMS % IC == 0, "tiling");
};

// Dot products of a 16-lane share of two bf16/fp32 vectors held in LDS.
template <typename IT, int EPL>
struct SegDot {
  static constexpr bool kPacked = std::is_same<IT, bf16>::value && EPL % 2 == 0;
  uint32_t pk[kPacked ? EPL / 2 : 1];
  float fv[kPacked ? 1 : EPL];
  __device__ inline void load(const char* base, int e0) {
    if constexpr (kPacked) {
      const uint32_t* q = reinterpret_cast<const uint32_t*>(base + 2 * e0);
#pragma unroll
      for (int k = 0; k < EPL / 2; ++k) pk[k] = q[k];
    } else {
      LdsRead<IT>::template seg<EPL>(base, e0, fv);
    }
  }
  __device__ inline float dot(const SegDot& o) const {
    float d = 0.f;
    if constexpr (kPacked) {
#pragma unroll
      for (int k = 0; k < EPL / 2; ++k) {
        const uint32_t x = pk[k], y = o.pk[k];  // scalars first: see RowDot
        d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x),
                                            __builtin_bit_cast(bf16x2_t, y), d, false);
      }
    } else {
#pragma unroll
      for (int k = 0; k < EPL; ++k) d = fmaf(fv[k], o.fv[k], d);
    }
    return d;
  }
};

}  // namespace rssm
