// Gated-delta-rule (GDN) decode kernels for gfx950: the recurrent update and
// the ReplaySSM ring decode (checkpoint S0 + ring of (d, k, g), fold on flush
// rows only).
//
// Method: sglang #28451 (GDN/KDA ReplaySSM decode) - Motivation (GDN decode
// reads and writes the full [HV, V, K] state every step and is bandwidth
// bound at large batch) and Implementation item 1 (non-flush steps rebuild
// the output from S0 plus the ring; the state is refreshed every L steps);
// the ring contents d [L, V], k [L, K], g [L] per slot follow the memory-pool
// snippet of sglang #28695 "[GDN] Support ReplaySSM Ring Spec-Verify".
// Formulas: see the contract in replayssm.h.
//
// Mapping (one workgroup per (row, value head) tile of the [V, K] state):
// the tile is streamed with 16-byte non-temporal loads into registers; LPR
// consecutive lanes hold one state row and reduce S0 @ k and S0 @ q over K
// with xor shuffles.  The ring rows, q, v and the gates are staged in LDS.
// The contractions here are two matrix-vector products and, on flush rows,
// a rank-(w+1) update with w+1 <= L: too thin for the matrix cores to pay,
// and the kernel is bound by the state stream, so they run on the VALU.
#include <math.h>

#include "rssm_device.hpp"
#include "rssm_host.hpp"

namespace rssm {

struct GdnArgs {
  float* state;
  float* d_ring;
  void* k_ring;
  float* g_ring;
  const int32_t* slot_idx;
  const int32_t* write_pos;
  const uint8_t* is_flush;
  int32_t* next_write_pos;
  uint8_t* next_is_flush;
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  void* o;
  int32_t* status;
  int32_t k_heads;
  int32_t v_heads;
  int32_t vpk;  // value heads per key head
  int32_t ring_len;
  int32_t num_slots;
  float scale;
};

template <int V, int K>
__host__ __device__ constexpr int gdn_lds_floats(int L) {
  return L * K + L * V + K + V + 4 * L + 4;
}

template <typename IT, typename OT, int V, int K, int NT, bool REPLAY>
__global__ void __launch_bounds__(NT) gdn_decode_kernel(const GdnArgs a) {
  constexpr int SV = 4;              // fp32 state elements per vector
  constexpr int LPR = K / SV;        // lanes per state row
  static_assert(LPR <= 64 && 64 % LPR == 0, "a state row must fit one wave");
  constexpr int NVEC = V * K / SV;
  static_assert(NT % 64 == 0 && NVEC % NT == 0, "whole waves, whole tile");
  constexpr int ITEMS = NVEC / NT;
  constexpr int RPI = NT / LPR;
  constexpr int IV = Elt<IT>::kPer16;
  static_assert(K % IV == 0 && V % IV == 0, "rows are whole vectors");
  constexpr int KV = K / IV;
  constexpr int VV = V / IV;
  constexpr long kIo = sizeof(IT);

  extern __shared__ __attribute__((aligned(16))) float lds[];
  const int L = REPLAY ? a.ring_len : 1;
  float* ks = lds;            // [L][K]  k of entries 0..w
  float* ds = ks + L * K;     // [L][V]  d of entries 0..w-1, then d_w
  float* qs = ds + L * V;     // [K]
  float* vs = qs + K;         // [V]     v of the current step
  float* gs = vs + V;         // [L]     g of entries 0..w
  float* gam = gs + L;        // [L]     prod_{i<j<=w} g_j
  float* kk = gam + L;        // [L]     k_i . k_w
  float* kq = kk + L;         // [L]     k_i . q
  float* scal = kq + L;       // [0] = Gamma

  const int HV = a.v_heads;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int b = tile / HV;
  const int hv = tile - b * HV;
  const int hk = hv / a.vpk;
  const int tid = threadIdx.x;

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
  if (hv == 0 && tid == 0) {
    if (REPLAY) {
      const int nw = (f || bad_slot) ? 0 : w + 1;
      if (a.next_write_pos) a.next_write_pos[b] = nw;
      if (a.next_is_flush) a.next_is_flush[b] = (nw == L - 1) ? 1 : 0;
    }
    if (st && a.status) atomicOr(a.status, st);
  }
  const long ooff = ((long)b * HV + hv) * V;
  if (bad_slot) {
    for (int p = tid; p < V; p += NT) Elt<OT>::store1(a.o, ooff + p, __builtin_nanf(""));
    return;
  }

  // ---- 1. stream S0 = state[s, hv]
  const long tile_byte = ((long)s * HV + hv) * (long)V * K * 4;
  u32x4 sv[ITEMS];
#pragma unroll
  for (int it = 0; it < ITEMS; ++it)
    sv[it] = ld16_stream(a.state, tile_byte + ((long)it * NT + tid) * 16);

  // ---- 2. stage q, v, k_0..k_w, d_0..d_{w-1}, g_0..g_w
  const bool append = REPLAY && !f;
  const bool k_writer = (hv % a.vpk) == 0;
  const long qk_cur = ((long)b * a.k_heads + hk) * K;
  const long kring0 = ((long)s * a.k_heads + hk) * (long)L * K;
  const long dring0 = ((long)s * HV + hv) * (long)L * V;
  const long gring0 = ((long)s * HV + hv) * L;
  const int nQ = KV, nV = VV, nK = (w + 1) * KV, nD = w * (V / 4);
  const int nAll = nQ + nV + nK + nD;
  for (int u = tid; u < nAll; u += NT) {
    int c = u;
    if (c < nQ) {
      float fv[IV];
      Elt<IT>::unpack(ld16(a.q, (qk_cur + c * IV) * kIo), fv);
#pragma unroll
      for (int j = 0; j < IV; ++j) qs[c * IV + j] = fv[j];
      continue;
    }
    c -= nQ;
    if (c < nV) {
      float fv[IV];
      Elt<IT>::unpack(ld16(a.v, (ooff + c * IV) * kIo), fv);
#pragma unroll
      for (int j = 0; j < IV; ++j) vs[c * IV + j] = fv[j];
      continue;
    }
    c -= nV;
    if (c < nK) {
      const int i = c / KV;
      const int cc = c - i * KV;
      u32x4 raw;
      if (REPLAY && i < w) {
        raw = ld16(a.k_ring, (kring0 + (long)i * K + cc * IV) * kIo);
      } else {
        raw = ld16(a.k, (qk_cur + cc * IV) * kIo);
        if (append && k_writer) st16(a.k_ring, (kring0 + (long)w * K + cc * IV) * kIo, raw);
      }
      float fv[IV];
      Elt<IT>::unpack(raw, fv);
#pragma unroll
      for (int j = 0; j < IV; ++j) ks[i * K + cc * IV + j] = fv[j];
      continue;
    }
    c -= nK;
    {
      // d ring rows are fp32: 4 per vector
      const int i = c / (V / 4);
      const int cc = c - i * (V / 4);
      float fv[4];
      Elt<float>::unpack(ld16(a.d_ring, (dring0 + (long)i * V + cc * 4) * 4), fv);
#pragma unroll
      for (int j = 0; j < 4; ++j) ds[i * V + cc * 4 + j] = fv[j];
    }
  }
  const float gw = a.g[(long)b * HV + hv];
  for (int i = tid; i <= w; i += NT) {
    if (REPLAY && i < w) {
      gs[i] = a.g_ring[gring0 + i];
    } else {
      gs[i] = gw;
      if (append) a.g_ring[gring0 + w] = gw;
    }
  }
  __syncthreads();

  // ---- 3. gates and ring dots
  for (int i = tid; i <= w; i += NT) {
    float p = 1.f;
    for (int j = w; j > i; --j) p *= gs[j];
    gam[i] = p;
  }
  if (tid == 0) {
    float p = 1.f;
    for (int j = w; j >= 0; --j) p *= gs[j];
    scal[0] = p;
  }
  {
    constexpr int DG = 16;
    const int grp = tid / DG;
    const int lane = tid % DG;
    // 2w+1 dots: kk_i = k_i.k_w (i < w), kq_i = k_i.q (i <= w)
    const int ndot = 2 * w + 1;
    for (int t0 = 0; t0 < ndot; t0 += NT / DG) {
      const int t = t0 + grp;
      float acc = 0.f;
      const bool live = t < ndot;
      const int i = t <= w ? t : t - (w + 1);
      const float* other = t <= w ? qs : ks + w * K;
      if (live)
        for (int n = lane; n < K; n += DG) acc = fmaf(ks[i * K + n], other[n], acc);
      acc = group_sum<DG>(acc);
      if (live && lane == 0) {
        if (t <= w) kq[i] = acc;
        else kk[i] = acc;
      }
    }
  }
  __syncthreads();

  // ---- 4. S0 @ k_w and S0 @ q per state row
  const int c = tid % LPR;
  const int prow = tid / LPR;
  float kv4[SV], qv4[SV];
#pragma unroll
  for (int j = 0; j < SV; ++j) {
    kv4[j] = ks[w * K + c * SV + j];
    qv4[j] = qs[c * SV + j];
  }
  float dk_acc[ITEMS], dq_acc[ITEMS];
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    float sf[SV];
    Elt<float>::unpack(sv[it], sf);
    float a1 = 0.f, a2 = 0.f;
#pragma unroll
    for (int j = 0; j < SV; ++j) {
      a1 = fmaf(sf[j], kv4[j], a1);
      a2 = fmaf(sf[j], qv4[j], a2);
    }
    dk_acc[it] = group_sum<LPR>(a1);
    dq_acc[it] = group_sum<LPR>(a2);
  }
  const float Gam = scal[0];
  const float bw = a.beta[(long)b * HV + hv];
  // ---- 5. delta d_w and output (lane 0 of each row)
  if (c == 0) {
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int p = it * RPI + prow;
      float pred = Gam * dk_acc[it];
      float outv = Gam * dq_acc[it];
      for (int i = 0; i < w; ++i) {
        const float gd = gam[i] * ds[i * V + p];
        pred = fmaf(gd, kk[i], pred);
        outv = fmaf(gd, kq[i], outv);
      }
      const float dw = bw * (vs[p] - pred);
      outv = fmaf(dw, kq[w], outv);
      ds[w * V + p] = dw;
      Elt<OT>::store1(a.o, ooff + p, a.scale * outv);
      if (append) a.d_ring[dring0 + (long)w * V + p] = dw;
    }
  }
  if (f) {
    __syncthreads();
    // ---- 6. fold: S_new = Gamma * S0 + sum_i gamma_i * outer(d_i, k_i)
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int p = it * RPI + prow;
      float sf[SV];
      Elt<float>::unpack(sv[it], sf);
#pragma unroll
      for (int j = 0; j < SV; ++j) sf[j] *= Gam;
      for (int i = 0; i <= w; ++i) {
        const float coef = gam[i] * ds[i * V + p];
        const float* kp = ks + i * K + c * SV;
#pragma unroll
        for (int j = 0; j < SV; ++j) sf[j] = fmaf(coef, kp[j], sf[j]);
      }
      st16_stream(a.state, tile_byte + ((long)it * NT + tid) * 16, Elt<float>::pack(sf));
    }
  }
}

template <typename IT, typename OT, int V, int K, bool REPLAY>
static int launch_gdn(const GdnArgs& a, int batch, hipStream_t stream) {
  constexpr int NVEC = V * K / 4;
  constexpr int NT = NVEC >= 512 ? 512 : NVEC;
  const int L = REPLAY ? a.ring_len : 1;
  const size_t lds = sizeof(float) * (size_t)gdn_lds_floats<V, K>(L);
  if (lds > kMaxLds) return RSSM_ESHAPE;  // ring rows must fit one workgroup's LDS
  return launch_kernel(
      reinterpret_cast<const void*>(&gdn_decode_kernel<IT, OT, V, K, NT, REPLAY>),
      (unsigned)((long)batch * a.v_heads), NT, lds, stream, a);
}

template <bool REPLAY, typename IT, typename OT>
static int gdn_dispatch_shape(const GdnArgs& a, const rssm_gdn_dims& d, hipStream_t s) {
  if (d.dv == 128 && d.dk == 128) return launch_gdn<IT, OT, 128, 128, REPLAY>(a, d.batch, s);
  if (d.dv == 64 && d.dk == 64) return launch_gdn<IT, OT, 64, 64, REPLAY>(a, d.batch, s);
  if (d.dv == 128 && d.dk == 64) return launch_gdn<IT, OT, 128, 64, REPLAY>(a, d.batch, s);
  if (d.dv == 64 && d.dk == 128) return launch_gdn<IT, OT, 64, 128, REPLAY>(a, d.batch, s);
  return RSSM_ESHAPE;
}

template <bool REPLAY>
static int gdn_dispatch(const GdnArgs& a, const rssm_gdn_dims& d, hipStream_t s) {
  switch (d.io_dtype * 2 + d.out_dtype) {
    case 0: return gdn_dispatch_shape<REPLAY, float, float>(a, d, s);
    case 1: return gdn_dispatch_shape<REPLAY, float, bf16>(a, d, s);
    case 2: return gdn_dispatch_shape<REPLAY, bf16, float>(a, d, s);
    case 3: return gdn_dispatch_shape<REPLAY, bf16, bf16>(a, d, s);
  }
  return RSSM_EDTYPE;
}

static int gdn_check(const rssm_gdn_dims* d, bool replay) {
  if (!d) return RSSM_EINVAL;
  if (d->batch < 0 || d->k_heads < 1 || d->v_heads < 1 || d->v_heads % d->k_heads ||
      d->num_slots < 1)
    return RSSM_EINVAL;
  if ((long)d->batch * d->v_heads > 0x7fffffffL) return RSSM_EINVAL;
  if (d->state_dtype != RSSM_F32 || !valid_dtype(d->io_dtype) || !valid_dtype(d->out_dtype))
    return RSSM_EDTYPE;
  if (!((d->dk == 64 || d->dk == 128) && (d->dv == 64 || d->dv == 128))) return RSSM_ESHAPE;
  if (replay && (d->ring_len < 1 || d->ring_len > 64)) return RSSM_ESHAPE;
  return RSSM_OK;
}

static GdnArgs gdn_args(const rssm_gdn_dims* d) {
  GdnArgs a{};
  a.k_heads = d->k_heads;
  a.v_heads = d->v_heads;
  a.vpk = d->v_heads / d->k_heads;
  a.num_slots = d->num_slots;
  a.scale = d->scale > 0.f ? d->scale : 1.0f / sqrtf((float)d->dk);
  return a;
}

}  // namespace rssm

using namespace rssm;

extern "C" int gdn_standard_decode(const rssm_gdn_dims* dims, void* state, const int32_t* slot_idx,
                                   const void* q, const void* k, const void* v, const float* g,
                                   const float* beta, void* o, int32_t* status,
                                   hipStream_t stream) {
  int rc = gdn_check(dims, false);
  if (rc) return rc;
  if (dims->batch == 0) return RSSM_OK;  // empty batch: nothing to read or write
  if (!state || !slot_idx || !q || !k || !v || !g || !beta || !o) return RSSM_EINVAL;
  if (!aligned16(state) || !aligned16(q) || !aligned16(k) || !aligned16(v)) return RSSM_EINVAL;
  GdnArgs a = gdn_args(dims);
  a.state = static_cast<float*>(state);
  a.slot_idx = slot_idx;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.o = o;
  a.status = status;
  a.ring_len = 1;
  return gdn_dispatch<false>(a, *dims, stream);
}

extern "C" int replayssm_gdn_decode(const rssm_gdn_dims* dims, void* state, float* d_ring,
                                    void* k_ring, float* g_ring, const int32_t* slot_idx,
                                    const int32_t* write_pos, const uint8_t* is_flush,
                                    int32_t* next_write_pos, uint8_t* next_is_flush,
                                    const void* q, const void* k, const void* v, const float* g,
                                    const float* beta, void* o, int32_t* status,
                                    hipStream_t stream) {
  int rc = gdn_check(dims, true);
  if (rc) return rc;
  if (dims->batch == 0) return RSSM_OK;  // empty batch: nothing to read or write
  if (!state || !d_ring || !k_ring || !g_ring || !slot_idx || !write_pos || !is_flush || !q ||
      !k || !v || !g || !beta || !o)
    return RSSM_EINVAL;
  if (!aligned16(state) || !aligned16(d_ring) || !aligned16(k_ring) || !aligned16(q) ||
      !aligned16(k) || !aligned16(v))
    return RSSM_EINVAL;
  if ((const void*)next_write_pos == (const void*)write_pos && next_write_pos) return RSSM_EINVAL;
  if ((const void*)next_is_flush == (const void*)is_flush && next_is_flush) return RSSM_EINVAL;
  GdnArgs a = gdn_args(dims);
  a.state = static_cast<float*>(state);
  a.d_ring = d_ring;
  a.k_ring = k_ring;
  a.g_ring = g_ring;
  a.slot_idx = slot_idx;
  a.write_pos = write_pos;
  a.is_flush = is_flush;
  a.next_write_pos = next_write_pos;
  a.next_is_flush = next_is_flush;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.o = o;
  a.status = status;
  a.ring_len = dims->ring_len;
  return gdn_dispatch<true>(a, *dims, stream);
}
