// Gated-delta-rule decode kernels for gfx950: the recurrent update and the
// ReplaySSM ring decode (checkpoint S0 + ring of (d, k, g), fold on flush
// rows only), for the GDN scalar gate and the KDA per-key-channel gate.
//
// Method: sglang #28451 (GDN/KDA ReplaySSM decode) - Motivation (GDN decode
// reads and writes the full [HV, V, K] state every step and is bandwidth
// bound at large batch) and Implementation item 1 (non-flush steps rebuild
// the output from S0 plus the ring; the state is refreshed every L steps);
// the ring contents d [L, V], k [L, K], g [L] per slot follow the memory-pool
// snippet of sglang #28695 "[GDN] Support ReplaySSM Ring Spec-Verify".
// One kernel serves both gates through a compile-time switch (sglang #28451,
// Implementation item 1); the KDA ring keeps a [K] gate row per entry
// (review notes of the same report).  Formulas: see the contract in
// replayssm.h.
//
// Mapping (one workgroup per (row, value head) tile of the [V, K] fp32
// state; LPR = K/4 adjacent lanes hold one state row):
//  * every global read of the step is issued at once: q, v, k_0..k_w and
//    d_0..d_{w-1} into LDS with direct-to-LDS loads, the gates into lanes,
//    then the tile into registers with raw buffer loads; the gate and ring
//    work waits only for the staged rows, not for the tile;
//  * gate products by DPP suffix scans, ring dots k_i.k_w and k_i.q on 16
//    lanes each (packed bf16 dot2 for bf16 inputs), their weights broadcast
//    through LDS;
//  * S0.k_w and S0.q per state row by a butterfly transpose-reduce, then
//    one lane per row forms pred, d_w and o;
//  * flush rows fold Gamma*S0 + sum_i gamma_i outer(d_i, k_i) in chunks of
//    the registers, with gamma_i*d_i precomputed in LDS, and store with
//    global stores.
// The contractions are two matrix-vector products and, on flush rows, a
// rank-(w+1) update with w+1 <= L: too thin for the matrix cores to pay,
// and the kernel is bound by the state stream, so they run on the VALU.
//
// KDA (per-channel gate g_j in R^K): gamma_i and Gamma are vectors over the
// key channels.  The gate rows go to LDS with the other ring rows; one
// thread per channel walks the entries from w down to 0 and replaces gate
// row i by kt_i = gamma_i * k_i in place, leaving Gamma_c.  Every scalar gate
// factor of the GDN path then moves into kt_i (ring dots kt_i . k_w,
// kt_i . q and the rank update) and into Gamma * k_w, Gamma * q (S0 dots and
// the fold's diagonal scale).
#include <math.h>

#include "gdn_common.hpp"
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

// LDS: 16-byte chunks [q | v | k rows (8-row multiples) | d rows 0..L-1 (fp32)
// | KDA: gate rows (fp32, 8-row multiples)]
template <typename IT, int V, int K, bool KDA = false>
struct GdnStage {
  static constexpr int IV = Elt<IT>::kPer16;
  static constexpr int QV = K / IV;  // chunks per q / k row
  static constexpr int VV = V / IV;  // chunks per v row
  static constexpr int DV = V / 4;   // chunks per d row
  static constexpr int GV = K / 4;   // chunks per KDA gate row
  static_assert(K % IV == 0 && V % IV == 0, "rows are whole chunks");
  static constexpr int oK = QV + VV;
  static constexpr int oD(int L) { return oK + ((L + 7) & ~7) * QV; }
  static constexpr int oG(int L) { return oD(L) + L * DV; }
  static constexpr int chunks(int L) { return oG(L) + (KDA ? ((L + 7) & ~7) * GV : 0); }
};

template <typename IT, typename OT, int V, int K, bool REPLAY, bool KDA>
__global__ void __launch_bounds__((GdnShape<V, K, REPLAY>::NT)) gdn_decode_kernel(const GdnArgs a) {
  using GS = GdnShape<V, K, REPLAY>;
  using SG = GdnStage<IT, V, K, KDA>;
  constexpr int SV = GS::SV, LPR = GS::LPR, NT = GS::NT, ITEMS = GS::ITEMS, RPI = GS::RPI;
  constexpr int IC = GS::IC;
  constexpr int QV = SG::QV, VV = SG::VV, DV = SG::DV, GV = SG::GV;
  constexpr long kIo = sizeof(IT);

  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ __attribute__((aligned(16))) float cf_lds[2 * NT];  // per wave: ring weights
  __shared__ float gm_lds[64];                                   // gamma_i (GDN)
  __shared__ __attribute__((aligned(16))) float gk_lds[KDA ? K : 4];  // Gamma_c (KDA)

  const int L = REPLAY ? a.ring_len : 1;
  const int HV = a.v_heads;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rank = tile / HV;  // row rank; replay visits flush rows first
  const int hv = tile - rank * HV;
  const int hk = hv / a.vpk;

  RowPick pick{rank, 0, 0, true};
  if constexpr (REPLAY)
    pick = flush_first_pick(rank, gridDim.x / HV, a.slot_idx, a.write_pos, a.is_flush, lane);
  else
    pick.s = a.slot_idx[rank];
  const int b = pick.b;
  const int s = pick.s;
  int w = 0;
  bool f = true;
  int st = 0;
  if (REPLAY) {
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

  // ---- 1. every global read of the step: staged rows and gates, then the tile
  char* const tptr = (char*)a.state + ((long)s * HV + hv) * (long)V * K * 4;
  const rsrc_t trs = tile_rsrc(tptr, (uint32_t)(V * K * 4));
  const uint32_t lane_off = tid * 16;
  u32x4 sv[ITEMS];

  const long qk_cur = ((long)b * a.k_heads + hk) * K;             // q, k[b, hk, :]
  const long kring0 = ((long)s * a.k_heads + hk) * (long)L * K;   // k_ring[s, hk, 0, :]
  const long dring0 = ((long)s * HV + hv) * (long)L * V;          // d_ring[s, hv, 0, :]
  const long gring0 = ((long)s * HV + hv) * L * (KDA ? K : 1);
  const int oK = SG::oK;
  const int oD = SG::oD(L);
  const int oG = SG::oG(L);
  auto dma_span = [&](int c0, int n, const char* ring, int nring, const char* cur) {
    for (int j = wave * 64; j < n; j += NT) {
      const int u = j + lane;
      if (u < n) {
        const char* src = u < nring ? ring + (long)u * 16 : cur + (long)(u - nring) * 16;
        dma16<REPLAY>(src, lds + (long)(c0 + j) * 16);
      }
    }
  };
  {
    const char* qg = (const char*)a.q + qk_cur * kIo;
    const char* vg = (const char*)a.v + ooff * kIo;
    dma_span(0, QV, qg, QV, qg);
    dma_span(QV, VV, vg, VV, vg);
    dma_span(oK, (w + 1) * QV, REPLAY ? (const char*)a.k_ring + kring0 * kIo : nullptr,
             REPLAY ? w * QV : 0, (const char*)a.k + qk_cur * kIo);
    if (REPLAY && w > 0) {
      const char* dg = (const char*)a.d_ring + dring0 * 4;
      dma_span(oD, w * DV, dg, w * DV, dg);
    }
    if constexpr (KDA)  // gate rows 0..w-1 from the ring, row w the current gate
      dma_span(oG, (w + 1) * GV, REPLAY ? (const char*)(a.g_ring + gring0) : nullptr,
               REPLAY ? w * GV : 0, (const char*)(a.g + ((long)b * HV + hv) * K));
  }
  const float gw = KDA ? 1.f : a.g[(long)b * HV + hv];
  const float bw = a.beta[(long)b * HV + hv];
  float gl = 1.f;  // g of entry `lane` (1 past w: neutral in products)
  if constexpr (!KDA) {
    if (REPLAY && lane < w) gl = a.g_ring[gring0 + lane];
  }
  // the tile last: steps 2 and 3 need only the staged rows and the gates, so
  // they run while the tile is still in flight (the scheduling barriers keep
  // the issue order the counter wait below relies on)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) sv[it] = bload16_nt(trs, lane_off, it * NT * 16);
  static_assert(ITEMS < 64, "the vmcnt field holds 6 bits");
  // everything but the ITEMS tile loads has landed: vmcnt <= ITEMS (bits 3:0
  // and 15:14 of the immediate), expcnt and lgkmcnt 0
  __builtin_amdgcn_s_waitcnt((ITEMS & 15) | ((ITEMS >> 4) << 14));
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  if (!KDA && lane == w) gl = gw;

  const char* Qs = lds;
  const char* Vs = lds + QV * 16;
  const char* Ks = lds + oK * 16;
  float* Ds = reinterpret_cast<float*>(lds + (long)oD * 16);
  float* Gs = reinterpret_cast<float*>(lds + (long)oG * 16);  // KDA gate rows -> kt rows

  // ---- 2. gates: gamma_i = prod_{i<j<=w} g_j (lane i), Gamma = prod_{j<=w} g_j
  float gam = 1.f, Gam = 1.f;
  if constexpr (KDA) {
    // per channel c: kt_i[c] = gamma_i[c] * k_i[c] over gate row i, Gamma_c;
    // the current gate row goes to the ring here when the row appends
    for (int c = tid; c < K; c += NT) {
      if (REPLAY && !f) a.g_ring[gring0 + (long)w * K + c] = Gs[w * K + c];
      float gp = 1.f;
      for (int i = w; i >= 0; --i) {
        const float gi = Gs[i * K + c];
        Gs[i * K + c] = gp * LdsRead<IT>::one(Ks + (long)i * QV * 16, c);
        gp *= gi;
      }
      gk_lds[c] = gp;
    }
    __syncthreads();
  } else {
    gam = L <= 16 ? row16_suffix_product_exclusive(gl) : wave_suffix_product_exclusive(gl, lane);
    Gam = lane_value(gl * gam, 0);
  }

  // ---- 3. ring dots kk_i = k_i . k_w, kq_i = k_i . q (KDA: kt_i in place of
  // k_i): 16 lanes per row i
  float kk = 0.f, kq = 0.f;
  if constexpr (KDA) {
    constexpr int EPL = K / 16;
    const int q16 = lane & 15;
    float kw[EPL], qq[EPL];
    LdsRead<IT>::template seg<EPL>(Ks + (long)w * QV * 16, q16 * EPL, kw);
    LdsRead<IT>::template seg<EPL>(Qs, q16 * EPL, qq);
    for (int pass = 0; pass * 4 <= w; ++pass) {
      const int i = pass * 4 + (lane >> 4);  // rows past w: unused values
      float kt[EPL];
      LdsRead<float>::template seg<EPL>(reinterpret_cast<const char*>(Gs + i * K), q16 * EPL, kt);
      float a1 = 0.f, a2 = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        a1 = fmaf(kt[e], kw[e], a1);
        a2 = fmaf(kt[e], qq[e], a2);
      }
      a1 = group_sum<16>(a1);
      a2 = group_sum<16>(a2);
      a1 = __shfl(a1, (lane & 3) * 16, 64);
      a2 = __shfl(a2, (lane & 3) * 16, 64);
      if ((lane >> 2) == pass) {
        kk = a1;
        kq = a2;
      }
    }
  } else {
    constexpr int EPL = K / 16;
    const int q16 = lane & 15;
    SegDot<IT, EPL> kw, qq;
    kw.load(Ks + (long)w * QV * 16, q16 * EPL);
    qq.load(Qs, q16 * EPL);
    for (int pass = 0; pass * 4 <= w; ++pass) {
      const int i = pass * 4 + (lane >> 4);
      SegDot<IT, EPL> ki;
      ki.load(Ks + (long)i * QV * 16, q16 * EPL);  // rows past w: unused values
      float a1 = group_sum<16>(ki.dot(kw));
      float a2 = group_sum<16>(ki.dot(qq));
      a1 = __shfl(a1, (lane & 3) * 16, 64);
      a2 = __shfl(a2, (lane & 3) * 16, 64);
      if ((lane >> 2) == pass) {
        kk = a1;
        kq = a2;
      }
    }
  }
  const float kqw = lane_value(kq, w);        // k_w . q (gamma_w = 1)
  float* cw = cf_lds + wave * 128;            // [gamma_i kk_i (i<w) | gamma_i kq_i (i<w)]
  cw[lane] = lane < w ? gam * kk : 0.f;
  cw[64 + lane] = lane < w ? gam * kq : 0.f;
  __builtin_amdgcn_wave_barrier();

  // ---- 4. S0 . k_w and S0 . q per state row (KDA: S0 . (Gamma*k_w), S0 . (Gamma*q))
  const int c = tid % LPR;
  const int prow = tid / LPR;
  float kseg[SV], qseg[SV], gseg[SV];
  LdsRead<IT>::template seg<SV>(Ks + (long)w * QV * 16, c * SV, kseg);
  LdsRead<IT>::template seg<SV>(Qs, c * SV, qseg);
  if constexpr (KDA) {
    LdsRead<float>::template seg<SV>(reinterpret_cast<const char*>(gk_lds), c * SV, gseg);
#pragma unroll
    for (int j = 0; j < SV; ++j) {
      kseg[j] *= gseg[j];
      qseg[j] *= gseg[j];
    }
  }
  float pk[ITEMS], pq[ITEMS];
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
    float sf[SV];
    Elt<float>::unpack(sv[it], sf);
    float a1 = 0.f, a2 = 0.f;
#pragma unroll
    for (int j = 0; j < SV; ++j) {
      a1 = fmaf(sf[j], kseg[j], a1);
      a2 = fmaf(sf[j], qseg[j], a2);
    }
    pk[it] = a1;
    pq[it] = a2;
  }
  using RR = RowReduce<ITEMS, LPR>;
  RR::run(pk, tid);
  RR::run(pq, tid);

  // ---- 5. per state row: pred, d_w, o
  const bool writer = (c % RR::DUP) == 0;
#pragma unroll
  for (int j = 0; j < RR::NF; ++j) {
    const int vr = RR::item(j, tid) * RPI + prow;
    float pred = Gam * pk[j];
    float outv = Gam * pq[j];
    for (int ib = 0; ib < w; ib += 4) {
#pragma unroll
      for (int k2 = 0; k2 < 4; ++k2) {
        const int i = ib + k2;
        const int ic = i < w ? i : w - 1;  // weights are 0 past w-1
        const float dv = Ds[ic * V + vr];
        pred = fmaf(cw[i], dv, pred);
        outv = fmaf(cw[64 + i], dv, outv);
      }
    }
    const float dw = bw * (LdsRead<IT>::one(Vs, vr) - pred);
    outv = fmaf(kqw, dw, outv);
    if (writer) {
      Elt<OT>::store1(a.o, ooff + vr, a.scale * outv);
      Ds[w * V + vr] = dw;
    }
  }
  if (wave == 0) gm_lds[lane] = gam;
  __syncthreads();  // d_w of every row and the gamma_i are in LDS

  if (!f) {
    // ---- 6a. append (d_w, k_w, g_w) at ring position w (a KDA gate row went
    // out in step 2)
    if (wave == 0) {
      const bool k_writer = (hv % a.vpk) == 0;  // one writer per key head
      for (int k2 = lane; k2 < DV + QV; k2 += 64) {
        if (k2 < DV) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(lds + ((long)oD + w * DV + k2) * 16);
          st16(a.d_ring, (dring0 + (long)w * V) * 4 + k2 * 16, v);
        } else if (k_writer) {
          const int cc = k2 - DV;
          const u32x4 v = *reinterpret_cast<const u32x4*>(Ks + ((long)w * QV + cc) * 16);
          st16(a.k_ring, (kring0 + (long)w * K) * kIo + cc * 16, v);
        }
      }
      if (!KDA && lane == 0) a.g_ring[gring0 + w] = gw;
    }
    return;
  }

  // ---- 6b. flush: S_new = Gamma*S0 + sum_{i<=w} outer(gamma_i d_i, k_i)
  // (KDA: S0 diag(Gamma) + sum_{i<=w} outer(d_i, kt_i))
  if constexpr (!KDA) {
    for (int e = tid; e < (w + 1) * V; e += NT) {
      const int i = e / V;
      Ds[e] *= gm_lds[i];
    }
  }
  __syncthreads();
#pragma unroll
  for (int i0 = 0; i0 < ITEMS; i0 += IC) {
    float sf[IC][SV];
#pragma unroll
    for (int q = 0; q < IC; ++q)
#pragma unroll
      for (int j = 0; j < SV; ++j) sf[q][j] = 0.f;
    for (int i = 0; i <= w; ++i) {
      float kv[SV];
      if constexpr (KDA)
        LdsRead<float>::template seg<SV>(reinterpret_cast<const char*>(Gs + i * K), c * SV, kv);
      else
        LdsRead<IT>::template seg<SV>(Ks + (long)i * QV * 16, c * SV, kv);
#pragma unroll
      for (int q = 0; q < IC; ++q) {
        const float dv = Ds[i * V + (i0 + q) * RPI + prow];
#pragma unroll
        for (int j = 0; j < SV; ++j) sf[q][j] = fmaf(dv, kv[j], sf[q][j]);
      }
    }
#pragma unroll
    for (int q = 0; q < IC; ++q) {
      float s0[SV];
      Elt<float>::unpack(sv[i0 + q], s0);
#pragma unroll
      for (int j = 0; j < SV; ++j) sf[q][j] = fmaf(KDA ? gseg[j] : Gam, s0[j], sf[q][j]);
      st16_stream(tptr, (long)lane_off + (i0 + q) * NT * 16, Elt<float>::pack(sf[q]));
    }
  }
}

template <typename IT, typename OT, int V, int K, bool REPLAY, bool KDA>
static int launch_gdn(const GdnArgs& a, int batch, hipStream_t stream) {
  using GS = GdnShape<V, K, REPLAY>;
  const int L = REPLAY ? a.ring_len : 1;  // L <= 64: one gate per lane of a wave
  const size_t lds = (size_t)GdnStage<IT, V, K, KDA>::chunks(L) * 16;
  const size_t fixed = (2 * GS::NT + 64 + (KDA ? K : 4)) * sizeof(float);  // weights, gates
  if (lds + fixed > kMaxLds) return RSSM_ESHAPE;  // ring rows must fit one workgroup's LDS
  return launch_kernel(
      reinterpret_cast<const void*>(&gdn_decode_kernel<IT, OT, V, K, REPLAY, KDA>),
      (unsigned)((long)batch * a.v_heads), GS::NT, lds, stream, a);
}

template <bool REPLAY, bool KDA, typename IT, typename OT>
static int gdn_dispatch_shape(const GdnArgs& a, const rssm_gdn_dims& d, hipStream_t s) {
  if (d.dv == 128 && d.dk == 128) return launch_gdn<IT, OT, 128, 128, REPLAY, KDA>(a, d.batch, s);
  if (d.dv == 64 && d.dk == 64) return launch_gdn<IT, OT, 64, 64, REPLAY, KDA>(a, d.batch, s);
  if (d.dv == 128 && d.dk == 64) return launch_gdn<IT, OT, 128, 64, REPLAY, KDA>(a, d.batch, s);
  if (d.dv == 64 && d.dk == 128) return launch_gdn<IT, OT, 64, 128, REPLAY, KDA>(a, d.batch, s);
  return RSSM_ESHAPE;
}

template <bool REPLAY, bool KDA>
static int gdn_dispatch(const GdnArgs& a, const rssm_gdn_dims& d, hipStream_t s) {
  switch (d.io_dtype * 2 + d.out_dtype) {
    case 0: return gdn_dispatch_shape<REPLAY, KDA, float, float>(a, d, s);
    case 1: return gdn_dispatch_shape<REPLAY, KDA, float, bf16>(a, d, s);
    case 2: return gdn_dispatch_shape<REPLAY, KDA, bf16, float>(a, d, s);
    case 3: return gdn_dispatch_shape<REPLAY, KDA, bf16, bf16>(a, d, s);
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

template <bool KDA>
static int standard_entry(const rssm_gdn_dims* dims, void* state, const int32_t* slot_idx,
                          const void* q, const void* k, const void* v, const float* g,
                          const float* beta, void* o, int32_t* status, hipStream_t stream) {
  int rc = gdn_check(dims, false);
  if (rc) return rc;
  if (dims->batch == 0) return RSSM_OK;  // empty batch: nothing to read or write
  if (!state || !slot_idx || !q || !k || !v || !g || !beta || !o) return RSSM_EINVAL;
  if (!aligned16(state) || !aligned16(q) || !aligned16(k) || !aligned16(v)) return RSSM_EINVAL;
  if (KDA && !aligned16(g)) return RSSM_EINVAL;
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
  return gdn_dispatch<false, KDA>(a, *dims, stream);
}

template <bool KDA>
static int replay_entry(const rssm_gdn_dims* dims, void* state, float* d_ring, void* k_ring,
                        float* g_ring, const int32_t* slot_idx, const int32_t* write_pos,
                        const uint8_t* is_flush, int32_t* next_write_pos, uint8_t* next_is_flush,
                        const void* q, const void* k, const void* v, const float* g,
                        const float* beta, void* o, int32_t* status, hipStream_t stream) {
  int rc = gdn_check(dims, true);
  if (rc) return rc;
  if (dims->batch == 0) return RSSM_OK;  // empty batch: nothing to read or write
  if (!state || !d_ring || !k_ring || !g_ring || !slot_idx || !write_pos || !is_flush || !q ||
      !k || !v || !g || !beta || !o)
    return RSSM_EINVAL;
  if (!aligned16(state) || !aligned16(d_ring) || !aligned16(k_ring) || !aligned16(q) ||
      !aligned16(k) || !aligned16(v))
    return RSSM_EINVAL;
  if (KDA && (!aligned16(g) || !aligned16(g_ring))) return RSSM_EINVAL;
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
  return gdn_dispatch<true, KDA>(a, *dims, stream);
}

}  // namespace rssm

using namespace rssm;

extern "C" int gdn_standard_decode(const rssm_gdn_dims* dims, void* state, const int32_t* slot_idx,
                                   const void* q, const void* k, const void* v, const float* g,
                                   const float* beta, void* o, int32_t* status,
                                   hipStream_t stream) {
  return standard_entry<false>(dims, state, slot_idx, q, k, v, g, beta, o, status, stream);
}

extern "C" int replayssm_gdn_decode(const rssm_gdn_dims* dims, void* state, float* d_ring,
                                    void* k_ring, float* g_ring, const int32_t* slot_idx,
                                    const int32_t* write_pos, const uint8_t* is_flush,
                                    int32_t* next_write_pos, uint8_t* next_is_flush,
                                    const void* q, const void* k, const void* v, const float* g,
                                    const float* beta, void* o, int32_t* status,
                                    hipStream_t stream) {
  return replay_entry<false>(dims, state, d_ring, k_ring, g_ring, slot_idx, write_pos, is_flush,
                             next_write_pos, next_is_flush, q, k, v, g, beta, o, status, stream);
}

extern "C" int kda_standard_decode(const rssm_gdn_dims* dims, void* state, const int32_t* slot_idx,
                                   const void* q, const void* k, const void* v, const float* g,
                                   const float* beta, void* o, int32_t* status,
                                   hipStream_t stream) {
  return standard_entry<true>(dims, state, slot_idx, q, k, v, g, beta, o, status, stream);
}

extern "C" int replayssm_kda_decode(const rssm_gdn_dims* dims, void* state, float* d_ring,
                                    void* k_ring, float* g_ring, const int32_t* slot_idx,
                                    const int32_t* write_pos, const uint8_t* is_flush,
                                    int32_t* next_write_pos, uint8_t* next_is_flush,
                                    const void* q, const void* k, const void* v, const float* g,
                                    const float* beta, void* o, int32_t* status,
                                    hipStream_t stream) {
  return replay_entry<true>(dims, state, d_ring, k_ring, g_ring, slot_idx, write_pos, is_flush,
                            next_write_pos, next_is_flush, q, k, v, g, beta, o, status, stream);
}
