// GDN speculative verify from the checkpoint + ring, and the commit with its
// exact fold, for gfx950.
//
// Method: sglang #28695 "[GDN] Support ReplaySSM Ring Spec-Verify" -
// Motivation (the recurrent verify keeps a full state snapshot per draft
// token), Implementation items 2-4 (per-slot ring of d, k, g and of the raw
// inputs v, k, beta; a verify kernel that rebuilds every draft's output from
// the frozen checkpoint and the ring; an exact-fold kernel that replays the
// raw inputs in order through the recurrent update on flush; the commit
// advances the cursor instead of copying a snapshot; linear draft chains;
// ring length at least twice the draft count) and the review notes (the
// closed-form fold drifted on long outputs, the exact fold restored parity).
// Formulas: see the contract in replayssm.h.
//
// Verify mapping: one workgroup per (row, value head) fp32 [V, K] tile.  q, v
// of the T drafts, the k rows of the committed entries and of the drafts,
// and the committed d rows are staged in LDS by direct-to-LDS loads, then
// the tile is read once into registers, 1 KB contiguous per load instruction.
// While the tile is in flight the waves form, per draft t at ring position
// p = w + t (one draft per wave at a time), the gate products (DPP suffix
// products over the lanes holding g_0..g_p) and the weighted dots
// gamma_i*(k_i.k_p), gamma_i*(k_i.q_t).  Then S0.k_p and S0.q_t for every
// state row by 2T butterfly row reductions, and each state row walks the
// drafts in order, keeping the new d values in registers.  The drafts' d, v
// and k rows are written to ring entries w..w+T-1 as one contiguous run per
// array with non-temporal stores, then g and beta; the state and the cursor
// are not touched.  (A matrix-core form of the 2T products needs the tile in
// the operand layout, 16 state rows per load instruction, and measured
// slower: the access pattern costs more than the products save.)
//
// Commit mapping: only about one row in L/(mean acceptance) folds per round,
// so the commit is a small grid working through a task list (batches of up
// to 512 rows): each workgroup reads every row's cursor, accepted count,
// force flag and slot in one round trip and lists the folding rows in LDS;
// workgroup 0 writes the cursor outputs; the (folding row, value head) tasks
// are shared out over the grid, the same count to every XCD.  Larger batches
// take one workgroup per (row, value head).  A fold holds the tile in fp32
// registers, eight lanes per state row (128-byte segments per load), and
// applies the recurrence entry by entry in order: the decays are carried as
// one running product instead of scaling every element, the row dots with k
// are sums over eight lanes by DPP, d passes within the wave through LDS,
// then the rank-1 update (the waves never wait for one another); the tile is
// stored scaled by the product.
//
// Deferred-fold rounds: instead of the commit, an advance only moves the
// cursors and marks the rows whose next verify would not fit (a per-row
// is_flush flag); that verify folds their ring on the tile registers it has
// just loaded (the same recurrence on the verify's lane layout, row sums
// over 16 or 32 lanes by row swaps and DPP), stores the folded tile and
// verifies the drafts at entries 0..T-1, so the folding tile is read from
// memory once instead of twice.  In these rounds the verify writes only the drafts' d rows; the
// advance writes the kept drafts' v, k, g and beta rows from the inputs (in
// the verify the other value heads of a folding row's key head may still
// be reading its old k rows, and writes inside the tile read stream cost
// several times their bytes).
#include <math.h>

#include "gdn_common.hpp"
#include "rssm_device.hpp"
#include "rssm_host.hpp"

namespace rssm {

constexpr int kMaxDraft = 8;

struct SpecArgs {
  float* state;
  float* d_ring;
  void* k_ring;
  float* g_ring;
  void* v_ring;
  float* beta_ring;
  const int32_t* slot_idx;
  const int32_t* write_pos;
  const int32_t* accepted;
  const uint8_t* force_flush;
  int32_t* next_write_pos;
  uint8_t* flushed;
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  void* o;
  int32_t* status;
  int32_t k_heads;
  int32_t v_heads;
  int32_t vpk;
  int32_t ring_len;
  int32_t num_slots;
  int32_t n_draft;
  float scale;
  int32_t fold_tasks;  // commit: a small grid working through a list of fold tasks
  int32_t n_rows;      // commit, advance: batch rows
  const uint8_t* is_flush;  // verify with flush, advance: rows whose ring folds before the verify
  uint8_t* next_is_flush;   // advance: the next round's flags
};

// Commit decision of one row: the cursor after its accepted drafts (clamped
// to the ring, with the status bit, when the counts are bad), whether the
// row folds its ring into the checkpoint, and its status bits.  Both the
// cursor outputs and the fold work follow this one rule.
struct CommitRow {
  int wn;
  int st;
  bool flush;
};
__device__ static inline CommitRow commit_row(int s, int w, int acc, bool force,
                                              const SpecArgs& a) {
  const int T = a.n_draft, L = a.ring_len;
  int wn = (int)((uint32_t)w + (uint32_t)acc);
  int st = 0;
  if (acc < 0 || acc > T || wn < 0 || wn > L) {
    st |= RSSM_ST_RING_OVERFLOW;
    wn = wn < 0 ? 0 : (wn > L ? L : wn);
  }
  const bool bad_slot = s < 0 || s >= a.num_slots;
  if (bad_slot) st |= RSSM_ST_BAD_SLOT;
  return {wn, st, !bad_slot && (wn + T > L || force)};
}

// Largest batch the task-list commit takes (one row list in LDS).
constexpr int kTaskRows = 512;

// Verify LDS, 16-byte chunks: [q rows 0..T-1 | v rows 0..T-1 |
// k rows 0..L-1 (multiple of 8) | d rows 0..L-1 (fp32)]
template <typename IT, int V, int K>
struct VerifyStage {
  static constexpr int IV = Elt<IT>::kPer16;
  static constexpr int QV = K / IV;
  static constexpr int VV = V / IV;
  static constexpr int DV = V / 4;
  static constexpr int oV(int T) { return T * QV; }
  static constexpr int oK(int T) { return T * (QV + VV); }
  static constexpr int oD(int T, int L) { return oK(T) + ((L + 7) & ~7) * QV; }
  static constexpr int chunks(int T, int L) { return oD(T, L) + L * DV; }
};

// Matrix-core form of the verify's 2T products (bf16 inputs, V = K = 128,
// 256 threads): each wave owns 32 state rows of the contiguously loaded tile
// (rows it*8 + 2*wave + h) and a private LDS region, first the staging
// buffer of one 16-row x 32-column block (row pitch 36 floats against bank
// conflicts), then its rows' products [32][16].
struct VerifyMfma {
  static constexpr int kPitch = 36;
  static constexpr int kRegionFloats = 16 * kPitch;  // >= 32 * 16
  static constexpr size_t kBytes = 4 * kRegionFloats * sizeof(float);
};

// Dynamic LDS of the verify: the staged rows, then the matrix-core regions.
template <typename IT, int V, int K, bool MF>
__host__ __device__ constexpr size_t verify_lds_bytes(int T, int L) {
  return (size_t)VerifyStage<IT, V, K>::chunks(T, L) * 16 + (MF ? VerifyMfma::kBytes : 0);
}

// A folding row's stage after it: k rows and v rows of the whole ring as
// stored, then two V-float buffers of d.
template <typename IT, int V, int K>
constexpr size_t verify_fold_bytes(int L) {
  return (size_t)L * (K + V) * sizeof(IT) + 2 * V * sizeof(float);
}

// 16-byte chunks [c0, c0+n) of LDS from global memory, one wave-wide
// direct-to-LDS load per 64 chunks; chunk u comes from src + 16*u.  NT: the
// non-temporal policy, for rows only this workgroup reads (a value head's
// own v and d rows; the q and k rows are shared by the value heads of a key
// head and stay temporal).
template <bool NT = false>
__device__ static inline void dma_rows(char* lds, int c0, int n, const char* src, int wave,
                                       int lane, int nt) {
  for (int j = wave * 64; j < n; j += nt) {
    const int u = j + lane;
    if (u < n) dma16<NT>(src + (long)u * 16, lds + (long)(c0 + j) * 16);
  }
}

// The fold holds the tile as gam * S: a step's decay g multiplies the scalar
// gam instead of every element, the row dot is gam * (S.k) and the rank-1
// update adds (d / gam) k to S.  Algebraically the recurrence; when gam
// would leave [2^-60, 2^60] (or g is 0 or not finite) the pending decay and
// the step's own are applied to S element by element and gam restarts at 1.
constexpr float kLazyFloor = 0x1p-60f, kLazyCeil = 0x1p60f;

// Sums of ITEMS per-lane partials over the LPR (16 or 32) lanes of a state
// row, folded as RowReduce does it (lane keeps the total of partial
// RowReduce::item(0, lane)), by VALU lane exchanges only: lanes 16 apart by
// a row swap (the two values each pair of lanes adds arrive in the two
// swapped registers), then half-row mirror partners and quad permutations.
template <int ITEMS, int LPR>
struct FoldReduce {
  static_assert(ITEMS == 16 && (LPR == 16 || LPR == 32), "fold reduce shape");
  template <int ctrl>
  __device__ static inline float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), ctrl, 0xF, 0xF, false));
  }
  template <int H, int O, int ctrl>
  __device__ static inline void level(float (&v)[ITEMS], int lane) {
    const bool up = (lane & O) != 0;
#pragma unroll
    for (int j = 0; j < H; ++j) {
      const float send = up ? v[j] : v[j + H];
      const float keep = up ? v[j + H] : v[j];
      v[j] = keep + dpp<ctrl>(send);
    }
  }
  __device__ static inline void run(float (&v)[ITEMS], int lane) {
    if constexpr (LPR == 32) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[j]),
                                                        __float_as_uint(v[j + 8]), false, false);
        v[j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
      }
      level<4, 8, 0x140>(v, lane);  // row mirror
      level<2, 4, 0x141>(v, lane);  // half-row mirror
      level<1, 2, 0x4E>(v, lane);   // quad xor 2
      v[0] += dpp<0xB1>(v[0]);      // quad xor 1: two lanes hold each total
    } else {
      level<8, 8, 0x140>(v, lane);
      level<4, 4, 0x141>(v, lane);
      level<2, 2, 0x4E>(v, lane);
      level<1, 1, 0xB1>(v, lane);
    }
  }
};

// The exact fold on the verify's tile layout (lane tid holds 16 bytes of
// every NT*16-byte item: state row it*RPI + tid/LPR, columns SV*(tid%LPR)
// onwards), for a row whose ring folds before its drafts are verified: the
// same recurrence, lazy decay and order as the commit's fold, entries
// 0..wn-1 from their raw inputs (k and v rows as stored in Ks, Vs; g and
// beta of entry i in lane i of gl, bl); the row dots are folded sums over
// the LPR lanes of a row (a row's lanes never span two waves) and each
// row's d goes to its lanes through dbuf.
template <typename IT, int V, int K, int ITEMS>
__device__ static inline void fold_steps_v(u32x4 (&sv)[ITEMS], const char* Ks, const char* Vs,
                                           float* dbuf, float gl, float bl, int wn, int tid) {
  using GS = GdnShape<V, K, true>;
  constexpr int SV = GS::SV, LPR = GS::LPR, RPI = GS::RPI;
  static_assert(ITEMS == GS::ITEMS, "verify tile layout");
  constexpr int QV = K / Elt<IT>::kPer16;
  constexpr long kIo = sizeof(IT);
  using RR = RowReduce<ITEMS, LPR>;
  static_assert(RR::NF == 1 && ITEMS % 4 == 0, "one row total per lane");
  const int c = tid % LPR;
  const int prow = tid / LPR;
  const int my_item = RR::item(0, tid);
  const bool writer = (c % RR::DUP) == 0;
  float S[ITEMS][SV];
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) Elt<float>::unpack(sv[it], S[it]);
  float gam = 1.f;
  for (int i = 0; i < wn; ++i) {
    const float gi = lane_value(gl, i), bi = lane_value(bl, i);
    float gn = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(gam * gi)));
    if (!(gn >= kLazyFloor && gn <= kLazyCeil)) {
#pragma unroll
      for (int it = 0; it < ITEMS; ++it)
#pragma unroll
        for (int e = 0; e < SV; ++e) S[it][e] = (S[it][e] * gam) * gi;
      gn = 1.f;
    }
    float kv[SV];
    LdsRead<IT>::template seg<SV>(Ks + (long)i * QV * 16, c * SV, kv);
    float part[ITEMS];
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      float x = 0.f;
#pragma unroll
      for (int e = 0; e < SV; ++e) x = fmaf(S[it][e], kv[e], x);
      part[it] = x;
    }
    FoldReduce<ITEMS, LPR>::run(part, tid);
    const float rinv = 1.f / gn;
    float* db = dbuf + (i & 1) * V;  // row it*RPI + prow at prow*ITEMS + it
    if (writer) {
      const float vr = LdsRead<IT>::one(Vs + (long)i * V * kIo, my_item * RPI + prow);
      db[prow * ITEMS + my_item] = (bi * fmaf(-gn, part[0], vr)) * rinv;
    }
    __builtin_amdgcn_wave_barrier();  // a row's d comes from its own wave's lanes
    float dv[ITEMS];
#pragma unroll
    for (int j = 0; j < ITEMS; j += 4)
      Elt<float>::unpack(*reinterpret_cast<const u32x4*>(db + prow * ITEMS + j), dv + j);
#pragma unroll
    for (int it = 0; it < ITEMS; ++it)
#pragma unroll
      for (int e = 0; e < SV; ++e) S[it][e] = fmaf(dv[it], kv[e], S[it][e]);
    gam = gn;
  }
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) {
#pragma unroll
    for (int e = 0; e < SV; ++e) S[it][e] *= gam;
    sv[it] = Elt<float>::pack(S[it]);
  }
}

// TM: draft capacity of the per-draft tables and loops (4 when T <= 4, else
// kMaxDraft), so a short draft chain does not pay for eight.  FL: rows with
// is_flush set first fold ring entries 0..w-1 into the state (the exact fold
// of the commit) and then verify their drafts at entries 0..T-1.
template <typename IT, typename OT, int V, int K, bool MF, int TM, bool FL>
__global__ void __launch_bounds__((GdnShape<V, K, true>::NT)) gdn_spec_verify_kernel(const SpecArgs a) {
  using GS = GdnShape<V, K, true>;
  using SG = VerifyStage<IT, V, K>;
  static_assert(!MF || (std::is_same<IT, bf16>::value && V == 128 && K == 128 && GS::NT == 256),
                "matrix-core products: bf16 inputs, V = K = 128, four waves");
  constexpr int SV = GS::SV, LPR = GS::LPR, NT = GS::NT, ITEMS = GS::ITEMS, RPI = GS::RPI;
  constexpr int QV = SG::QV, VV = SG::VV, DV = SG::DV;
  constexpr long kIo = sizeof(IT);
  using RR = RowReduce<ITEMS, LPR>;

  extern __shared__ __attribute__((aligned(16))) char lds[];
  // [i][t]: gamma_{i,t} (k_i . k_{w+t}) for i < w+t, gamma_{i,t} (k_i . q_t)
  // for i <= w+t; entry-major, so one entry's weights for all drafts are one
  // vector read
  __shared__ __attribute__((aligned(16))) float cK[64][TM];
  __shared__ __attribute__((aligned(16))) float cQ[64][TM];
  __shared__ float gamS[TM];    // Gamma_t = prod_{j <= w+t} g_j

  const int HV = a.v_heads, HK = a.k_heads, T = a.n_draft, L = a.ring_len;
  const int tile = xcd_tile(blockIdx.x, gridDim.x);
  const int b = tile / HV;
  const int hv = tile - b * HV;
  const int hk = hv / a.vpk;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int s = a.slot_idx[b];
  const int w_in = a.write_pos[b];
  const bool fold = FL && a.is_flush[b] != 0;
  int st = 0;
  if (s < 0 || s >= a.num_slots) st |= RSSM_ST_BAD_SLOT;
  if (w_in < 0 || (fold ? w_in > L : w_in + T > L)) st |= RSSM_ST_RING_OVERFLOW;
  const int w = fold ? 0 : w_in;    // committed entries the drafts are verified against
  const int wf = fold ? w_in : 0;   // entries folded into the state first
  if (st) {
    if (hv == 0 && tid == 0 && a.status) atomicOr(a.status, st);
    for (int e = tid; e < T * V; e += NT) {
      const int t = e / V;
      Elt<OT>::store1(a.o, ((long)(b * T + t) * HV + hv) * V + (e - t * V), __builtin_nanf(""));
    }
    return;
  }

  // ---- 1. every global read: the staged rows and gates, then the tile
  char* const tptr = (char*)a.state + ((long)s * HV + hv) * (long)V * K * 4;
  const rsrc_t trs = tile_rsrc(tptr, (uint32_t)(V * K * 4));
  const uint32_t lane_off = tid * 16;
  u32x4 sv[ITEMS];

  const long kring0 = ((long)s * HK + hk) * (long)L * K;
  const long dring0 = ((long)s * HV + hv) * (long)L * V;
  const long gring0 = ((long)s * HV + hv) * L;
  const int oV = SG::oV(T), oK = SG::oK(T), oD = SG::oD(T, L);
  for (int t = 0; t < T; ++t) {
    const long qk = ((long)(b * T + t) * HK + hk) * K;
    dma_rows(lds, t * QV, QV, (const char*)a.q + qk * kIo, wave, lane, NT);
    dma_rows(lds, oK + (w + t) * QV, QV, (const char*)a.k + qk * kIo, wave, lane, NT);
    dma_rows<true>(lds, oV + t * VV, VV,
                   (const char*)a.v + ((long)(b * T + t) * HV + hv) * V * kIo, wave, lane, NT);
  }
  if (w > 0) {
    dma_rows(lds, oK, w * QV, (const char*)a.k_ring + kring0 * kIo, wave, lane, NT);
    dma_rows<true>(lds, oD, w * DV, (const char*)(a.d_ring + dring0), wave, lane, NT);
  }
  // a folding row's raw k and v rows, after the verify's own regions
  char* const Fs = lds + verify_lds_bytes<IT, V, K, MF>(T, L);
  if constexpr (FL) {
    if (wf > 0) {
      dma_rows(Fs, 0, wf * QV, (const char*)a.k_ring + kring0 * kIo, wave, lane, NT);
      dma_rows<true>(Fs, L * QV, wf * VV, (const char*)a.v_ring + dring0 * kIo, wave, lane, NT);
    }
  }
  // gates: committed (or folded) entries from the ring, the drafts from the
  // inputs, all loaded by clamped indices (a load in a branch would make the
  // compiler wait for every staged row before the tile is even issued);
  // selected below
  const int td = lane - w < 0 ? 0 : (lane - w < T ? lane - w : T - 1);
  const float g_ring_l = a.g_ring[gring0 + (lane < w_in ? lane : 0)];
  const float b_ring_l = FL ? a.beta_ring[gring0 + (lane < wf ? lane : 0)] : 0.f;
  const float g_new_l = a.g[(long)(b * T + td) * HV + hv];
  const float b_new_l = a.beta[(long)(b * T + (lane < T ? lane : T - 1)) * HV + hv];
  // the tile last: step 2 needs only the staged rows and the gates, so it
  // runs while the tile is still in flight (the scheduling barriers keep the
  // issue order the counter wait below relies on)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int it = 0; it < ITEMS; ++it) sv[it] = bload16_nt(trs, lane_off, it * NT * 16);
  static_assert(ITEMS < 64, "the vmcnt field holds 6 bits");
  // everything but the ITEMS tile loads has landed: vmcnt <= ITEMS (bits 3:0
  // and 15:14 of the immediate), expcnt and lgkmcnt 0
  __builtin_amdgcn_s_waitcnt((ITEMS & 15) | ((ITEMS >> 4) << 14));
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  if constexpr (FL) {
    if (wf > 0) {
      // fold ring entries 0..wf-1 into the tile (its loads are waited for at
      // the first use), store it; the drafts then see the folded state
      fold_steps_v<IT, V, K>(sv, Fs, Fs + (long)L * QV * 16,
                             reinterpret_cast<float*>(Fs + (long)L * (QV + VV) * 16), g_ring_l,
                             b_ring_l, wf, tid);
#pragma unroll
      for (int it = 0; it < ITEMS; ++it)
        st16_stream(tptr, (long)lane_off + it * NT * 16, sv[it]);
    }
  }
  // gate of ring entry `lane` (committed entries, then the drafts); 1 past them
  const float gl = lane < w ? g_ring_l : (lane < w + T ? g_new_l : 1.f);
  const float bl = lane < T ? b_new_l : 0.f;

  const char* Qs = lds;
  const char* Vs = lds + (long)oV * 16;
  const char* Ks = lds + (long)oK * 16;
  float* Ds = reinterpret_cast<float*>(lds + (long)oD * 16);

  // ---- 2. gate products and weighted dots of every draft (draft t on wave
  // t mod (waves))
  {
    constexpr int EPL = K / 16;
    constexpr int NW = NT / 64;
    const int q16 = lane & 15;
    for (int t = wave; t < T; t += NW) {
      const int p = w + t;
      const float gt = lane <= p ? gl : 1.f;
      const float gam = L <= 16 ? row16_suffix_product_exclusive(gt)
                                : wave_suffix_product_exclusive(gt, lane);
      if (lane == 0) gamS[t] = gt * gam;
      SegDot<IT, EPL> kp, qt;
      kp.load(Ks + (long)p * QV * 16, q16 * EPL);
      qt.load(Qs + (long)t * QV * 16, q16 * EPL);
      float kk = 0.f, kq = 0.f;
      for (int pass = 0; pass * 4 <= p; ++pass) {
        const int i = pass * 4 + (lane >> 4);  // rows past p: unused values
        SegDot<IT, EPL> ki;
        ki.load(Ks + (long)i * QV * 16, q16 * EPL);
        float a1 = group_sum<16>(ki.dot(kp));
        float a2 = group_sum<16>(ki.dot(qt));
        a1 = __shfl(a1, (lane & 3) * 16, 64);
        a2 = __shfl(a2, (lane & 3) * 16, 64);
        if ((lane >> 2) == pass) {
          kk = a1;
          kq = a2;
        }
      }
      cK[lane][t] = lane < p ? gam * kk : 0.f;
      cQ[lane][t] = lane <= p ? gam * kq : 0.f;
    }
  }
  // (no barrier here: only the draft walk reads cK, cQ and gamS; step 3
  // reads the staged rows and the tile and writes per-wave LDS regions, so
  // each wave starts it as soon as its own tile has landed, and the barrier
  // before the walk covers both steps)

  // ---- 4 (per state row, the drafts in order), given S0.k_{w+t}, S0.q_t
  auto draft_row = [&](int vr, const float* pkv, const float* pqv, bool writer) {
    float hist_k[TM], hist_q[TM];  // committed-entry terms per draft
#pragma unroll
    for (int t = 0; t < TM; ++t) hist_k[t] = hist_q[t] = 0.f;
    for (int i = 0; i < w; ++i) {
      const float di = Ds[i * V + vr];
      float ck[TM], cq[TM];
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        ck[t] = cK[i][t];
        cq[t] = cQ[i][t];
      }
#pragma unroll
      for (int t = 0; t < TM; ++t) {  // sums past T are never used
        hist_k[t] = fmaf(ck[t], di, hist_k[t]);
        hist_q[t] = fmaf(cq[t], di, hist_q[t]);
      }
    }
    float dn[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      dn[t] = 0.f;
      if (t < T) {
        const float G = gamS[t];
        float pred = fmaf(G, pkv[t], hist_k[t]);
#pragma unroll
        for (int u = 0; u < t; ++u) pred = fmaf(cK[w + u][t], dn[u], pred);
        dn[t] = lane_value(bl, t) * (LdsRead<IT>::one(Vs + (long)t * VV * 16, vr) - pred);
        float out = fmaf(G, pqv[t], hist_q[t]);
#pragma unroll
        for (int u = 0; u <= t; ++u) out = fmaf(cQ[w + u][t], dn[u], out);
        if (writer) {
          Elt<OT>::store1(a.o, ((long)(b * T + t) * HV + hv) * V + vr, a.scale * out);
          Ds[(w + t) * V + vr] = dn[t];
        }
      }
    }
  };

  if constexpr (MF) {
    // ---- 3. D[m][row] = sum_k A[m][k] S0[row][k] on the matrix cores, A =
    // (k_w .. k_{w+T-1}, q_0 .. q_{T-1}, zero rows) exact in bf16, S0 split
    // into bf16 hi + lo halves (two products per block).  A wave's block of
    // 16 rows x 32 columns goes through its LDS region into the B operand
    // layout (lane l: row l%16, columns 8*(l/16) ..+8) while the tile loads
    // stay 1 KB contiguous per instruction.
    float* const Wb = reinterpret_cast<float*>(lds + (long)SG::chunks(T, L) * 16) +
                      wave * VerifyMfma::kRegionFloats;
    constexpr int PI = VerifyMfma::kPitch;
    const int h = lane >> 5, q32 = lane & 31;  // this lane's row of the pair, 16-byte column
    const int m = lane & 15, g4 = lane >> 4;   // operand row / column group
    const char* arow = m < T ? Ks + (long)(w + m) * QV * 16
                             : (m < 2 * T ? Qs + (long)(m - T) * QV * 16 : nullptr);
    f32x4 acc[2];
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2) {
      acc[b2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        if ((q32 >> 3) == kb) {
#pragma unroll
          for (int i = 0; i < 8; ++i)
            *reinterpret_cast<u32x4*>(Wb + (2 * i + h) * PI + 4 * (q32 & 7)) = sv[8 * b2 + i];
        }
        __builtin_amdgcn_wave_barrier();
        const float* src = Wb + m * PI + 8 * g4;
        float f[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = src[e];
        u32x4 hi, lo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t hb = bf16_pair(f[2 * e], f[2 * e + 1]);
          hi[e] = hb;
          lo[e] = bf16_pair(f[2 * e] - __uint_as_float(hb << 16),
                            f[2 * e + 1] - __uint_as_float(hb & 0xffff0000u));
        }
        const u32x4 afr = arow ? *reinterpret_cast<const u32x4*>(arow + (32 * kb + 8 * g4) * 2)
                               : u32x4{0u, 0u, 0u, 0u};
        acc[b2] = mfma16x16x32_bf16(afr, hi, acc[b2]);
        acc[b2] = mfma16x16x32_bf16(afr, lo, acc[b2]);
        __builtin_amdgcn_wave_barrier();
      }
    }
    // lane holds products 4*g4 + r of the wave's local row 16*b2 + m
#pragma unroll
    for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
      for (int r = 0; r < 4; ++r) Wb[(16 * b2 + m) * 16 + 4 * g4 + r] = acc[b2][r];
    __syncthreads();
    for (int vr = tid; vr < V; vr += NT) {
      // row vr = it*8 + 2*w' + h' lives in wave w' as local row 2*it + h'
      const float* Pr = reinterpret_cast<const float*>(lds + (long)SG::chunks(T, L) * 16) +
                        ((vr & 7) >> 1) * VerifyMfma::kRegionFloats +
                        (2 * (vr >> 3) + (vr & 1)) * 16;
      float pkv[TM], pqv[TM];
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        pkv[t] = t < T ? Pr[t] : 0.f;
        pqv[t] = t < T ? Pr[T + t] : 0.f;
      }
      draft_row(vr, pkv, pqv, true);
    }
  } else {
    // ---- 3. S0 . k_{w+t} and S0 . q_t for this lane's state rows
    const int c = tid % LPR;
    const int prow = tid / LPR;
    float pk[TM][RR::NF], pq[TM][RR::NF];
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      if (t < T) {
        float kseg[SV], qseg[SV];
        LdsRead<IT>::template seg<SV>(Ks + (long)(w + t) * QV * 16, c * SV, kseg);
        LdsRead<IT>::template seg<SV>(Qs + (long)t * QV * 16, c * SV, qseg);
        float a1[ITEMS], a2[ITEMS];
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
          float sf[SV];
          Elt<float>::unpack(sv[it], sf);
          float x1 = 0.f, x2 = 0.f;
#pragma unroll
          for (int j = 0; j < SV; ++j) {
            x1 = fmaf(sf[j], kseg[j], x1);
            x2 = fmaf(sf[j], qseg[j], x2);
          }
          a1[it] = x1;
          a2[it] = x2;
        }
        RR::run(a1, tid);
        RR::run(a2, tid);
#pragma unroll
        for (int j = 0; j < RR::NF; ++j) {
          pk[t][j] = a1[j];
          pq[t][j] = a2[j];
        }
      }
    }
    const bool writer = (c % RR::DUP) == 0;
    __syncthreads();  // the weighted dots of step 2 are in LDS
#pragma unroll
    for (int j = 0; j < RR::NF; ++j) {
      float pkv[TM], pqv[TM];
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        pkv[t] = t < T ? pk[t][j] : 0.f;
        pqv[t] = t < T ? pq[t][j] : 0.f;
      }
      draft_row(RR::item(j, tid) * RPI + prow, pkv, pqv, writer);
    }
  }
  __syncthreads();  // the drafts' d rows are in LDS

  // ---- 5. ring entries w..w+T-1 of d, v and k (one writer per key head):
  // each array's T rows are one contiguous run in the ring, written by
  // consecutive lanes with non-temporal stores (written this way, scattered
  // ring writes inside the tile read stream cost a third of the per-row
  // layout); then g and beta.  The deferred-fold rounds (FL) write the d
  // rows only: the advance writes the accepted drafts' v, k, g and beta
  // rows from the inputs, outside this read stream (and after every value
  // head of a folding row has read its old k rows).
  const bool k_writer = !FL && (hv % a.vpk) == 0;
  {
    const int nd = T * DV, nv = FL ? 0 : T * VV, nk = k_writer ? T * QV : 0;
    for (int e = tid; e < nd + nv + nk; e += NT) {
      if (e < nd) {
        const u32x4 x = *reinterpret_cast<const u32x4*>(lds + ((long)oD + w * DV + e) * 16);
        st16_stream(a.d_ring, (dring0 + (long)w * V) * 4 + (long)e * 16, x);
      } else if (e < nd + nv) {
        const int u = e - nd;  // draft rows t = u / VV, staged contiguously
        const u32x4 x = *reinterpret_cast<const u32x4*>(Vs + (long)u * 16);
        st16_stream(a.v_ring, (dring0 + (long)w * V) * kIo + (long)u * 16, x);
      } else {
        const int u = e - nd - nv;
        const u32x4 x = *reinterpret_cast<const u32x4*>(Ks + ((long)w * QV + u) * 16);
        st16_stream(a.k_ring, (kring0 + (long)w * K) * kIo + (long)u * 16, x);
      }
    }
  }
  if (FL) return;
  if (wave == 0) {
    if (lane >= w && lane < w + T) a.g_ring[gring0 + lane] = gl;
    if (lane < T) a.beta_ring[gring0 + w + lane] = bl;
  }
}

// Commit LDS: [k rows 0..L-1 as fp32 | v rows 0..L-1 as stored]; then 2*V
// floats for the d of the step in flight (double buffered).
template <typename IT, int V, int K>
struct CommitStage {
  static constexpr int VV = V / Elt<IT>::kPer16;  // 16-byte chunks of a v row
  static constexpr size_t oV(int L) { return (size_t)L * K * 4; }
  static constexpr size_t oD(int L) { return oV(L) + (size_t)L * V * sizeof(IT); }
  static constexpr size_t bytes(int L) { return oD(L) + 2 * V * 4; }
};

// Lanes of a fold tile: lane m of the eight lanes of group g holds 16 bytes
// of each of the NSEG 128-byte segments of RPL state rows (rows
// wave*RPW + 8*rr + g), so each load or store instruction moves eight whole
// 128-byte segments and a row's dot with k is a sum over eight lanes.
template <int V, int K, int NT>
struct FoldLayout {
  static constexpr int NSEG = K / 32;
  static constexpr int ITEMS = V * K / 4 / NT;
  static constexpr int RPL = ITEMS / NSEG;
  static constexpr int RPW = 8 * RPL;
  static_assert(RPW * (NT / 64) == V && RPL * NSEG == ITEMS, "fold tile layout");
};

// Sums of RPL per-lane partials over the eight lanes of each group, folded:
// every level halves the partials a lane keeps (partners: mirror within the
// 8 lanes, then lane xor 2, lane xor 1, all by DPP), so lane m ends with the
// total of partial item(m), held by DUP lanes.
template <int RPL>
struct Reduce8 {
  static constexpr int LV = RPL >= 8 ? 3 : (RPL >= 4 ? 2 : (RPL >= 2 ? 1 : 0));
  static constexpr int DUP = 8 >> LV;
  template <int O>
  __device__ static inline float partner(float x) {
    constexpr int ctrl = O == 4 ? 0x141 : (O == 2 ? 0x4E : 0xB1);  // half-row mirror, quad perms
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), ctrl, 0xF, 0xF, false));
  }
  template <int LVL>
  __device__ static inline void level(float (&v)[RPL], int m) {
    if constexpr (LVL < 3) {
      constexpr int O = 4 >> LVL;
      if constexpr (LVL < LV) {
        constexpr int h = (RPL >> LVL) >> 1;
        const bool up = (m & O) != 0;
#pragma unroll
        for (int j = 0; j < h; ++j) {
          const float send = up ? v[j] : v[j + h];
          const float keep = up ? v[j + h] : v[j];
          v[j] = keep + partner<O>(send);
        }
      } else {
        v[0] += partner<O>(v[0]);
      }
      level<LVL + 1>(v, m);
    }
  }
  __device__ static inline void run(float (&v)[RPL], int m) { level<0>(v, m); }
  __device__ static inline int item(int m) {
    int it = 0;
    if (LV > 0 && (m & 4)) it += RPL / 2;
    if (LV > 1 && (m & 2)) it += RPL / 4;
    if (LV > 2 && (m & 1)) it += RPL / 8;
    return it;
  }
};

// The entry loop of a fold: this lane's rows S of the tile, entries 0..wn-1
// in order (k rows as fp32 in K32, v rows as stored in Vs, g and beta of
// entry i in lane i of gl, bl), the result left in S.
template <typename IT, int V, int K, int NT, int RPL, int E>
__device__ static inline void fold_steps(float (&S)[RPL][E], const float* K32, const char* Vs,
                                         float* dbuf, float gl, float bl, int wn, int tid) {
  using FL = FoldLayout<V, K, NT>;
  using RD = Reduce8<RPL>;
  static_assert(RPL == FL::RPL && E == FL::NSEG * 4, "fold registers");
  constexpr int NSEG = FL::NSEG, RPW = FL::RPW;
  constexpr long kIo = sizeof(IT);
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 7;
  const int row0 = wave * RPW + (lane >> 3);
  const int my_row = row0 + 8 * RD::item(m);  // the row whose total this lane ends with
  const bool writer = (m % RD::DUP) == 0;
  float gam = 1.f;
  for (int i = 0; i < wn; ++i) {
    const float gi = lane_value(gl, i), bi = lane_value(bl, i);
    float gn = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(gam * gi)));
    if (!(gn >= kLazyFloor && gn <= kLazyCeil)) {
#pragma unroll
      for (int rr = 0; rr < RPL; ++rr)
#pragma unroll
        for (int e = 0; e < NSEG * 4; ++e) S[rr][e] = (S[rr][e] * gam) * gi;
      gn = 1.f;
    }
    float kv[NSEG * 4];
#pragma unroll
    for (int sg = 0; sg < NSEG; ++sg)
      Elt<float>::unpack(*reinterpret_cast<const u32x4*>(K32 + (long)i * K + sg * 32 + m * 4),
                         &kv[sg * 4]);
    float part[RPL];
#pragma unroll
    for (int rr = 0; rr < RPL; ++rr) {
      float x = 0.f;
#pragma unroll
      for (int e = 0; e < NSEG * 4; ++e) x = fmaf(S[rr][e], kv[e], x);
      part[rr] = x;
    }
    RD::run(part, m);
    const float rinv = 1.f / gn;
    float* db = dbuf + (i & 1) * V;
    if (writer) {
      const float vr = LdsRead<IT>::one(Vs + (long)i * V * kIo, my_row);
      db[my_row] = (bi * fmaf(-gn, part[0], vr)) * rinv;
    }
    // the d values of a wave's state rows come from that wave's own lanes
    // (a row's lanes never span two waves) and one wave's LDS operations
    // complete in order, so no workgroup barrier is needed here
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int rr = 0; rr < RPL; ++rr) {
      const float dv = db[row0 + 8 * rr];
#pragma unroll
      for (int e = 0; e < NSEG * 4; ++e) S[rr][e] = fmaf(dv, kv[e], S[rr][e]);
    }
    gam = gn;
  }
#pragma unroll
  for (int rr = 0; rr < RPL; ++rr)
#pragma unroll
    for (int e = 0; e < NSEG * 4; ++e) S[rr][e] *= gam;
}

// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector
// memory operations are outstanding and leaves the other counters alone.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// Barrier for LDS only: this wave's LDS operations complete, s_barrier, then
// an acquire fence so that no LDS access moves above it (the release fence
// of __syncthreads() would also wait for the tile loads still in flight).
__device__ static inline void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(63) & ~(15 << 8));  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Exact fold of one (slot, value head) tile: the recurrence over ring entries
// 0..wn-1 from their raw inputs, in order, the state held in fp32 registers.
// Every thread of the workgroup calls it; the staged rows go to `stage`.
template <typename IT, int V, int K>
__device__ static inline void fold_tile(const SpecArgs& a, int s, int hv, int wn, char* stage,
                                        int tid) {
  using GS = GdnShape<V, K, true>;
  using FL = FoldLayout<V, K, GS::NT>;
  using SG = CommitStage<IT, V, K>;
  constexpr int NT = GS::NT, ITEMS = FL::ITEMS, NSEG = FL::NSEG, RPL = FL::RPL, RPW = FL::RPW;
  constexpr int EPV = Elt<IT>::kPer16;
  constexpr long kIo = sizeof(IT);
  const int HV = a.v_heads, HK = a.k_heads, L = a.ring_len;
  const int hk = hv / a.vpk;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 7;
  const int row0 = wave * RPW + (lane >> 3);  // this lane's rows: row0 + 8*rr

  char* const tptr = (char*)a.state + ((long)s * HV + hv) * (long)V * K * 4;
  const rsrc_t trs = tile_rsrc(tptr, (uint32_t)(V * K * 4));
  const uint32_t voff = (uint32_t)(row0 * K * 4 + m * 16);
  const long kring0 = ((long)s * HK + hk) * (long)L * K;
  const long vring0 = ((long)s * HV + hv) * (long)L * V;
  const long gring0 = ((long)s * HV + hv) * L;
  // the ring rows first (v rows to LDS, k rows into registers, gates by a
  // clamped index: lanes at or past wn are never read), then the tile, so
  // that waiting until only the tile's ITEMS loads are outstanding waits
  // for exactly the ring rows (the k rows follow the DMA loop, so their own
  // wait counts only the loads after them)
  dma_rows(stage, (int)(SG::oV(L) / 16), wn * SG::VV, (const char*)a.v_ring + vring0 * kIo,
           wave, lane, NT);
  constexpr int KPT = (64 * K / EPV + NT - 1) / NT;  // k-ring vectors per thread, L <= 64
  u32x4 kr[KPT];
  const int nkv = wn * K / EPV;
#pragma unroll
  for (int q = 0; q < KPT; ++q) {
    const int e = tid + q * NT < nkv ? tid + q * NT : nkv - 1;  // clamped: no load in a branch
    kr[q] = ld16(a.k_ring, (kring0 + (long)e * EPV) * kIo);
  }
  const int li = lane < wn ? lane : 0;
  const float gl = a.g_ring[gring0 + li];
  const float bl = a.beta_ring[gring0 + li];
  __builtin_amdgcn_sched_barrier(0);
  u32x4 sv[ITEMS];
#pragma unroll
  for (int rr = 0; rr < RPL; ++rr)
#pragma unroll
    for (int sg = 0; sg < NSEG; ++sg)
      sv[rr * NSEG + sg] = bload16_nt(trs, voff, rr * 8 * K * 4 + sg * 128);
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(ITEMS));  // the ring rows (older than the tile)
  __builtin_amdgcn_sched_barrier(0);
  // k rows 0..wn-1 to LDS as fp32
  float* const K32 = reinterpret_cast<float*>(stage);
  // (lanes past the last vector write that vector again: same values, no branch)
#pragma unroll
  for (int q = 0; q < KPT; ++q) {
    const int e = tid + q * NT < nkv ? tid + q * NT : nkv - 1;
    float f[EPV];
    Elt<IT>::unpack(kr[q], f);
#pragma unroll
    for (int j = 0; j < EPV; j += 4)
      *reinterpret_cast<u32x4*>(K32 + (long)e * EPV + j) = Elt<float>::pack(f + j);
  }
  lds_barrier();

  float S[RPL][NSEG * 4];
#pragma unroll
  for (int rr = 0; rr < RPL; ++rr)
#pragma unroll
    for (int sg = 0; sg < NSEG; ++sg) Elt<float>::unpack(sv[rr * NSEG + sg], &S[rr][sg * 4]);
  fold_steps<IT, V, K, NT>(S, K32, stage + SG::oV(L),
                           reinterpret_cast<float*>(stage + SG::oD(L)), gl, bl, wn, tid);
#pragma unroll
  for (int rr = 0; rr < RPL; ++rr)
#pragma unroll
    for (int sg = 0; sg < NSEG; ++sg)
      st16_stream(tptr, (long)voff + rr * 8 * K * 4 + sg * 128, Elt<float>::pack(&S[rr][sg * 4]));
}

template <typename IT, int V, int K>
__global__ void __launch_bounds__((GdnShape<V, K, true>::NT)) gdn_spec_commit_kernel(const SpecArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int HV = a.v_heads;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  if (!a.fold_tasks) {
    // one workgroup per (row, value head), rows in batch order
    const int tile = xcd_tile(blockIdx.x, gridDim.x);
    const int b = tile / HV;
    const int hv = tile - b * HV;
    const int s = a.slot_idx[b];
    const CommitRow cr = commit_row(s, a.write_pos[b], a.accepted[b],
                                    a.force_flush && a.force_flush[b], a);
    if (hv == 0 && tid == 0) {
      if (a.next_write_pos) a.next_write_pos[b] = cr.flush ? 0 : cr.wn;
      if (a.flushed) a.flushed[b] = cr.flush ? 1 : 0;
      if (cr.st && a.status) atomicOr(a.status, cr.st);
    }
    if (cr.flush && cr.wn > 0) fold_tile<IT, V, K>(a, s, hv, cr.wn, lds, tid);
    return;
  }

  // Task list: wave 0 reads every row's (slot, cursor, accepted, force) in one
  // round trip, lane l rows 8l..8l+7, and lists the folding rows' slot and
  // cursor in LDS; workgroup 0 also writes every row's cursor outputs.  The
  // fold tasks (folding row f, value head hv), f-major, are taken by
  // workgroups j, j + P, ... of the P-workgroup grid; with P a multiple of 8
  // each XCD receives the same share of them.
  __shared__ int fold_slot[kTaskRows];
  __shared__ uint8_t fold_wn[kTaskRows];
  __shared__ int fold_count;
  const int nb = a.n_rows;
  if (wave == 0) {
    const int r0 = 8 * lane;
    // every load before any store (the outputs could alias the inputs as far
    // as the compiler knows), so the rows cost one round trip
    // (without force flags the flag loads read bytes of slot_idx, in bounds
    // for every row, and are masked off: no load sits behind a branch)
    const bool has_force = a.force_flush != nullptr;
    const uint8_t* const fsrc =
        has_force ? a.force_flush : reinterpret_cast<const uint8_t*>(a.slot_idx);
    int sk[8], wk[8], ak[8], fk[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int r = r0 + k < nb ? r0 + k : nb - 1;
      sk[k] = a.slot_idx[r];
      wk[k] = a.write_pos[r];
      ak[k] = a.accepted[r];
      fk[k] = fsrc[r];
    }
    bool fb[8];
    int st = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int r = r0 + k;
      fb[k] = false;
      if (r < nb) {
        const CommitRow cr = commit_row(sk[k], wk[k], ak[k], has_force && fk[k] != 0, a);
        fb[k] = cr.flush && cr.wn > 0;
        wk[k] = cr.wn;
        st |= cr.st;
        if (blockIdx.x == 0) {
          if (a.next_write_pos) a.next_write_pos[r] = cr.flush ? 0 : cr.wn;
          if (a.flushed) a.flushed[r] = cr.flush ? 1 : 0;
        }
      }
    }
    int base = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint64_t m = __ballot(fb[k]);
      if (fb[k]) {
        const int f = base + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                       __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        fold_slot[f] = sk[k];
        fold_wn[f] = (uint8_t)wk[k];
      }
      base += __popcll(m);
    }
    if (lane == 0) fold_count = base;
    if (blockIdx.x == 0 && a.status && __ballot(st != 0)) {
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) st |= __shfl_xor(st, o, 64);
      if (lane == 0) atomicOr(a.status, st);
    }
  }
  __syncthreads();
  const int ntask = fold_count * HV;
  for (int t = blockIdx.x; t < ntask; t += gridDim.x) {
    const int f = t / HV;
    const int hv = t - f * HV;
    if (t != (int)blockIdx.x) __syncthreads();  // every wave is done with the staged rows
    fold_tile<IT, V, K>(a, fold_slot[f], hv, fold_wn[f], lds, tid);
  }
}

// Cursor advance of the deferred-fold rounds, one workgroup per row: a row
// that folded in this round's verify starts from entry 0, then keeps its
// accepted drafts (commit_row); the next verify folds it when the flag is
// set.  The kept drafts' v, k, g and beta rows go from this round's inputs
// to their ring entries here (the verify wrote their d rows): written by a
// launch of their own they do not interrupt the verify's tile reads, only
// the kept drafts are written, and no value head of a folding row can
// still be reading the old k rows of its key head.
template <typename IT, int V, int K>
__global__ void __launch_bounds__(256) gdn_spec_advance_kernel(const SpecArgs a) {
  constexpr int EPV = Elt<IT>::kPer16;
  constexpr int QV = K / EPV, VV = V / EPV;
  constexpr int NT = 256, B = 8;
  constexpr long kIo = sizeof(IT);
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int T = a.n_draft, L = a.ring_len, HK = a.k_heads, HV = a.v_heads;
  const int s = a.slot_idx[r];
  const bool folded = a.is_flush[r] != 0;
  const int w = folded ? 0 : a.write_pos[r];
  const CommitRow cr = commit_row(s, w, a.accepted[r], a.force_flush && a.force_flush[r], a);
  if (tid == 0) {
    a.next_write_pos[r] = cr.wn;
    a.next_is_flush[r] = cr.flush ? 1 : 0;
    if (cr.st && a.status) atomicOr(a.status, cr.st);
  }
  const int w0 = w < 0 ? 0 : (w > L ? L : w);
  // kept drafts (entries w0..wn-1, within the ring; at most the T inputs
  // even when accepted is out of range)
  const int na = cr.wn - w0 < T ? cr.wn - w0 : T;
  if (na <= 0 || s < 0 || s >= a.num_slots) return;
  // vectors: v rows [t][hv] then k rows [t][hk]; scalars: g and beta [t][hv];
  // every load of a batch (clamped indices, no load in a branch) before its
  // stores
  const int nvv = na * HV * VV, nvec = nvv + na * HK * QV, nsc = na * HV;
  for (int i = 0; i * B * NT < nvec || i * NT < nsc; ++i) {
    const int u0 = i * B * NT, s0 = i * NT;  // this batch's vectors and scalars
    u32x4 x[B];
    long dst[B];
    bool isv[B];
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int uj = u0 + j * NT + tid;
      const int u = uj < nvec ? uj : nvec - 1;
      isv[j] = u < nvv;
      if (u < nvv) {
        const int t = u / (HV * VV);
        const int hv = (u - t * HV * VV) / VV;
        const int c = u - (t * HV + hv) * VV;
        x[j] = ld16(a.v, (((long)(r * T + t) * HV + hv) * V) * kIo + (long)c * 16);
        dst[j] = ((((long)s * HV + hv) * L + w0 + t) * V) * kIo + (long)c * 16;
      } else {
        const int uk = u - nvv;
        const int t = uk / (HK * QV);
        const int hk = (uk - t * HK * QV) / QV;
        const int c = uk - (t * HK + hk) * QV;
        x[j] = ld16(a.k, (((long)(r * T + t) * HK + hk) * K) * kIo + (long)c * 16);
        dst[j] = ((((long)s * HK + hk) * L + w0 + t) * K) * kIo + (long)c * 16;
      }
    }
    const int us = s0 + tid < nsc ? s0 + tid : nsc - 1;
    const int ts = us / HV, hs = us - ts * HV;
    const long ssrc = (long)(r * T + ts) * HV + hs;
    const float gv = a.g[ssrc], bv = a.beta[ssrc];
#pragma unroll
    for (int j = 0; j < B; ++j)
      if (u0 + j * NT + tid < nvec) st16(isv[j] ? a.v_ring : a.k_ring, dst[j], x[j]);
    if (s0 + tid < nsc) {
      const long sdst = ((long)s * HV + hs) * L + w0 + ts;
      a.g_ring[sdst] = gv;
      a.beta_ring[sdst] = bv;
    }
  }
}

// bf16 inputs at V = K = 128 take the matrix-core products when the extra
// LDS fits; otherwise (fp32 inputs, other shapes, the largest rings) the
// vector path.
template <typename IT, typename OT, int V, int K, int TM, bool FL>
static int launch_verify_tm(const SpecArgs& a, int batch, hipStream_t stream) {
  constexpr int NT = GdnShape<V, K, true>::NT;
  const size_t fixed = (2 * TM * 64 + TM) * sizeof(float);
  const unsigned grid = (unsigned)((long)batch * a.v_heads);
  // a folding row stages its raw ring rows after the verify's regions
  const size_t fold = FL ? verify_fold_bytes<IT, V, K>(a.ring_len) : 0;
  if constexpr (std::is_same<IT, bf16>::value && V == 128 && K == 128 && NT == 256) {
    const size_t lds = verify_lds_bytes<IT, V, K, true>(a.n_draft, a.ring_len) + fold;
    if (lds + fixed <= kMaxLds)
      return launch_kernel(
          reinterpret_cast<const void*>(&gdn_spec_verify_kernel<IT, OT, V, K, true, TM, FL>),
          grid, NT, lds, stream, a);
  }
  const size_t lds = verify_lds_bytes<IT, V, K, false>(a.n_draft, a.ring_len) + fold;
  if (lds + fixed > kMaxLds) return RSSM_ESHAPE;  // staged rows must fit one workgroup's LDS
  return launch_kernel(
      reinterpret_cast<const void*>(&gdn_spec_verify_kernel<IT, OT, V, K, false, TM, FL>), grid,
      NT, lds, stream, a);
}

template <typename IT, typename OT, int V, int K>
static int launch_verify(const SpecArgs& a, int batch, hipStream_t stream) {
  if (a.is_flush)
    return a.n_draft <= 4 ? launch_verify_tm<IT, OT, V, K, 4, true>(a, batch, stream)
                          : launch_verify_tm<IT, OT, V, K, kMaxDraft, true>(a, batch, stream);
  return a.n_draft <= 4 ? launch_verify_tm<IT, OT, V, K, 4, false>(a, batch, stream)
                        : launch_verify_tm<IT, OT, V, K, kMaxDraft, false>(a, batch, stream);
}

// Grid of the task-list commit: enough resident workgroups to keep every CU
// busy with the folds of a typical round, a multiple of 8 (one share per XCD).
constexpr long kCommitGrid = 1024;

template <typename IT, int V, int K>
static int launch_commit(const SpecArgs& a, int batch, hipStream_t stream) {
  const size_t lds = CommitStage<IT, V, K>::bytes(a.ring_len);
  if (lds > kMaxLds) return RSSM_ESHAPE;
  const long tiles = (long)batch * a.v_heads;
  const long grid = a.fold_tasks ? (tiles < kCommitGrid ? tiles : kCommitGrid) : tiles;
  return launch_kernel(reinterpret_cast<const void*>(&gdn_spec_commit_kernel<IT, V, K>),
                       (unsigned)grid, GdnShape<V, K, true>::NT, lds, stream, a);
}

template <typename IT, typename OT>
static int verify_shape(const SpecArgs& a, const rssm_gdn_dims& d, hipStream_t s) {
  if (d.dv == 128 && d.dk == 128) return launch_verify<IT, OT, 128, 128>(a, d.batch, s);
  if (d.dv == 64 && d.dk == 64) return launch_verify<IT, OT, 64, 64>(a, d.batch, s);
  if (d.dv == 128 && d.dk == 64) return launch_verify<IT, OT, 128, 64>(a, d.batch, s);
  if (d.dv == 64 && d.dk == 128) return launch_verify<IT, OT, 64, 128>(a, d.batch, s);
  return RSSM_ESHAPE;
}

template <typename IT>
static int commit_shape(const SpecArgs& a, const rssm_gdn_dims& d, hipStream_t s) {
  if (d.dv == 128 && d.dk == 128) return launch_commit<IT, 128, 128>(a, d.batch, s);
  if (d.dv == 64 && d.dk == 64) return launch_commit<IT, 64, 64>(a, d.batch, s);
  if (d.dv == 128 && d.dk == 64) return launch_commit<IT, 128, 64>(a, d.batch, s);
  if (d.dv == 64 && d.dk == 128) return launch_commit<IT, 64, 128>(a, d.batch, s);
  return RSSM_ESHAPE;
}

template <typename IT>
static int launch_advance(const SpecArgs& a, const rssm_gdn_dims& d, hipStream_t s) {
  const void* fn;
  if (d.dv == 128 && d.dk == 128)
    fn = reinterpret_cast<const void*>(&gdn_spec_advance_kernel<IT, 128, 128>);
  else if (d.dv == 64 && d.dk == 64)
    fn = reinterpret_cast<const void*>(&gdn_spec_advance_kernel<IT, 64, 64>);
  else if (d.dv == 128 && d.dk == 64)
    fn = reinterpret_cast<const void*>(&gdn_spec_advance_kernel<IT, 128, 64>);
  else
    fn = reinterpret_cast<const void*>(&gdn_spec_advance_kernel<IT, 64, 128>);
  return launch_kernel(fn, (unsigned)d.batch, 256, 0, s, a);
}

static int spec_check(const rssm_gdn_dims* d, int32_t n_draft) {
  if (!d) return RSSM_EINVAL;
  if (d->batch < 0 || d->k_heads < 1 || d->v_heads < 1 || d->v_heads % d->k_heads ||
      d->num_slots < 1)
    return RSSM_EINVAL;
  if ((long)d->batch * d->v_heads > 0x7fffffffL) return RSSM_EINVAL;
  if (d->state_dtype != RSSM_F32 || !valid_dtype(d->io_dtype) || !valid_dtype(d->out_dtype))
    return RSSM_EDTYPE;
  if (!((d->dk == 64 || d->dk == 128) && (d->dv == 64 || d->dv == 128))) return RSSM_ESHAPE;
  if (n_draft < 1 || n_draft > kMaxDraft) return RSSM_ESHAPE;
  if (d->ring_len < 2 * n_draft || d->ring_len > 64) return RSSM_ESHAPE;
  return RSSM_OK;
}

static SpecArgs spec_args(const rssm_gdn_dims* d, int32_t n_draft) {
  SpecArgs a{};
  a.k_heads = d->k_heads;
  a.v_heads = d->v_heads;
  a.vpk = d->v_heads / d->k_heads;
  a.ring_len = d->ring_len;
  a.num_slots = d->num_slots;
  a.n_draft = n_draft;
  a.scale = d->scale > 0.f ? d->scale : 1.0f / sqrtf((float)d->dk);
  return a;
}

}  // namespace rssm

using namespace rssm;

static int spec_verify(const rssm_gdn_dims* dims, int32_t n_draft, const void* state,
                       float* d_ring, void* k_ring, float* g_ring, void* v_ring,
                       float* beta_ring, const int32_t* slot_idx, const int32_t* write_pos,
                       const uint8_t* is_flush, const void* q, const void* k, const void* v,
                       const float* g, const float* beta, void* o, int32_t* status,
                       hipStream_t stream) {
  int rc = spec_check(dims, n_draft);
  if (rc) return rc;
  if (dims->batch == 0) return RSSM_OK;
  if (!state || !d_ring || !k_ring || !g_ring || !v_ring || !beta_ring || !slot_idx ||
      !write_pos || !q || !k || !v || !g || !beta || !o)
    return RSSM_EINVAL;
  if (!aligned16(state) || !aligned16(d_ring) || !aligned16(k_ring) || !aligned16(v_ring) ||
      !aligned16(q) || !aligned16(k) || !aligned16(v))
    return RSSM_EINVAL;
  SpecArgs a = spec_args(dims, n_draft);
  a.is_flush = is_flush;
  a.state = const_cast<float*>(static_cast<const float*>(state));
  a.d_ring = d_ring;
  a.k_ring = k_ring;
  a.g_ring = g_ring;
  a.v_ring = v_ring;
  a.beta_ring = beta_ring;
  a.slot_idx = slot_idx;
  a.write_pos = write_pos;
  a.q = q;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.o = o;
  a.status = status;
  switch (dims->io_dtype * 2 + dims->out_dtype) {
    case 0: return verify_shape<float, float>(a, *dims, stream);
    case 1: return verify_shape<float, bf16>(a, *dims, stream);
    case 2: return verify_shape<bf16, float>(a, *dims, stream);
    case 3: return verify_shape<bf16, bf16>(a, *dims, stream);
  }
  return RSSM_EDTYPE;
}

extern "C" int replayssm_gdn_spec_verify(const rssm_gdn_dims* dims, int32_t n_draft,
                                         const void* state, float* d_ring, void* k_ring,
                                         float* g_ring, void* v_ring, float* beta_ring,
                                         const int32_t* slot_idx, const int32_t* write_pos,
                                         const void* q, const void* k, const void* v,
                                         const float* g, const float* beta, void* o,
                                         int32_t* status, hipStream_t stream) {
  return spec_verify(dims, n_draft, state, d_ring, k_ring, g_ring, v_ring, beta_ring, slot_idx,
                     write_pos, nullptr, q, k, v, g, beta, o, status, stream);
}

extern "C" int replayssm_gdn_spec_verify_flush(
    const rssm_gdn_dims* dims, int32_t n_draft, float* state, float* d_ring, void* k_ring,
    float* g_ring, void* v_ring, float* beta_ring, const int32_t* slot_idx,
    const int32_t* write_pos, const uint8_t* is_flush, const void* q, const void* k,
    const void* v, const float* g, const float* beta, void* o, int32_t* status,
    hipStream_t stream) {
  if (!is_flush && dims && dims->batch > 0) return RSSM_EINVAL;
  return spec_verify(dims, n_draft, state, d_ring, k_ring, g_ring, v_ring, beta_ring, slot_idx,
                     write_pos, is_flush, q, k, v, g, beta, o, status, stream);
}

extern "C" int replayssm_gdn_spec_advance(const rssm_gdn_dims* dims, int32_t n_draft,
                                          void* k_ring, float* g_ring, void* v_ring,
                                          float* beta_ring, const void* k, const void* v,
                                          const float* g, const float* beta,
                                          const int32_t* slot_idx, const int32_t* write_pos,
                                          const uint8_t* is_flush, const int32_t* accepted,
                                          const uint8_t* force_flush, int32_t* next_write_pos,
                                          uint8_t* next_is_flush, int32_t* status,
                                          hipStream_t stream) {
  int rc = spec_check(dims, n_draft);
  if (rc) return rc;
  if (dims->batch == 0) return RSSM_OK;
  if (!k_ring || !g_ring || !v_ring || !beta_ring || !k || !v || !g || !beta || !slot_idx ||
      !write_pos || !is_flush || !accepted || !next_write_pos || !next_is_flush)
    return RSSM_EINVAL;
  if (!aligned16(k_ring) || !aligned16(v_ring) || !aligned16(k) || !aligned16(v))
    return RSSM_EINVAL;
  if ((const void*)next_write_pos == (const void*)write_pos ||
      (const void*)next_is_flush == (const void*)is_flush)
    return RSSM_EINVAL;
  SpecArgs a = spec_args(dims, n_draft);
  a.k_ring = k_ring;
  a.g_ring = g_ring;
  a.v_ring = v_ring;
  a.beta_ring = beta_ring;
  a.k = k;
  a.v = v;
  a.g = g;
  a.beta = beta;
  a.slot_idx = slot_idx;
  a.write_pos = write_pos;
  a.is_flush = is_flush;
  a.accepted = accepted;
  a.force_flush = force_flush;
  a.next_write_pos = next_write_pos;
  a.next_is_flush = next_is_flush;
  a.status = status;
  a.n_rows = dims->batch;
  switch (dims->io_dtype) {
    case RSSM_F32: return launch_advance<float>(a, *dims, stream);
    case RSSM_BF16: return launch_advance<bf16>(a, *dims, stream);
  }
  return RSSM_EDTYPE;
}

extern "C" int replayssm_gdn_spec_commit(const rssm_gdn_dims* dims, int32_t n_draft, void* state,
                                         const void* k_ring, const float* g_ring,
                                         const void* v_ring, const float* beta_ring,
                                         const int32_t* slot_idx, const int32_t* write_pos,
                                         const int32_t* accepted, const uint8_t* force_flush,
                                         int32_t* next_write_pos, uint8_t* flushed,
                                         int32_t* status, hipStream_t stream) {
  int rc = spec_check(dims, n_draft);
  if (rc) return rc;
  if (dims->batch == 0) return RSSM_OK;
  if (!state || !k_ring || !g_ring || !v_ring || !beta_ring || !slot_idx || !write_pos ||
      !accepted || !next_write_pos)
    return RSSM_EINVAL;
  if (!aligned16(state) || !aligned16(k_ring) || !aligned16(v_ring)) return RSSM_EINVAL;
  if ((const void*)next_write_pos == (const void*)write_pos) return RSSM_EINVAL;
  SpecArgs a = spec_args(dims, n_draft);
  a.state = static_cast<float*>(state);
  a.k_ring = const_cast<void*>(k_ring);
  a.g_ring = const_cast<float*>(g_ring);
  a.v_ring = const_cast<void*>(v_ring);
  a.beta_ring = const_cast<float*>(beta_ring);
  a.slot_idx = slot_idx;
  a.write_pos = write_pos;
  a.accepted = accepted;
  a.force_flush = force_flush;
  a.next_write_pos = next_write_pos;
  a.flushed = flushed;
  a.status = status;
  // batches of up to kTaskRows rows: a small grid works through the list of
  // fold tasks; larger batches: one workgroup per (row, value head)
  a.n_rows = dims->batch;
  a.fold_tasks = dims->batch <= kTaskRows;
  switch (dims->io_dtype) {
    case RSSM_F32: return commit_shape<float>(a, *dims, stream);
    case RSSM_BF16: return commit_shape<bf16>(a, *dims, stream);
  }
  return RSSM_EDTYPE;
}
