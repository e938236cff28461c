/*
 * replayssm.h - C ABI of the MI355X (gfx950) ReplaySSM decode library.
 *
 * One decode step of a Mamba2 selective state update for a batch of rows,
 * either the standard read+write update or the ReplaySSM output-only form
 * (a checkpoint S0 plus a per-slot ring of the last inputs, folded into the
 * state only on flush rows), plus the gated-delta-rule counterparts (GDN
 * with a scalar gate, KDA with a per-key-channel gate), GDN speculative
 * verify and commit from the ring, and host-side cursor helpers.
 *
 * Sources (page title, then section):
 *  - vLLM #48018 "[Kernel] ReplaySSM: cache SSM inputs for faster Mamba2
 *    standard decode": Motivation (state traffic; ring + periodic checkpoint;
 *    write-back once every L steps), Implementation items 1-3 (per-row
 *    is_flush branch; x/dt/B ring caches; per-row write_pos and is_flush
 *    from the metadata builder), key source snippet of mamba_mixer2.py (the
 *    argument lists of the replay op and of the baseline update).
 *  - sglang #28451 (GDN/KDA ReplaySSM decode): Motivation, Implementation
 *    items 1-3 (one ring decode kernel for the GDN and KDA gates, static
 *    cursor buffers, copy rules) and review notes (the KDA gate ring).
 *  - sglang #28695 "[GDN] Support ReplaySSM Ring Spec-Verify": memory-pool
 *    snippet (the GDN ring holds d [L,V], k [L,K], g [L] per slot) and
 *    Implementation items 2-4 (spec verify from the ring, exact fold).
 *  - vLLM #52506 "[Mamba] Add FlashInfer ReplaySSM backend": Implementation
 *    item 1 (ring cursors are reset when a slot is reused).
 *
 * Conventions shared by every entry point
 *  - Every pointer is a DEVICE pointer to memory the caller owns (except
 *    for the host-side metadata helpers at the end), allocated
 *    on the device that is current when the call is made.  The library never
 *    allocates, frees or synchronises, keeps no global mutable state, and is
 *    re-entrant: it validates the arguments, enqueues kernels on `stream`
 *    (0 = the null stream) and returns.
 *  - All tensors are dense, row-major (last index fastest), with no padding.
 *    Pointers accessed with 16-byte vector loads (marked [16B]) must be
 *    16-byte aligned.
 *  - Element types follow the *_dtype fields (RSSM_F32 = float, RSSM_BF16 =
 *    bfloat16 bit pattern).  A, D, dt_bias, dt_ring, the GDN/KDA d and g
 *    rings, g and beta are always float32.  bf16 stores round to nearest
 *    even from the fp32 value (or stochastically, where rssm_dims.rounding
 *    asks for it); all arithmetic is fp32.
 *  - Return value: RSSM_OK (0) or a negative RSSM_E* code (nothing is
 *    enqueued on an error other than RSSM_ELAUNCH).  No exception crosses
 *    the ABI.
 *  - Device-side metadata errors do not fail the call: the kernel ORs
 *    RSSM_ST_* bits into *status (if status != NULL) and handles the row
 *    safely; outputs of such rows are unspecified (y is NaN for bad slots).
 *  - Contract: slot indices within one call are distinct; the next_* cursor
 *    buffers do not alias write_pos / is_flush.  Calls that share a state
 *    pool or rings must be ordered by the caller (same stream or events).
 */
#ifndef REPLAYSSM_H
#define REPLAYSSM_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
enum { RSSM_F32 = 0, RSSM_BF16 = 1 };

/* return codes */
enum {
  RSSM_OK = 0,
  RSSM_EINVAL = -1,      /* NULL required pointer, bad size, misalignment, aliasing */
  RSSM_EDTYPE = -2,      /* unsupported dtype combination */
  RSSM_ELAUNCH = -3,     /* the kernel launch reported an error */
  RSSM_ESHAPE = -4       /* headdim / dstate / ring length not supported */
};

/* device status bits (ORed into *status) */
enum {
  RSSM_ST_BAD_WRITE_POS = 1, /* write_pos outside [0, L): clamped, row flushed */
  RSSM_ST_RING_OVERFLOW = 2, /* write_pos == L-1 without is_flush: row flushed */
  RSSM_ST_BAD_SLOT = 4,      /* slot index outside [0, num_slots): row skipped */
  RSSM_ST_BAD_ROW = 8        /* ring reset or row order: row index outside [0, batch) */
};

/*
 * Rounding of the bf16 state write-back (vLLM #48018, review notes:
 * stochastic rounding was added for quantised models whose baseline relies
 * on it).  RSSM_ROUND_STOCHASTIC rounds each element of a written bf16
 * state tile up or down with probability given by the dropped 16 bits of its
 * fp32 value, using 16 random bits per element from Philox4x64-10 (Salmon
 * et al., SC 2011) with key (sr_seed, sr_offset) and counter
 * (tile * P*N/16 + e/16, 0, 0, 0), tile = slot * nheads + head, e = p*N + n:
 * element e takes bits 16*(e%4).. of output word (e%16)/4 and its bf16 bit
 * pattern is (fp32 bits + those 16 bits) >> 16 (Inf and NaN round to
 * nearest).  Applies to every state store of ssu_standard_decode and to the
 * flush write-back of replayssm_decode.  Other values: RSSM_EINVAL;
 * stochastic with an fp32 state: RSSM_EDTYPE.
 */
enum { RSSM_ROUND_NEAREST = 0, RSSM_ROUND_STOCHASTIC = 1 };

/*
 * Mamba2 dimensions.  Supported: headdim in {32, 64, 128}; dstate in {16,
 * 32, 64, 128, 256}; 1 <= ring_len <= 64 with the ring rows a workgroup
 * stages, about 4*ring_len*(P+N) bytes, within 64 KB (RSSM_ESHAPE otherwise);
 * ngroups divides nheads; state,
 * io and out dtypes each RSSM_F32 or RSSM_BF16.
 */
typedef struct rssm_dims {
  int32_t batch;       /* decode rows (0: return RSSM_OK, read nothing)     */
  int32_t nheads;      /* H                                                 */
  int32_t headdim;     /* P                                                 */
  int32_t dstate;      /* N                                                 */
  int32_t ngroups;     /* G: head h reads B/C group h / (H / G)             */
  int32_t ring_len;    /* L (ignored by ssu_standard_decode)                */
  int32_t num_slots;   /* first dimension of the state pool and the rings   */
  int32_t state_dtype; /* state pool                                        */
  int32_t io_dtype;    /* x, z, dt, B, C and the x / B rings                */
  int32_t out_dtype;   /* y                                                 */
  int32_t dt_softplus; /* nonzero: dt = softplus(dt + dt_bias)              */
  int32_t rounding;    /* state write-back: RSSM_ROUND_NEAREST or           */
                       /* RSSM_ROUND_STOCHASTIC (bf16 state only)           */
  uint64_t sr_seed;    /* stochastic rounding: Philox key word 0            */
  uint64_t sr_offset;  /* stochastic rounding: Philox key word 1; change it */
                       /* on every call so each write-back draws new bits   */
} rssm_dims;

/*
 * ssu_standard_decode - the standard selective state update (the baseline
 * the replay is measured against; vLLM #48018, Motivation and the baseline
 * call in the mamba_mixer2.py snippet).  For each row b, head h, with
 * s = slot_idx[b], g = h / (H/G):
 *     dt = softplus(dt[b,h] + dt_bias[h])      (no softplus if !dt_softplus)
 *     S  = exp(dt*A[h]) * state[s,h] + dt * outer(x[b,h,:], B[b,g,:])
 *     y[b,h,:] = S @ C[b,g,:] + D[h] * x[b,h,:];   y *= z * sigmoid(z)
 *     state[s,h] = S
 *
 *   state   [num_slots, H, P, N]  state_dtype   [16B] read and written
 *   slot_idx [batch] int32        pool slot of each row
 *   x, z    [batch, H, P]         io_dtype      [16B] z may be NULL (no gate)
 *   dt      [batch, H]            io_dtype      raw dt
 *   A       [H] float32; D [H] float32 or NULL; dt_bias [H] float32 or NULL
 *   B, C    [batch, G, N]         io_dtype      [16B]
 *   y       [batch, H, P]         out_dtype     written
 *   status  int32 or NULL         RSSM_ST_BAD_SLOT rows are skipped
 */
int ssu_standard_decode(const rssm_dims* dims, void* state,
                        const int32_t* slot_idx, const void* x, const void* dt,
                        const float* A, const void* B, const void* C,
                        const float* D, const void* z, const float* dt_bias,
                        void* y, int32_t* status, hipStream_t stream);

/*
 * replayssm_decode - one ReplaySSM output-only decode step (vLLM #48018,
 * Motivation and Implementation item 1).  Row b with s = slot_idx[b],
 * w = write_pos[b], f = is_flush[b] uses ring entries 0..w-1 of slot s and
 * the current step as entry w.  With T = sum_{j<=w} dt_j and
 * r_i = sum_{i<j<=w} dt_j (dt_j after softplus):
 *     cumdecay = exp(A[h]*T),  wt_i = dt_i * exp(A[h]*r_i)
 *     y = cumdecay*(S0 @ C) + sum_{i<=w} wt_i*(B_i . C)*x_i + D*x_w; gate
 *   f == 0: (x_w, dt_w, B_w) is written at ring position w; the state is not
 *           touched; next position w+1.
 *   f != 0: S_new = cumdecay*S0 + sum_{i<=w} wt_i*outer(x_i, B_i) is written
 *           to state[s,h]; y = S_new @ C + D*x_w (gated); next position 0.
 *   next_write_pos[b] = next position; next_is_flush[b] = (next == L-1).
 * A flush may be requested early (w < L-1).  write_pos == L-1 without
 * is_flush sets RSSM_ST_RING_OVERFLOW and the row is flushed.
 *
 *   state    [num_slots, H, P, N]  state_dtype  [16B] checkpoints S0
 *   x_ring   [num_slots, H, L, P]  io_dtype     [16B] stored x (bit copies)
 *   dt_ring  [num_slots, H, L]     float32      stored dt after softplus
 *   B_ring   [num_slots, G, L, N]  io_dtype     [16B] stored B (bit copies)
 *   slot_idx [batch] int32; write_pos [batch] int32; is_flush [batch] uint8
 *   next_write_pos [batch] int32 or NULL; next_is_flush [batch] uint8 or NULL
 *   x, dt, A, B, C, D, z, dt_bias, y: as for ssu_standard_decode
 *   status   int32 or NULL
 * Ring entries at positions >= write_pos are never read.  The order in
 * which rows are processed does not change any result; the kernel takes the
 * flush rows first, dealt evenly over the GPU's eight dies (XCDs) when the
 * batch has at most 512 rows and is_flush is 8-byte aligned, otherwise by
 * aligned groups of 64 rows.
 */
int replayssm_decode(const rssm_dims* dims, void* state, void* x_ring,
                     float* dt_ring, void* B_ring, const int32_t* slot_idx,
                     const int32_t* write_pos, const uint8_t* is_flush,
                     int32_t* next_write_pos, uint8_t* next_is_flush,
                     const void* x, const void* dt, const float* A,
                     const void* B, const void* C, const float* D,
                     const void* z, const float* dt_bias, void* y,
                     int32_t* status, hipStream_t stream);

/*
 * replayssm_decode_ordered - replayssm_decode with the batch rows handed in
 * flush-first order by the host (not on the pages: a scheduling hint for
 * this GPU).  row_order [batch] int32 (device pointer) must be a
 * permutation of 0..batch-1; replayssm_flush_first_order builds it from the
 * flush flags the host metadata path already has.  The results are those
 * of replayssm_decode for any permutation; the order only decides which
 * rows each of the GPU's eight dies (XCDs) takes: the positions of the list
 * are dealt to them in turn, so each takes an equal share of the flush rows,
 * first (replayssm_decode does the same dealing itself for batches of up
 * to 512 rows; a host list can also order the rows by slot).  An entry
 * outside [0, batch) sets
 * RSSM_ST_BAD_ROW and its position processes nothing: the row missing from
 * the list gets no y, no next cursors and no fold (its ring append, which
 * does not depend on the order, still happens); every other row is
 * processed as by replayssm_decode.  A list that repeats a row is a
 * contract violation: that row's y, cursors and (on a flush) checkpoint are
 * undefined, and another row is left unprocessed.  row_order == NULL:
 * RSSM_EINVAL.
 */
int replayssm_decode_ordered(const rssm_dims* dims, void* state, void* x_ring,
                             float* dt_ring, void* B_ring, const int32_t* slot_idx,
                             const int32_t* write_pos, const uint8_t* is_flush,
                             int32_t* next_write_pos, uint8_t* next_is_flush,
                             const void* x, const void* dt, const float* A, const void* B,
                             const void* C, const float* D, const void* z,
                             const float* dt_bias, void* y, const int32_t* row_order,
                             int32_t* status, hipStream_t stream);

/*
 * replayssm_ring_reset - rows whose slot just received a fresh checkpoint
 * restart with an empty ring (vLLM #52506, Implementation item 1; sglang
 * #28451, Implementation item 3): for r in rows[0..n_rows):
 *     write_pos[r] = 0;  is_flush[r] = (ring_len == 1)
 * Uses dims->batch (row bound) and dims->ring_len only.  The caller writes
 * the fresh state itself.  rows is a device array; rows outside [0, batch)
 * are skipped and set RSSM_ST_BAD_ROW in *status (if not NULL).
 */
int replayssm_ring_reset(const rssm_dims* dims, int32_t* write_pos,
                         uint8_t* is_flush, const int32_t* rows,
                         int32_t n_rows, int32_t* status, hipStream_t stream);

/*
 * GDN dimensions.  Supported: dk == dv == 128 (also 64); v_heads a multiple
 * of k_heads (value head hv reads key head hv / (v_heads / k_heads));
 * 1 <= ring_len <= 64 with the staged ring rows within 64 KB of LDS (about
 * ring_len*(2K + 4V) bytes for bf16 q/k/v, plus 4*ring_len*K for the KDA gate
 * rows; RSSM_ESHAPE otherwise); state_dtype RSSM_F32; io_dtype (q, k, v, k ring) and
 * out_dtype RSSM_F32 or RSSM_BF16.  scale <= 0 selects 1/sqrt(dk).
 */
typedef struct rssm_gdn_dims {
  int32_t batch;
  int32_t k_heads;
  int32_t v_heads;
  int32_t dk;          /* K */
  int32_t dv;          /* V */
  int32_t ring_len;
  int32_t num_slots;
  int32_t state_dtype;
  int32_t io_dtype;
  int32_t out_dtype;
  float scale;
} rssm_gdn_dims;

/*
 * gdn_standard_decode - the recurrent gated delta rule (sglang #28451,
 * Motivation: each step reads and writes the full [HV, V, K] state):
 *     S = g*S;  S += beta * outer(v - S@k, k);  o = scale * S@q
 *   state [num_slots, HV, V, K] float32 [16B]; slot_idx [batch] int32
 *   q, k [batch, HK, K] io_dtype [16B]; v [batch, HV, V] io_dtype [16B]
 *   g, beta [batch, HV] float32 (already activated); o [batch, HV, V] out_dtype
 */
int gdn_standard_decode(const rssm_gdn_dims* dims, void* state,
                        const int32_t* slot_idx, const void* q, const void* k,
                        const void* v, const float* g, const float* beta,
                        void* o, int32_t* status, hipStream_t stream);

/*
 * replayssm_gdn_decode - GDN ReplaySSM decode (sglang #28451, Implementation
 * item 1; ring contents per sglang #28695, memory-pool snippet).  With
 * Gamma = prod_{j<=w} g_j and gamma_i = prod_{i<j<=w} g_j:
 *     pred = Gamma*(S0@k_w) + sum_{i<w} gamma_i*d_i*(k_i . k_w)
 *     d_w  = beta_w*(v_w - pred)
 *     o    = scale*[Gamma*(S0@q) + sum_{i<=w} gamma_i*d_i*(k_i . q)]
 *   f == 0: (d_w, k_w, g_w) written at ring position w;
 *   f != 0: state = Gamma*S0 + sum_{i<=w} gamma_i*outer(d_i, k_i).
 *   d_ring [num_slots, HV, L, V] float32 [16B]; k_ring [num_slots, HK, L, K]
 *   io_dtype [16B] (bit copies of k); g_ring [num_slots, HV, L] float32.
 *   Cursor and status rules as for replayssm_decode.
 */
int replayssm_gdn_decode(const rssm_gdn_dims* dims, void* state, float* d_ring,
                         void* k_ring, float* g_ring, const int32_t* slot_idx,
                         const int32_t* write_pos, const uint8_t* is_flush,
                         int32_t* next_write_pos, uint8_t* next_is_flush,
                         const void* q, const void* k, const void* v,
                         const float* g, const float* beta, void* o,
                         int32_t* status, hipStream_t stream);

/*
 * KDA: the gated delta rule with a per-key-channel gate g in R^K (sglang
 * #28451: Implementation item 1 - one decode kernel serves the GDN scalar
 * gate and the KDA per-K gate; review notes - the KDA ring holds a gate row
 * per entry, g_cache [slots, HV, L, K]).  Same dims, layouts, cursor and
 * status rules as the GDN calls, except that g is [batch, HV, K] float32
 * [16B] and g_ring [num_slots, HV, L, K] float32 [16B].
 *
 * kda_standard_decode - the recurrence, per value head:
 *     S = S diag(g);  S += beta * outer(v - S@k, k);  o = scale * S@q
 *
 * replayssm_kda_decode - ReplaySSM decode.  With Gamma = prod_{j<=w} g_j and
 * gamma_i = prod_{i<j<=w} g_j taken per channel and kt_i = gamma_i * k_i:
 *     pred = S0@(Gamma*k_w) + sum_{i<w} d_i*(kt_i . k_w)
 *     d_w  = beta_w*(v_w - pred)
 *     o    = scale*[S0@(Gamma*q) + sum_{i<=w} d_i*(kt_i . q)]
 *   f == 0: (d_w, k_w, g_w) written at ring position w;
 *   f != 0: state = S0 diag(Gamma) + sum_{i<=w} outer(d_i, kt_i).
 */
int kda_standard_decode(const rssm_gdn_dims* dims, void* state,
                        const int32_t* slot_idx, const void* q, const void* k,
                        const void* v, const float* g, const float* beta,
                        void* o, int32_t* status, hipStream_t stream);

int replayssm_kda_decode(const rssm_gdn_dims* dims, void* state, float* d_ring,
                         void* k_ring, float* g_ring, const int32_t* slot_idx,
                         const int32_t* write_pos, const uint8_t* is_flush,
                         int32_t* next_write_pos, uint8_t* next_is_flush,
                         const void* q, const void* k, const void* v,
                         const float* g, const float* beta, void* o,
                         int32_t* status, hipStream_t stream);

/*
 * GDN speculative decoding from the ring (sglang #28695 "[GDN] Support
 * ReplaySSM Ring Spec-Verify": Implementation items 2-4 - a per-slot ring of
 * d, k, g plus the raw inputs v, k, beta; the verify rebuilds every draft's
 * output from the frozen checkpoint and the ring; the commit advances the
 * cursor and, on flush, replays the raw inputs in order through the
 * recurrent update ("exact fold"); linear draft chains only; the ring holds
 * at least twice the drafts).  Per slot the rings are those of
 * replayssm_gdn_decode plus v_ring [num_slots, HV, L, V] (io_dtype [16B]) and
 * beta_ring [num_slots, HV, L] float32.  1 <= n_draft (T) <= 8 and
 * 2*T <= ring_len <= 64 (RSSM_ESHAPE otherwise).
 *
 * replayssm_gdn_spec_verify - for row b at cursor w (entries 0..w-1
 * committed; w + T <= L, else RSSM_ST_RING_OVERFLOW and o = NaN for the
 * row), draft t is ring entry p = w + t and is formed exactly like a decode
 * step of replayssm_gdn_decode at position p (Gamma and gamma over entries
 * 0..p, pred, d_p, o).  Writes o [batch, T, HV, V] (out_dtype) and ring
 * entries w..w+T-1 (d, k, g, v, beta); the state and the cursor are not
 * modified.  q, k [batch, T, HK, K] and v [batch, T, HV, V] io_dtype [16B];
 * g, beta [batch, T, HV] float32.
 */
int replayssm_gdn_spec_verify(const rssm_gdn_dims* dims, int32_t n_draft,
                              const void* state, float* d_ring, void* k_ring,
                              float* g_ring, void* v_ring, float* beta_ring,
                              const int32_t* slot_idx, const int32_t* write_pos,
                              const void* q, const void* k, const void* v,
                              const float* g, const float* beta, void* o,
                              int32_t* status, hipStream_t stream);

/*
 * replayssm_gdn_spec_commit - keep accepted[b] (0..T) verified drafts:
 * w' = write_pos[b] + accepted[b].  If w' + T > ring_len (the next verify
 * would not fit) or force_flush[b] != 0 (force_flush may be NULL), the state
 * is rebuilt by the recurrence over entries 0..w'-1 from their raw inputs,
 *     S = g_i*S;  d = beta_i*(v_i - S@k_i);  S += outer(d, k_i),
 * stored, and w' = 0 (fp32 arithmetic; the decays are carried as one running
 * product and applied to the state at the end, or earlier when that product
 * leaves [2^-60, 2^60]: the same recurrence up to rounding).  Writes next_write_pos[b] = w' (must not alias
 * write_pos) and flushed[b] (may be NULL).  accepted outside [0, T] sets
 * RSSM_ST_RING_OVERFLOW and is clamped.
 */
int replayssm_gdn_spec_commit(const rssm_gdn_dims* dims, int32_t n_draft, void* state,
                              const void* k_ring, const float* g_ring,
                              const void* v_ring, const float* beta_ring,
                              const int32_t* slot_idx, const int32_t* write_pos,
                              const int32_t* accepted, const uint8_t* force_flush,
                              int32_t* next_write_pos, uint8_t* flushed,
                              int32_t* status, hipStream_t stream);

/*
 * Deferred-fold rounds (the same method with the fold moved into the next
 * verify, where it reuses that verify's read of the state tile: sglang
 * #28695 Implementation items 2-4 name a per-slot is_flush cursor next to
 * write_pos, and the exact fold runs on flush).  A round is
 * replayssm_gdn_spec_verify_flush then replayssm_gdn_spec_advance; between
 * rounds a row's logical state is its checkpoint folded with ring entries
 * 0..write_pos-1, and is_flush marks rows whose next verify folds first.
 * Cursors start at write_pos = 0, is_flush = 0.  A row keeps to one kind of
 * round (a pending fold is not visible to replayssm_gdn_spec_verify).  To
 * empty a row's ring at once (before copying its slot, say),
 * replayssm_gdn_spec_commit with accepted = 0 and force_flush set folds its
 * entries 0..write_pos-1 and returns write_pos 0; then clear its is_flush.
 * A row the verify refused (status bit) is left unspecified by the advance,
 * which cannot tell that no fold took place.
 *
 * replayssm_gdn_spec_verify_flush - rows with is_flush[b] != 0 (is_flush
 * [batch] uint8, required) first fold ring entries 0..write_pos[b]-1 into
 * the state exactly as replayssm_gdn_spec_commit does (0 <= write_pos[b] <=
 * L, else RSSM_ST_RING_OVERFLOW), store it, then verify their drafts at ring
 * entries 0..T-1 (w = 0); other rows verify at w = write_pos[b] as in
 * replayssm_gdn_spec_verify (w + T <= L).  Writes o and the drafts' d rows
 * at ring entries w..w+T-1 only: their v, k, g and beta rows are written by
 * replayssm_gdn_spec_advance for the drafts kept.  Arguments otherwise as
 * replayssm_gdn_spec_verify, with the state written.  A folding row stages
 * the k and v rows of the whole ring next to the verify's own rows:
 * RSSM_ESHAPE when they do not fit one workgroup's 64 KB of LDS (at K = V =
 * 128 the longest rings are 46 entries for T <= 4 and 42 for T = 8 with bf16
 * inputs, 27 and 24 with fp32 ones).
 *
 * replayssm_gdn_spec_advance - after the verify, with accepted[b] (0..T)
 * drafts kept: w = is_flush[b] ? 0 : write_pos[b]; w' = w + accepted[b];
 * next_write_pos[b] = w'; next_is_flush[b] = (w' + T > L) or
 * force_flush[b] (may be NULL).  The kept drafts' rows go from this round's
 * verify inputs (k [batch, T, HK, K], v [batch, T, HV, V] io_dtype [16B];
 * g, beta [batch, T, HV] float32) to ring entries w..w'-1 of k_ring (per key
 * head), v_ring, g_ring and beta_ring.  The next_* buffers must not alias
 * write_pos / is_flush.  dims as for the verify.  accepted outside [0, T]
 * sets RSSM_ST_RING_OVERFLOW and is clamped; a slot out of range sets
 * RSSM_ST_BAD_SLOT and its row is neither marked nor written.
 */
int replayssm_gdn_spec_verify_flush(const rssm_gdn_dims* dims, int32_t n_draft,
                                    float* state, float* d_ring, void* k_ring,
                                    float* g_ring, void* v_ring, float* beta_ring,
                                    const int32_t* slot_idx, const int32_t* write_pos,
                                    const uint8_t* is_flush, const void* q,
                                    const void* k, const void* v, const float* g,
                                    const float* beta, void* o, int32_t* status,
                                    hipStream_t stream);

int replayssm_gdn_spec_advance(const rssm_gdn_dims* dims, int32_t n_draft, void* k_ring,
                               float* g_ring, void* v_ring, float* beta_ring,
                               const void* k, const void* v, const float* g,
                               const float* beta, const int32_t* slot_idx,
                               const int32_t* write_pos, const uint8_t* is_flush,
                               const int32_t* accepted, const uint8_t* force_flush,
                               int32_t* next_write_pos, uint8_t* next_is_flush,
                               int32_t* status, hipStream_t stream);

/*
 * Host-side metadata (HOST pointers; plain CPU code, nothing is enqueued).
 *
 * replayssm_build_metadata - per-row cursors of one decode step from token
 * positions (vLLM #48018, Implementation item 3: write_pos and is_flush come
 * from a per-request decode base; align-mode re-anchoring; review notes on
 * the flush boundary, one-token prefills and preemption).  For row r:
 *     pos[r]          index of the token decoded in this step (tokens before it)
 *     decode_base[r]  number of tokens folded into the row's checkpoint S0;
 *                     set it to the prefill length for a fresh request, and
 *                     to the re-prefilled length when a preempted request
 *                     resumes (re-anchoring)
 *     w = pos - decode_base, which must lie in [0, ring_len)
 *     f = (w == ring_len-1) || force_flush[r] ||
 *         (align_block > 0 && (pos+1) % align_block == 0)
 * Writes write_pos[r] = w, is_flush[r] = f, and decode_base[r] = pos+1 when
 * f (the checkpoint will hold this token once the step has run).  With
 * align_block > 0 every checkpoint lands on a multiple of align_block or on
 * a ring-full boundary, so a prefix cache can snapshot block-aligned states.
 * force_flush may be NULL.  Returns RSSM_EINVAL, writing nothing, if any row
 * is out of range (w < 0, w >= ring_len, negative positions) or on bad
 * arguments.  For rows advancing one token per step this reproduces the
 * device-side cursor advance of replayssm_decode.
 */
int replayssm_build_metadata(int32_t n_rows, int32_t ring_len, int32_t align_block,
                             const int64_t* pos, int64_t* decode_base,
                             const uint8_t* force_flush, int32_t* write_pos,
                             uint8_t* is_flush);

/*
 * replayssm_check_copy_sources - the copy rule for slots (sglang #28451 and
 * #28695: a slot's state may be copied only when its ring is empty, else
 * the ring entries not yet folded would be lost).  src_write_pos [n] are the
 * current write positions of the source rows (HOST pointer).  RSSM_OK if
 * every one is 0, RSSM_EINVAL otherwise.  After copying a state into a new
 * slot, reset that row's cursors with replayssm_ring_reset.
 */
int replayssm_check_copy_sources(int32_t n, const int32_t* src_write_pos);

/*
 * replayssm_flush_first_order - the row order for replayssm_decode_ordered:
 * the rows with is_flush[r] != 0 in increasing r, then the others in
 * increasing r.  is_flush [n_rows] and row_order [n_rows] are HOST pointers.
 * RSSM_OK, or RSSM_EINVAL for n_rows < 0 or a NULL pointer with n_rows > 0.
 */
int replayssm_flush_first_order(int32_t n_rows, const uint8_t* is_flush, int32_t* row_order);

/* Human-readable text of a return code (static storage). */
const char* replayssm_strerror(int code);

/* Library ABI version (major * 100 + minor). */
int replayssm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* REPLAYSSM_H */
