/*
 * gdnverify.h -- C ABI of libgdnverify: the GDN (Gated DeltaNet) ReplaySSM
 * ring spec-verify on AMD Instinct MI355X (gfx950).
 *
 * The method (replayssm(B)SpecDecode, a walkthrough of SGLang PR #28695;
 * PR #28695, #33102 and #36821 summaries on prhub):  every state slot keeps a
 * frozen fp32 checkpoint S[slot] and a ring of the raw records committed since
 * (raw k, raw v, gate g, beta).  A verify reconstructs the outputs of the whole
 * draft window from checkpoint + ring history + window in closed form, never
 * writing a per-draft state; it also copies the window's raw records into the
 * ring as a side channel.  Rejecting drafts is a cursor move.  Before the ring
 * can overflow, an exact sequential fold replays the committed records into
 * the checkpoint.
 *
 * Conventions for every entry point
 *  - All tensor arguments are DEVICE pointers owned by the caller, packed
 *    row-major in the layouts given below.  The library never allocates,
 *    frees or synchronises; each call only enqueues kernels on `stream`
 *    (a hipStream_t, NULL for the legacy default stream) and returns.
 *  - Return value: GDN_OK (0) once everything is enqueued; a negative
 *    gdn_status on a host-side argument error, in which case nothing was
 *    enqueued; GDN_ELAUNCH if the HIP runtime rejected a launch.
 *  - Device-side there are no errors, only defined behaviour:
 *      * a row whose slot_idx is < 0 or >= num_slots is a padding row: it reads
 *        and writes nothing, its output rows are left untouched (the pages'
 *        NULL_BLOCK_ID rows, replayssm(B)SpecDecode App. A.1; PR #36821 summary:
 *        no writes through negative slots);
 *      * accept counts are clamped to [0, T];
 *      * write_pos is clamped to [0, L-T] wherever it is read, which never
 *        binds while the early-flush invariant holds (replayssm(B)SpecDecode
 *        §8.2);
 *      * the slots of the non-padding rows of one call must be distinct.
 *  - Activations (q, k, v, a, b, o and the ring's rawk/rawv) are in the dtype
 *    `act` of the shape; S, snapshots and the ring's g/beta are fp32;
 *    indices and cursors are int32.
 *
 * Layouts (token index = row * T + t; GQA: value head hv reads qk-head
 * hv / (HV/H), replayssm(B)SpecDecode App. A.1 parameter table):
 *    q, k       [B*T, H, K]            v, o   [B*T, HV, V]
 *    a, b       [B*T, HV]              A_log, dt_bias [HV] fp32
 *    S          [num_slots, HV, V, K]  fp32 checkpoint, K contiguous
 *    ring_rawk  [num_slots, H, L, K]   ring_rawv [num_slots, HV, L, V]
 *    ring_g     [num_slots, HV, L]     ring_beta [num_slots, HV, L]   fp32
 *    write_pos, cache_base, is_flush   [num_slots] int32, shared by all layers
 *    slot_idx   [B] int32              snap [B, T, HV, V, K] fp32
 *  Record j of a slot's committed history is at physical ring position
 *  (cache_base + j) & (L-1) (replayssm(B)SpecDecode §10.1).
 */
#ifndef GDNVERIFY_H
#define GDNVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_EINVAL = -1,        /* malformed shape, null or misaligned pointer   */
    GDN_EUNSUPPORTED = -2,  /* well-formed but outside what the kernels cover */
    GDN_ELAUNCH = -3        /* the HIP runtime refused a kernel launch        */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/*
 * Geometry of one GDN layer's verify.  Host-side validation (mirrors the
 * pages' configuration checks: PR #28695 summary, server_args snippet: ring
 * length at least twice the draft count; PR #36821 summary, ring view checks):
 *   B >= 0; 1 <= T <= max_spec_len <= 16; L a power of two, 2*max_spec_len <= L
 *   <= 128; H >= 1; HV % H == 0; K in {64, 128, 256} (K = 256 only with L <= 64);
 *   V % 16 == 0, 16 <= V <= 256; 0 <= B <= 65535; num_slots >= 1;
 *   act in {GDN_F32, GDN_BF16}; l2norm_eps >= 0; finite scale and threshold.
 * Anything else returns GDN_EINVAL (malformed) or GDN_EUNSUPPORTED.
 *
 * Why the supported envelope is narrower than "K, V multiples of 16 up to
 * 256, L up to 256":
 *  - K: a state row is spread over 16 lanes holding K/16 columns each in
 *    4-wide vectors, and the closed form's key blocks are whole 64-column
 *    MFMA tiles, so K must be a multiple of 64; the kernels are instantiated
 *    for the three head widths 64, 128 and 256.
 *  - L: the verify solves history and window as one system inside a
 *    workgroup's LDS: up to L + 16 key rows, L + 16 value rows and the
 *    strictly lower panels of A.  At L = 256 that exceeds the 160 KB of LDS of
 *    a compute unit for every K, and at K = 256 already for L = 128; those
 *    shapes return GDN_EUNSUPPORTED instead of running a slower fallback.
 *  - max_spec_len <= 16: the window's query rows and Z columns are one
 *    16-row MFMA block.
 */
typedef struct gdn_shape {
    int32_t B, T, H, HV, K, V;
    int32_t L, max_spec_len, num_slots;
    int32_t act;                 /* gdn_dtype */
    float scale;                 /* output scale; 1.0 when unused            */
    float softplus_threshold;    /* softplus(x) = x above it; 20.0 typical   */
    float l2norm_eps;            /* q/k l2 norm: x / sqrt(sum x^2 + eps)     */
} gdn_shape;

/*
 * gdn_spec_verify_ring -- the verify step of one layer
 * (replayssm(B)SpecDecode §1.1, §4.1, §5.1, §9.1; PR #33102 report anchor 1;
 *  PR #36821 summary implementation item 1).
 *
 * For every non-padding row b with slot s = slot_idx[b] and value head hv:
 *   hist = is_flush[s] ? 0 : write_pos[s];
 *   S_c  = S[s,hv] stepped through the hist committed ring records;
 *   o[b*T+t, hv, :] = scale * S_t q_hat_t for t = 0..T-1, where S_t is S_c
 *   stepped through window tokens 0..t with g = -exp(A_log) softplus(a+dt_bias),
 *   beta = sigmoid(b) and l2-normalised q, k.  Every window position gets an
 *   output, later-rejected ones included.  The window states are never stored:
 *   the kernel evaluates the chunked closed form (I+A)^-1 over history+window
 *   from the frozen checkpoint.
 * fold_flagged = 1: rows whose slot has is_flush set first get their
 *   checkpoint S[s] advanced in place by the exact fold of their write_pos
 *   committed records (the two-launch verify-or-flush routing, §8.1, §9.1);
 *   fold_flagged = 0: the caller has already folded flagged rows (for example
 *   with gdn_exact_fold); they are verified with an empty history.  A flagged
 *   row must be folded exactly once per step.
 * write_ring = 1: the window's records are written, pre-mutation, at logical
 *   positions write_pos + t: ring_rawk[s, h, p, :] = k bits (once per qk-head),
 *   ring_rawv[s, hv, p, :] = v bits, ring_g/ring_beta[s, hv, p] = the fp32 gate
 *   and beta used by the kernel.  Nothing else in the ring is written and the
 *   outputs are bitwise identical with write_ring = 0.
 * S is never written for unflagged rows; cursors are never written.
 * o must not alias any input.  The ring pointers are always required (the
 * history is read from them even when write_ring = 0).
 * bf16 gate inputs: a and b are read as aligned 4-byte words holding two
 * activations, so for act = GDN_BF16 they must be 4-byte aligned
 * (GDN_EINVAL otherwise) and B*T*HV must be even (GDN_EUNSUPPORTED
 * otherwise), so that no word reaches past the last element.
 * fp32 activations: the key-side products run on bf16 matrix units, so fp32
 * keys and queries enter them as a bf16 high part plus a bf16 remainder
 * (about 16 significant bits; the remainder-by-remainder product is
 * dropped).  Everything else (norms, gates, the solve, the checkpoint
 * products, the state and the outputs) is fp32.  The outputs stay within
 * 1e-5 of the fp64 recurrence on the fp32 workloads, far inside 2e-3.
 */
int gdn_spec_verify_ring(const gdn_shape *shape,
                         const void *q, const void *k, const void *v,
                         const void *a, const void *b,
                         const float *A_log, const float *dt_bias,
                         float *S, const int32_t *slot_idx,
                         const int32_t *write_pos, const int32_t *cache_base,
                         const int32_t *is_flush,
                         void *ring_rawk, void *ring_rawv,
                         float *ring_g, float *ring_beta,
                         int write_ring, int fold_flagged,
                         void *o, void *stream);

/*
 * gdn_spec_verify_dcache -- the verify step through a ring of corrected
 * deltas (the first-generation ring of replayssm(B)SpecDecode §1.1 table,
 * which caches d, k and g per committed token; §12.6 defines the corrected
 * delta d = beta (v - e^g S k_hat), the rank-1 factor of a step).
 *
 * Same arguments, outputs and side effects as gdn_spec_verify_ring, plus
 *    ring_d  [num_slots, HV, L, V] fp32, caller-owned (gdn_dring_bytes).
 * The committed history enters only through ring_d: record j's stored delta
 * at physical position (cache_base + j) & (L-1), together with its raw key
 * and gate from the raw ring (its raw value is not read).  The window's
 * deltas follow from a T x T unit lower-triangular system, and the outputs
 * equal gdn_spec_verify_ring's up to rounding.
 * write_ring = 1: besides the raw records, ring_d[s, hv, p, :] receives the
 *   window token's corrected delta at p = (cache_base + write_pos + t) & (L-1).
 *   Nothing else in ring_d is written.
 * Precondition: for every unflagged row, ring_d holds at logical positions
 *   0..write_pos-1 the deltas recorded by d-cache verifies (with
 *   write_ring = 1) since the slot's last fold or reset.  A delta depends on
 *   the checkpoint it was formed against, so a slot folded for any other
 *   reason must be reset before its next d-cache verify.  Flagged rows are
 *   folded (fold_flagged = 1) from the raw records and verified with an empty
 *   history, so they need no stored deltas.
 * Returns GDN_EUNSUPPORTED where the kernel's LDS would exceed 160 KB
 * (never for the shapes gdn_validate_shape accepts).  ring_d must not alias o.
 */
int gdn_spec_verify_dcache(const gdn_shape *shape,
                           const void *q, const void *k, const void *v,
                           const void *a, const void *b,
                           const float *A_log, const float *dt_bias,
                           float *S, const int32_t *slot_idx,
                           const int32_t *write_pos, const int32_t *cache_base,
                           const int32_t *is_flush,
                           void *ring_rawk, void *ring_rawv,
                           float *ring_g, float *ring_beta, float *ring_d,
                           int write_ring, int fold_flagged,
                           void *o, void *stream);

/* Bytes of the d ring of gdn_spec_verify_dcache: num_slots*HV*L*V*4
 * (0 for an invalid shape). */
size_t gdn_dring_bytes(const gdn_shape *shape);

/*
 * gdn_exact_fold -- closed-loop exact fold of committed ring records into the
 * checkpoint (PR #28695 summary, implementation item 3: sequential replay from
 * the raw inputs, consistent with the recurrent update; replayssm(B)SpecDecode
 * §12.7).  For each non-padding row (only those whose slot has is_flush set
 * when only_flagged = 1) and every value head:
 *   for j in 0..write_pos-1:  S[s,hv] <- step(S[s,hv], record at
 *   (cache_base + j) & (L-1)), in place.
 * The step reads rawk/rawv/g/beta exactly as recorded, normalises the key
 * with l2norm_eps and uses the same arithmetic as gdn_recurrent_verify_snapshot,
 * so folding a ring written by a verify reproduces the snapshot path's state
 * bit for bit.  (Both carry a head's decay in one scalar instead of
 * multiplying every state element by e^g at every record: the same step in
 * exact arithmetic, rounded differently from the plain form.)  Cursors are not modified: a row folded while unflagged must
 * have its cursors rebased (e.g. gdn_reset_cursors) before its next verify.
 * num_layers >= 1 folds that many layers in one launch (out-of-forward work,
 * so the layer axis is parallel: PR #33102 report, the all-layer commit
 * fold).  Layer l's checkpoint starts at S + l * layer_stride_S (fp32
 * elements) and its ring at l * layer_stride_ring SLOTS past each ring base:
 * ring_rawk + l*layer_stride_ring*H*L*K, ring_rawv + l*layer_stride_ring*HV*L*V,
 * ring_g / ring_beta + l*layer_stride_ring*HV*L elements.  One slot count
 * describes all four ring arrays of a pool whose layers are laid out
 * [layer][slot][...].  A stride of 0 means back to back (num_slots*HV*V*K,
 * num_slots).  With num_layers > 1 a nonzero stride must not make layers
 * overlap (layer_stride_S >= num_slots*HV*V*K, layer_stride_ring >=
 * num_slots), layer_stride_S must be a multiple of 4 (16-byte aligned
 * layers), and negative strides are rejected (GDN_EINVAL).  Cursors are
 * shared by all layers.  shape->T is the draft window of the verifies that
 * wrote the ring (for the write_pos clamp); q/k/v/a/b are not read.
 */
int gdn_exact_fold(const gdn_shape *shape, int num_layers,
                   int64_t layer_stride_S, int64_t layer_stride_ring,
                   float *S, const void *ring_rawk, const void *ring_rawv,
                   const float *ring_g, const float *ring_beta,
                   const int32_t *slot_idx, const int32_t *write_pos,
                   const int32_t *cache_base, const int32_t *is_flush,
                   int only_flagged, void *stream);

/*
 * gdn_kda_spec_verify_ring -- the verify step of one KDA layer, whose gate is
 * a vector over the key channels (PR #36821 summary: the KDA spec ring keeps
 * g per record as K fp32 values, ring layout [slots, HV, L, K], beside raw k,
 * raw v and a scalar beta; the same ring discipline and lifecycle as the GDN
 * ring).  Same arguments and side effects as gdn_spec_verify_ring, except:
 *    a         [B*T, HV, K]             (act dtype)   b [B*T, HV] as before
 *    dt_bias   [HV, K] fp32             A_log [HV] fp32
 *    ring_g    [num_slots, HV, L, K] fp32
 * For every non-padding row b with slot s and value head hv:
 *   g_c = -exp(A_log[hv]) softplus(a[., hv, c] + dt_bias[hv, c]),
 *   beta = sigmoid(b);
 *   step: column c of the state decays by e^{g_c}, then the delta rule
 *   u = S k_hat, S += beta (v - u) k_hat^T;  o_t = scale S_t q_hat_t.
 *   hist = is_flush[s] ? 0 : write_pos[s]; the outputs come from S[s,hv]
 *   stepped through hist committed records, then window tokens 0..t.
 * The verify is one launch that replays the history from the frozen
 * checkpoint (the per-channel decay has no scalar closed form to regroup):
 * fold_flagged = 1 makes a flagged row store the state reached after its
 * write_pos records into S[s] (the exact fold, same records and arithmetic
 * as gdn_kda_exact_fold) and verify its window from there; fold_flagged = 0
 * verifies a flagged row from S[s] with an empty history.
 * write_ring = 1: ring_rawk/ring_rawv receive the k/v bits and
 *   ring_g[s, hv, p, :] / ring_beta[s, hv, p] the fp32 channel gates and
 *   beta the kernel used, at p = (cache_base + write_pos + t) & (L-1);
 *   outputs are bitwise identical with write_ring = 0.
 * Supported: the gdn_shape envelope with V a multiple of 64 (a workgroup
 * holds 64 state rows); other shapes return GDN_EUNSUPPORTED.  a and b are
 * read element by element (no word-pair rule).  ring_g must be 16-byte
 * aligned.  o must not alias any input.
 */
int gdn_kda_spec_verify_ring(const gdn_shape *shape,
                             const void *q, const void *k, const void *v,
                             const void *a, const void *b,
                             const float *A_log, const float *dt_bias,
                             float *S, const int32_t *slot_idx,
                             const int32_t *write_pos, const int32_t *cache_base,
                             const int32_t *is_flush,
                             void *ring_rawk, void *ring_rawv,
                             float *ring_g, float *ring_beta,
                             int write_ring, int fold_flagged,
                             void *o, void *stream);

/*
 * gdn_kda_exact_fold -- the exact fold of a KDA layer's committed records
 * into its checkpoint: gdn_exact_fold's contract (rows, only_flagged, layer
 * strides, cursors untouched) with the KDA step and ring_g [num_slots, HV,
 * L, K]; layer l's ring_g starts l * layer_stride_ring * HV * L * K elements
 * past ring_g.  Bitwise the state a fold_flagged verify stores.
 * Same support envelope as gdn_kda_spec_verify_ring.
 */
int gdn_kda_exact_fold(const gdn_shape *shape, int num_layers,
                       int64_t layer_stride_S, int64_t layer_stride_ring,
                       float *S, const void *ring_rawk, const void *ring_rawv,
                       const float *ring_g, const float *ring_beta,
                       const int32_t *slot_idx, const int32_t *write_pos,
                       const int32_t *cache_base, const int32_t *is_flush,
                       int only_flagged, void *stream);

/* Bytes of one KDA layer's ring: num_slots * L records of raw k, raw v,
 * K channel gates and beta (0 for an invalid or unsupported shape). */
size_t gdn_kda_ring_bytes(const gdn_shape *shape);

/*
 * gdn_advance_cursors -- commit by accept count (replayssm(B)SpecDecode §4.2,
 * §8.1-8.2, §9.3).  For each non-padding row with slot s and a = clamp(accept):
 *   if is_flush[s]: cache_base[s] = (cache_base[s] + write_pos[s]) & (L-1);
 *                   write_pos[s] = a
 *   else:           write_pos[s] += a
 *   is_flush[s] = (write_pos[s] + 2 * max_spec_len > L)      (strict)
 * One thread per row; called once per step after sampling.
 */
int gdn_advance_cursors(const gdn_shape *shape, const int32_t *slot_idx,
                        const int32_t *accept, int32_t *write_pos,
                        int32_t *cache_base, int32_t *is_flush, void *stream);

/*
 * gdn_reset_cursors -- prefill-to-decode handoff (replayssm(B)SpecDecode
 * App. A.2): write_pos = 0, cache_base = 0, is_flush = init_flush for the n
 * listed slots (entries outside [0, num_slots) are skipped).  n >= 0.
 */
int gdn_reset_cursors(const gdn_shape *shape, const int32_t *slots, int32_t n,
                      int32_t init_flush, int32_t *write_pos, int32_t *cache_base,
                      int32_t *is_flush, void *stream);

/*
 * gdn_recurrent_verify_snapshot -- the baseline the ring replaces
 * (PR #28695 summary, gdn_backend snippet: the recurrent target_verify with an
 * intermediate state buffer; PR #36821 summary: a full [K,V] fp32 snapshot per
 * head-step).  From S[slot] (read only, no ring history), step through the
 * window writing snap[b, t, hv] = S_t and o as in gdn_spec_verify_ring.
 * write_ring = 1 additionally records the window in the ring exactly as the
 * ring verify does (same positions, same g/beta bits); the ring and cursor
 * pointers may be NULL when write_ring = 0.  snap must not alias S.
 * There is no is_flush argument: the window's records land at
 * (cache_base + write_pos + t) & (L-1) whether or not the slot is flagged
 * (for a flagged slot that is the next history's start), and this path
 * reads no history, so the flag would change nothing it computes.
 */
int gdn_recurrent_verify_snapshot(const gdn_shape *shape,
                                  const void *q, const void *k, const void *v,
                                  const void *a, const void *b,
                                  const float *A_log, const float *dt_bias,
                                  const float *S, const int32_t *slot_idx,
                                  float *snap, void *o,
                                  void *ring_rawk, void *ring_rawv,
                                  float *ring_g, float *ring_beta,
                                  const int32_t *write_pos, const int32_t *cache_base,
                                  int write_ring, void *stream);

/*
 * gdn_snapshot_commit -- the baseline's commit: S[slot_idx[b]] =
 * snap[b, a-1] for rows with a = clamp(accept[b]) >= 1; rows accepting nothing
 * keep their state (PR #28695 summary: the recurrent path copies the accepted
 * intermediate state at commit).
 */
int gdn_snapshot_commit(const gdn_shape *shape, const float *snap,
                        const int32_t *slot_idx, const int32_t *accept, float *S,
                        void *stream);

/* Footprints in bytes (host only, no device work): the per-layer ring
 * (num_slots * L records) and the per-layer snapshot buffer (B*T*HV*V*K fp32).
 * 0 for an invalid shape. */
size_t gdn_ring_bytes(const gdn_shape *shape);
size_t gdn_snapshot_bytes(const gdn_shape *shape);

/* Host-side check of a shape alone; returns a gdn_status. */
int gdn_validate_shape(const gdn_shape *shape);

/* Static description of a status code. */
const char *gdn_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* GDNVERIFY_H */
