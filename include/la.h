/*
 * la.h -- C ABI of the MI355X (gfx950) linear-attention recurrence library (libla.so).
 *
 * The library computes, for every (batch b, head h) slice independently,
 *
 *     S_t = S_{t-1} A_t + beta_t v_t k_t^T ,        o_t = S_t q_t
 *
 * ("History Replays Itself: Unleashing Long-Context Capability in Linear Attention",
 * Sec. 2 Preliminary, Eq. (1); one layer, one head; output gates and normalisation are
 * outside the recurrence there and outside this library).  S_t is d_v x d_k, A_t acts
 * on the right, and o_t reads the state after token t's write.  Variants:
 *
 *   LA_ADDITIVE      A_t = I, beta_t = 1                 (same passage, additive case)
 *   LA_GATED         A_t = alpha_t I                      (scalar-gated state)
 *   LA_GATED_DELTA   A_t = alpha_t (I - beta_t k_t k_t^T) (gated delta rule)
 *   LA_BASED         second-order Taylor linear attention with normaliser
 *                    ("Simple linear attention language models balance the
 *                    recall-throughput tradeoff", reading notes Sec. 2.2 and 2.3, paper
 *                    Eqs. (1)-(4)):  phi(x) = [1, x, vec(x x^T)/sqrt(2)],
 *                    s_t = s_{t-1} + phi(k_t) v_t^T, z_t = z_{t-1} + phi(k_t),
 *                    o_t = s_t^T phi(q_t) / (z_t^T phi(q_t) + eps).
 *                    No input scaling is applied: callers that want the x/d'^(1/4)
 *                    scaling of the paper's listing pre-scale q and k.
 *   LA_BASED_COMPACT the same recurrence and outputs with the compact feature map of the
 *                    same notes' feature-width table (Sec. 2.3), which keeps every cross
 *                    term once: phi_c(x) = [1, x, x_a^2/sqrt(2) (a = b), x_a x_b (a < b)],
 *                    so phi_c(q).phi_c(k) = phi(q).phi(k) with 1 + d' + d'(d'+1)/2 features
 *                    (153 for d' = 16: 44% less state than 273).
 *
 * Layouts (row-major, last index fastest; every pointer is DEVICE memory):
 *   q, k      [B][H][T][d_k]        (BASED: d_k = d', the projected q/k width)
 *   v, o      [B][H][T][d_v]
 *   alpha,beta[B][H][T]             decay alpha_t in (0,1], write strength beta_t
 *   S         [B][H][d_v][d_k] fp32 (ADDITIVE, GATED, GATED_DELTA)
 *   s         [B][H][D][d_v]   fp32, z [B][H][D] fp32 (BASED, D = 1 + d' + d'^2,
 *             feature order [1, x_0..x_{d'-1}, x_i x_j / sqrt 2 at 1 + d' + i d' + j];
 *             BASED_COMPACT, D = 1 + d' + d'(d'+1)/2, order [1, x_0..x_{d'-1}, then the
 *             pairs a <= b in row-major upper-triangle order: pair (a, b) at
 *             1 + d' + a d' - a(a-1)/2 + (b - a)])
 *   Decode drops the T axis and replaces [B][H] by N independent states.
 * q, k, v, alpha, beta and o share one element type (LA_F32 or LA_BF16); states are
 * always fp32; all accumulation is fp32.  o is rounded to nearest-even on store.
 *
 * Inputs per variant (anything else returns LA_ERR_INVALID):
 *   ADDITIVE      alpha and beta must be NULL.
 *   GATED         alpha required; beta == NULL means beta_t = 1.
 *   GATED_DELTA   alpha and beta required.
 *   BASED, BASED_COMPACT
 *                 alpha and beta must be NULL; z pointers are required wherever the
 *                 corresponding s pointer is given.
 * Preconditions that are not checked: alpha_t in (0, 1] (outside it results are
 * unspecified), finite inputs (NaN/Inf propagate through the recurrence, except across a
 * point where the decay has taken the state's dependence on earlier tokens to exactly zero
 * in fp32: the chunked prefill stops carrying those tokens there, as it may).
 *
 * Ownership and threading: the caller owns every buffer, including the workspace.
 * The library allocates no device memory (its one static device array, the scratch of
 * la_prefill_noalloc, comes with the code object), keeps no per-call global state, and
 * only enqueues work on `stream` (a hipStream_t; NULL = the null stream).  Calls are
 * asynchronous: buffers must stay alive until the stream has passed them.  Calls on
 * distinct streams are independent.  Results are bitwise deterministic run to run.
 *
 * Alignment: states (S, s, z), the workspace, and -- for la_prefill -- q, k, v and o must
 * be 16-byte aligned; every other pointer must be aligned to its element size.
 *
 * Errors: arguments are validated before anything is launched; a negative la_status
 * is returned and no memory is touched.  LA_ERR_HIP means a launch failed.  Faults
 * inside kernels surface, as HIP reports them, at the caller's next synchronisation.
 * Nothing crosses the ABI as an exception and nothing is printed.
 */
#ifndef LA_H
#define LA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { LA_ADDITIVE = 0, LA_BASED = 1, LA_GATED = 2, LA_GATED_DELTA = 3, LA_BASED_COMPACT = 4 };
enum { LA_F32 = 0, LA_BF16 = 1 };

enum {
  LA_OK = 0,
  LA_ERR_NULL = -1,        /* a required pointer is NULL                               */
  LA_ERR_INVALID = -2,     /* bad variant/dtype, non-positive sizes, forbidden pointer */
  LA_ERR_UNSUPPORTED = -3, /* valid but not implemented (d_k / d_v / dtype combination)*/
  LA_ERR_ALIGN = -4,       /* a pointer is misaligned (see the alignment rules above)  */
  LA_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than la_prefill_workspace_size */
  LA_ERR_ALIAS = -6,       /* two buffers overlap where that is not allowed            */
  LA_ERR_HIP = -7          /* a HIP launch failed                                      */
};

/* Version of this ABI (bumped on any incompatible change). */
int la_abi_version(void);

/* Human-readable name of a status code (static string, never NULL). */
const char *la_status_string(int status);

/*
 * Workspace that la_prefill needs for this problem, in bytes (0 is possible).  The
 * workspace holds the chunked prefill's per-segment fp32 state maps and start states and,
 * for the gated delta rule at d_k = 256, one bf16 lower-triangular 64 x 64 transform per
 * chunk of 64 tokens (6 KiB per chunk and head: the zero blocks right of the diagonal in
 * its first 32 rows are not stored; see la_prefill_pass); for short fp32 ADDITIVE and GATED
 * problems, the start state and one fp32 d_v x d_k state sum per chunk.
 * Returns LA_OK and writes *bytes, or the same validation error la_prefill would give.
 */
int la_prefill_workspace_size(int variant, int dtype, int batch, int heads, int64_t seq_len,
                              int d_k, int d_v, size_t *bytes);

/*
 * la_prefill -- run the recurrence over T = seq_len tokens for B x H slices.
 *
 *   S0 / z0  start state (NULL = zero state, the empty-prefix state s_0 = 0, z_0 = 0 of
 *            the BASED notes, Sec. 2.2).  For BASED, S0/S_T are s and z0/z_T are z.
 *   o        outputs o_t for every token.
 *   S_T/z_T  end state (may be NULL when not wanted; BASED: both or neither).
 *   eps      BASED denominator epsilon (ignored otherwise).  The BASED notes (Sec. 2.3)
 *            say only that an implementation adds a small epsilon; 1e-6 is a sensible
 *            choice.  o = num / (den + eps).
 *   workspace, workspace_bytes
 *            device scratch of at least la_prefill_workspace_size() bytes (may be NULL
 *            when that size is 0).  Its contents on entry do not matter.
 *
 * Aliasing: o, S_T, z_T and the workspace must not overlap each other or any input.
 * S_T may equal S0 exactly (in-place state update), and z_T may equal z0.
 *
 * Method: bf16 inputs take the chunkwise path -- chunks of 64 tokens, intra-chunk
 * products on MFMA with fp32 accumulation, the gated delta rule's WY/UT transform
 * solved per chunk (at d_k = 128 inside the passes that use it, at 256 in a pass of its
 * own), and an fp32 state carried across chunks and
 * across segments of chunks (a three-pass segment scan: per-segment affine state maps,
 * a scan of the segment start states, then every segment replayed from its start
 * state).  fp32
 * inputs take an fp32 path (fp32 products and accumulation throughout): ADDITIVE and GATED
 * problems of 2 to 32 chunks (at most 2048 tokens, B H nch^2 <= 4096, d_k in {64, 128},
 * d_v a multiple of 16 up to 128) in a chunk form on fp32 MFMA whose per-chunk state sums
 * live in the workspace; other small ADDITIVE and GATED problems (T <= 2048,
 * B H ceil(T/64)^2 <= 4096, d_v <= 128) in the masked attention form that Eq. (1) unrolls
 * to (parallel over tokens, gate prefix sums in fp64); everything else token by token.
 *
 * Supported: bf16 -- ADDITIVE/GATED/GATED_DELTA with d_k = d_v in {64, 128, 256}
 *                    (128 and 256 chunkwise; 64 token-recurrent in fp32);
 *                    BASED and BASED_COMPACT with d' = 16, d_v = 64.
 *            fp32 -- ADDITIVE/GATED/GATED_DELTA with d_k in {64, 128, 256} and any d_v;
 *                    BASED and BASED_COMPACT with d' = 16 and d_v = 64.
 *            Any T >= 1 up to B H T <= 2^37 token-heads (a partial last chunk is
 *            masked; larger problems return LA_ERR_UNSUPPORTED).  T = 0 is the empty prefix:
 *            nothing is read from q, k, v, alpha, beta (they may be NULL), o is empty,
 *            and S_T/z_T receive the start state (zeros when S0 is NULL).
 */
int la_prefill(int variant, int dtype, int batch, int heads, int64_t seq_len, int d_k, int d_v,
               float eps, const void *q, const void *k, const void *v, const void *alpha,
               const void *beta, const float *S0, const float *z0, void *o, float *S_T,
               float *z_T, void *workspace, size_t workspace_bytes, void *stream);

/*
 * la_prefill_pass -- run one of the passes of la_prefill, for callers that schedule
 * them separately (to time them, to overlap them with other work, or to shard one
 * sequence across devices, where the scan becomes an exchange of per-slice maps).  With
 * the same arguments and workspace on one stream,
 *
 *   la_prefill(...)  ==  la_prefill_pass(LA_PASS_TRANSFORM, ...);
 *                        la_prefill_pass(LA_PASS_MAPS, ...);
 *                        la_prefill_pass(LA_PASS_SCAN, ...);
 *                        la_prefill_pass(LA_PASS_REPLAY, ...);
 *
 *   LA_PASS_TRANSFORM  gated delta rule on the chunked path at d_k = 256: every chunk's UT
 *                      transform (I + L)^{-1} diag(beta), which depends on keys and gates
 *                      only, written to the workspace for the passes that follow (at
 *                      d_k = 128 nothing: the map and replay passes form each chunk's
 *                      solve from the keys they load)
 *   LA_PASS_MAPS       per segment of chunks except the last, the affine map of its end
 *                      state on its start state (S_end = S_start M + B; M is d_k x d_k
 *                      for the gated delta rule, a scalar decay otherwise), written to
 *                      the workspace (when the decay over a segment's last 8 chunks takes
 *                      M to exactly zero in fp32, the map is formed from those chunks
 *                      alone: M = 0, B theirs)
 *   LA_PASS_SCAN       segment start states S_{i+1} = S_i M_i + B_i from S0
 *   LA_PASS_REPLAY     every segment from its start state: o, and S_T from the last one
 *
 * Passes that do not apply to a problem (one segment, no delta rule, fp32 inputs, other
 * widths) do nothing; LA_PASS_REPLAY then performs the rest of the computation.
 * Arguments, validation and return values are those of la_prefill.
 */
enum { LA_PASS_MAPS = 1, LA_PASS_SCAN = 2, LA_PASS_REPLAY = 3, LA_PASS_TRANSFORM = 4 };
int la_prefill_pass(int pass, int variant, int dtype, int batch, int heads, int64_t seq_len,
                    int d_k, int d_v, float eps, const void *q, const void *k, const void *v,
                    const void *alpha, const void *beta, const float *S0, const float *z0,
                    void *o, float *S_T, float *z_T, void *workspace, size_t workspace_bytes,
                    void *stream);

/*
 * How la_prefill splits each (b, h) sequence: *n_segments segments of
 * *chunks_per_segment chunks of 64 tokens (1 and 0 when the chunked path is not used).
 */
int la_prefill_segments(int variant, int dtype, int batch, int heads, int64_t seq_len, int d_k,
                        int d_v, int *n_segments, int *chunks_per_segment);

/*
 * la_prefill_noalloc -- la_prefill for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments without the workspace, which comes from a static device array of
 * LA_NOALLOC_SCRATCH_BYTES bytes that the library holds, one per device, until the
 * process ends.  The segment plan is chosen so that the workspace fits in it (fewer
 * segments than la_prefill may use, so results can differ from la_prefill's within the
 * rounding of the chunked path); a problem whose workspace exceeds it even with a single
 * segment returns LA_ERR_WORKSPACE before anything is launched (only the gated delta rule
 * with bf16 inputs at d_k = 256 beyond about B H T = 1.4 million token-heads: at d_k = 128
 * the workspace holds segment maps and start states only, at most about 96 MiB).  The stream must belong to
 * the current device.  Every call on a device shares that device's array and leaves its
 * contents behind: calls that overlap on one device (two streams, or two threads) race.
 * It calls no hipMalloc, hipFree or other allocating routine.
 */
#define LA_NOALLOC_SCRATCH_BYTES (128u << 20)
int la_prefill_noalloc(int variant, int dtype, int batch, int heads, int64_t seq_len, int d_k,
                       int d_v, float eps, const void *q, const void *k, const void *v,
                       const void *alpha, const void *beta, const float *S0, const float *z0,
                       void *o, float *S_T, float *z_T, void *stream);

/*
 * la_decode_step -- one token for N independent states (e.g. N = sequences x heads): one
 * step of Eq. (1) of "History Replays Itself" (Sec. 2 Preliminary), or of the BASED
 * recurrence (reading notes Sec. 2.2-2.3), from the given state:
 *
 *   S_out = S_in A + beta v k^T,  o = S_out q      (BASED: s, z updated, o normalised)
 *
 * Layouts: S_in/S_out [N][d_v][d_k] fp32 (BASED: s [N][D][d_v], z [N][D]),
 * q, k [N][d_k], v, o [N][d_v], alpha, beta [N].  S_out may equal S_in (and z_out may
 * equal z_in) for an in-place update; any other overlap returns LA_ERR_ALIAS.  Each
 * state is read once and written once (this step is bound by HBM bandwidth).
 *
 * Supported: ADDITIVE/GATED/GATED_DELTA with d_k in {64, 128, 256} and any d_v >= 1;
 *            BASED and BASED_COMPACT with d' = 16, d_v = 64; q/k/v/alpha/beta/o in fp32
 *            or bf16.
 */
int la_decode_step(int variant, int dtype, int n, int d_k, int d_v, float eps, const float *S_in,
                   const float *z_in, float *S_out, float *z_out, const void *q, const void *k,
                   const void *v, const void *alpha, const void *beta, void *o, void *stream);

/*
 * la_state_scale -- S_out = lambda * S_in over n fp32 elements (any state: S, s or z).
 * The state handling around a NoteBank replay ("History Replays Itself", App. B
 * Algorithm 1 and App. C.3): the retrieval and read branches each work on their own copy
 * of the retained state, and at the readout boundary the state is rescaled, S <- lambda S
 * with lambda in [0, 1] (1 leaves it unchanged, 0 resets it; NoteBank uses 0 right before
 * replay).  lambda = 1 with distinct buffers is the copy.  lambda = 0 writes zeros
 * without reading S_in (which may then be NULL), so a reset also clears non-finite
 * values.  Products are single fp32 multiplications (correctly rounded).
 * S_out may equal S_in (in place); any other overlap returns LA_ERR_ALIAS.  Both must be
 * 16-byte aligned.  n = 0 is a no-op; n < 0 or lambda outside [0, 1] returns
 * LA_ERR_INVALID.  One read and one write of the state (bound by HBM bandwidth).
 */
int la_state_scale(int64_t n, float lambda, const float *S_in, float *S_out, void *stream);

/*
 * ---------------------------------------------------------------------------------
 * NoteBank write and address steps on the recurrence's keys and queries
 * ("History Replays Itself: Unleashing Long-Context Capability in Linear Attention",
 * Sec. 3 Eqs. (3)-(5), App. B.2 Eq. (8), App. B.3 Eq. (9)).  The channels (l, h) are the
 * heads of one layer (a caller with several layers stacks them as heads).  Argmax ties go
 * to the earliest index; the pages fix a tie rule only for the vote ranking (earlier-
 * inserted notes first), and the same rule is used throughout.  Choosing the note spans
 * from sentence boundaries needs the text and is the caller's: the library scores windows
 * and builds addresses for given spans.  All pointers are DEVICE memory; the calls are
 * asynchronous on `stream`; nothing is allocated.
 * ---------------------------------------------------------------------------------
 */

/*
 * la_write_scores -- key distinctiveness (Eqs. (3), (8)).  Per write chunk of `chunk`
 * tokens (the last, possibly partial, chunk over its own tokens) and head:
 *   khat_t = k_t / |k_t|,  mubar = normalised mean of khat over the chunk,
 *   d_head[b][h][t] = 1 - <khat_t, mubar>       (a zero key or mean normalises to zero)
 *   d_mean[b][t]    = (1/H) sum_h d_head[b][h][t]   (the channel average; may be NULL)
 * k [B][H][T][d_k] in `dtype` (LA_F32 / LA_BF16), 16-byte aligned; d_head [B][H][T] and
 * d_mean [B][T] fp32.  Computed in fp32 (one read of k from HBM).
 * Supported: d_k in {64, 128, 256}, chunk >= 1.
 */
int la_write_scores(int dtype, int batch, int heads, int64_t seq_len, int d_k, int chunk,
                    const void *k, float *d_head, float *d_mean, void *stream);

/*
 * la_write_windows -- the write step's best window (App. B.2): for every COMPLETE write
 * chunk c (a final incomplete chunk makes no note), the candidate region is
 * [max(0, c chunk - tail), (c + 1) chunk) -- the chunk plus the previous chunk's last
 * `tail` tokens with their own scores -- and every `window` consecutive tokens in it (the
 * whole region if it is shorter) are scored by the sum of d_mean.  best_start [B][T/chunk]
 * (int64) receives the highest-scoring window's first token, best_sum (fp32, may be NULL)
 * its score.  Sums in fp32.  Requires chunk >= 1, window >= 1, 0 <= tail <= chunk.
 */
int la_write_windows(int batch, int64_t seq_len, int chunk, int window, int tail,
                     const float *d_mean, int64_t *best_start, float *best_sum, void *stream);

/*
 * la_note_addresses -- native addresses (Eqs. (4), (9)).  For note i with span
 * spans[b][i] = (start, length) and head h: t_star[b][i][h] = argmax over the span of
 * d_head[b][h][t], and rho[b][i][h][r] = q[b][h][t*][coords[h][r]] (the query, in q's
 * dtype, at the head's fixed coordinates; not normalised).  q [B][H][T][d_k];
 * spans [B][N][2] int64; coords [H][d_rho] int32 (distinct values in [0, d_k) per head).
 * A span outside [0, T) (or empty) yields t_star = -1 and a zero address; a coordinate
 * outside [0, d_k) yields a zero entry (device data is not inspected on the host).
 * Supported: heads <= 16, 1 <= d_rho <= d_k.
 */
int la_note_addresses(int dtype, int batch, int heads, int64_t seq_len, int d_k, int n_notes,
                      int d_rho, const float *d_head, const void *q, const int64_t *spans,
                      const int32_t *coords, int64_t *t_star, void *rho, void *stream);

/*
 * la_address_votes -- addressing and voting (Eq. (5)).  rho [N][J][d_rho] note addresses,
 * u [n_query][J][d_rho] question features, both in `dtype`; in fp32 (App. B.3: both cast
 * to fp32 and l2-normalised):  score[j][i] = max_tau <uhat_tau, rhohat_i> (a zero vector
 * has cosine 0; score may be NULL), choice[j] = argmax_i score[j][i], votes[i] = number of
 * channels choosing i.  selected [R] receives up to R notes with the most votes (and at
 * least one; equal votes: the lower index, i.e. the earlier-inserted note) in document
 * order (by positions[i], int64, then index), padded with -1.
 * Supported: d_rho in {8, 16, 32}, n_query <= 1024, n_notes <= 16384, 1 <= R <= 64.
 */
int la_address_votes(int dtype, int n_notes, int channels, int n_query, int d_rho,
                     const void *rho, const void *u, int R, const int64_t *positions, float *score,
                     int32_t *choice, int32_t *votes, int32_t *selected, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LA_H */
