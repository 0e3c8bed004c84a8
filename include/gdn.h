/*
 * gdn.h -- C ABI of the chunkwise gated delta rule forward for AMD MI355X (gfx950).
 *
 * The operation (per independent unit = one sequence x one head):
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t
 * with the state S of shape [Dv][Dk] (o = S q).  DeltaNet is the case alpha = 1.
 * Definition: Qiita article by Nyysyyan on the Linear Attention lineage, section
 * "Gated-DeltaNet" (update of S_i and the read h_i = S_i q_i); the same step order
 * (gate, predict, delta, write, read) is spelled out in the kkkzoz blog post
 * "linear-attention", sections "Gated DeltaNet" and "Workflow".
 *
 * gdn_chunk_fwd evaluates it chunk by chunk in the WY form with two kernels, a
 * parallel per-chunk prep and a serial per-sequence scan that also writes the
 * outputs: inside a chunk of C tokens the coupled writes are resolved by one
 * unit-lower-triangular solve
 * (LinearAttention系列解读(六)：DeltaNet的Chunkwise Form推导, sections 4.2-4.5; the
 * Qiita article, sections "Gated-DeltaNet" (triangular systems for W and U) and
 * "Chunk Computation"), and the state is carried serially from chunk to chunk.
 * The result equals the token recurrence up to rounding; the chunk size only
 * changes the rounding.
 *
 * Conventions shared by every entry point
 *  - All tensor arguments are DEVICE pointers (hipMalloc'd or torch CUDA tensors)
 *    to dense row-major arrays.  The caller owns every buffer, the workspace
 *    included; the library allocates nothing.  Its only global state is a cache
 *    of per-device queries (CU count, occupancy) and the static scratch buffer
 *    of gdn_chunk_fwd_noalloc (see there).
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default stream).
 *    Argument errors are detected on the host before anything is enqueued and
 *    nothing is written then.  Faults inside kernels surface at the caller's next
 *    synchronisation.  No C++ exception crosses this interface.
 *  - Floating-point inputs are not checked for NaN/Inf; they propagate.
 *  - Token-major layout: q, k [B][T][H][Dk], v and O [B][T][H][Dv]; per-token
 *    scalars log_alpha, beta [B][T][H] (fp32); states [N][H][Dv][Dk] (fp32).
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL = 1,          /* a required pointer is NULL */
    GDN_ERR_SHAPE = 2,         /* inconsistent or out-of-range sizes */
    GDN_ERR_UNSUPPORTED = 3,   /* (Dk, Dv, C, dtype) has no compiled kernel */
    GDN_ERR_WORKSPACE = 4,     /* workspace NULL or smaller than required */
    GDN_ERR_HIP = 5,           /* a HIP launch or runtime call failed */
    GDN_ERR_INTERNAL = 6,
    GDN_ERR_SCRATCH_LIMIT = 7  /* gdn_chunk_fwd_noalloc: the sizes need more than its static buffer */
} gdn_status;

typedef enum {
    GDN_F32 = 0,               /* q, k, v, O in fp32; all arithmetic in fp32 */
    GDN_BF16 = 1               /* q, k, v, O in bf16; fp32 accumulation and state */
} gdn_dtype;

/* The per-token update rule a chunked forward evaluates (see each entry point). */
typedef enum {
    GDN_RULE_DELTA = 0,        /* gdn_chunk_fwd:        S = a S (I - b k k^T) + b v k^T */
    GDN_RULE_MAMBA2 = 1,       /* gdn_mamba2_chunk_fwd: S = a S + b v k^T */
    GDN_RULE_GLA = 2           /* gdn_gla_chunk_fwd:    S = S diag(a) + b v k^T, a per key channel */
} gdn_rule;

/* Compiled (Dk, Dv, C, dtype) instantiations:
 *   (16, 16, 16, F32)  (64, 64, 16, F32)  (64, 64, 64, F32)
 *   (128, 128, 64, BF16) (128, 256, 64, BF16) (128, 128, 64, F32) (128, 256, 64, F32)
 * Returns 1 when the combination is compiled, 0 otherwise. */
int gdn_chunk_fwd_supported(int Dk, int Dv, int C, gdn_dtype dt);

/* As gdn_chunk_fwd_supported, for the entry point of `rule`.  Compiled for
 * GDN_RULE_MAMBA2 and GDN_RULE_GLA: (16, 16, 16, F32) (64, 64, 64, F32)
 * (128, 128, 64, BF16) (128, 256, 64, BF16).  0 for an unknown rule. */
int gdn_rule_supported(gdn_rule rule, int Dk, int Dv, int C, gdn_dtype dt);

/* As gdn_chunk_fwd_workspace_bytes, for the entry point of `rule`. */
size_t gdn_rule_workspace_bytes(gdn_rule rule, int B, int T, int H, int Dk, int Dv, int C,
                                int n_seqs, gdn_dtype dt);

/* Bytes of device workspace gdn_chunk_fwd needs for these sizes (0 on bad
 * sizes).  n_seqs is only read when cu_seqlens will be passed (B must then be
 * 1); pass n_seqs = 0 for fixed-length batches. */
size_t gdn_chunk_fwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, int C,
                                     int n_seqs, gdn_dtype dt);

/* Chunkwise forward over a batch.
 *
 *  q, k        [B][T][H][Dk] in dt.  Keys are used as given (no normalisation,
 *              no 1/sqrt(Dk) scale: the read is o = S q).
 *  v           [B][T][H][Dv] in dt.
 *  log_alpha   [B][T][H] fp32, log of the per-token gate alpha in (0, 1];
 *              NULL means alpha = 1 (DeltaNet).
 *  beta        [B][T][H] fp32, per-token write strength (not clamped).
 *  S0          [N][H][Dv][Dk] fp32 initial states; NULL means zero states.
 *              S0 and S_T are read and written in 16-byte pieces and must be
 *              16-byte aligned.
 *  cu_seqlens  NULL: the batch is N = B sequences of T tokens each.
 *              Otherwise a DEVICE int32 array [n_seqs + 1] of prefix offsets of
 *              n_seqs sequences packed along T (B must be 1, N = n_seqs):
 *              sequence i is tokens cu_seqlens[i] .. cu_seqlens[i+1]-1.  It must
 *              be non-decreasing with cu_seqlens[0] = 0 and cu_seqlens[n] = T;
 *              the device clamps it to a monotone sequence inside [0, T] so that
 *              no access leaves the buffers, and O rows of tokens outside every
 *              sequence are then left unwritten.  A sequence of length 0 gets
 *              S_T = S0.  Chunks never straddle two sequences.
 *  O           [B][T][H][Dv] in dt: o_t for every token.
 *  S_T         [N][H][Dv][Dk] fp32 final states; may be NULL (not written) and
 *              may equal S0 (updated in place).
 *  C           chunk size (16 or 64, see the instantiation list).
 *  workspace   device buffer of at least gdn_chunk_fwd_workspace_bytes(...)
 *              bytes, 16-byte aligned; its contents on entry are ignored and on
 *              return hold intermediates (no stable layout).  Two calls that
 *              overlap in time must not share a workspace.
 *  stream      hipStream_t to enqueue on.
 * With T = 0 nothing but S_T = S0 is computed and q, k, v, beta, O (and the
 * workspace, whose required size may then be 0) may be NULL.
 * Long sequences with few units: for a fixed-length batch of bf16 with
 * Dk = Dv = 128 or fp32 with Dk = Dv = 64 or 128 (C = 64), where a cost model
 * of the two paths (per-step costs measured on MI355X) puts the split scan of
 * gdn_chunk_fwd_split under 0.90 (bf16) or 0.95 (fp32) of the plain one (few units, or few units per
 * CU over long sequences), the call runs that split scan, with the span length
 * gdn_chunk_fwd_auto_span_chunks reports, when the workspace holds
 * gdn_chunk_fwd_workspace_bytes(...) for these sizes, which then includes room
 * for it; the results equal the plain scan's up to rounding.
 * gdn_chunk_fwd_profiled and gdn_chunk_fwd_noalloc always run the plain scan.
 * Errors: GDN_ERR_NULL (q, k, v, beta, O or workspace NULL), GDN_ERR_SHAPE
 * (B, H < 1, T < 0, n_seqs < 1 or B != 1 with cu_seqlens, more than 2^31-1
 * elements in a tensor, C * H * max(Dk, Dv) * element size above 2^31-1 bytes,
 * q/k/v/O/S0/S_T/workspace not 16-byte aligned),
 * GDN_ERR_UNSUPPORTED, GDN_ERR_WORKSPACE, GDN_ERR_HIP. */
gdn_status gdn_chunk_fwd(const void *q, const void *k, const void *v,
                         const float *log_alpha, const float *beta, const float *S0,
                         const int32_t *cu_seqlens, int n_seqs,
                         void *O, float *S_T,
                         int B, int T, int H, int Dk, int Dv, int C, gdn_dtype dt,
                         void *workspace, size_t workspace_bytes, void *stream);

/* Allocation-free variant of gdn_chunk_fwd, for callers that cannot allocate
 * device memory or pass a workspace: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments (minus the
 * workspace), same kernels and bitwise the same results as gdn_chunk_fwd; the
 * per-chunk intermediates go to a buffer of GDN_NOALLOC_SCRATCH_BYTES (64 MiB)
 * that the library holds in device memory, one copy per GPU, from its load
 * until the process ends.  The call itself allocates and frees nothing.
 *  - Limit: the call is refused with GDN_ERR_SCRATCH_LIMIT, before anything is
 *    enqueued, when gdn_chunk_fwd_workspace_bytes(...) for the same sizes
 *    exceeds GDN_NOALLOC_SCRATCH_BYTES (e.g. bf16, Dk = Dv = 128, C = 64 needs
 *    6912 bytes per chunk of 64 tokens and head: about 9700 chunk-heads).
 *  - Sharing: every call on one GPU uses that GPU's one buffer, which keeps the
 *    last call's contents; nothing in it needs to start at any value.  Calls
 *    ordered on one stream are safe; calls that overlap in time on one GPU (two
 *    streams, two host threads without ordering) race on the buffer and give
 *    undefined results.
 *  - The first call on each device looks up the buffer's device address
 *    (GDN_ERR_HIP if that fails).
 * Errors: as gdn_chunk_fwd (without GDN_ERR_WORKSPACE), plus
 * GDN_ERR_SCRATCH_LIMIT. */
#define GDN_NOALLOC_SCRATCH_BYTES (64ull << 20)
gdn_status gdn_chunk_fwd_noalloc(const void *q, const void *k, const void *v,
                                 const float *log_alpha, const float *beta, const float *S0,
                                 const int32_t *cu_seqlens, int n_seqs,
                                 void *O, float *S_T,
                                 int B, int T, int H, int Dk, int Dv, int C, gdn_dtype dt,
                                 void *stream);

/* gdn_chunk_fwd of a fixed-length batch with each sequence split into spans of
 * span_chunks chunks, for long sequences with few (sequence, head) units, where
 * one workgroup per state slice walking the whole sequence leaves most of the
 * GPU idle.  Over a span the state map is affine and the same for every row of
 * S: S_out = S_in M + b (the Qiita article on the Linear Attention lineage,
 * section "Gated-DeltaNet": the state after i tokens is an affine function of
 * S_0, gamma_i S_0 (I - W K^T) + sum (gamma_i / gamma_s) u_s k_s^T; section
 * "Chunk Computation": each chunk starts from the last state of the one before).
 * Three passes:
 *   1. every span's (M, b): the scan of the span with Dk extra state rows that
 *      start at the identity and take zero values (they end as M) next to the
 *      Dv rows from zero (they end as b);
 *   2. per sequence, in span order: S_in(0) = S0, S_in(p+1) = S_in(p) M_p + b_p,
 *      S_T = S_in(last + 1) (fp32 values; fp32 inputs: fp32 products, bf16
 *      inputs: products of operands split into two bf16 parts, about 2^-16
 *      relative error, fp32 sums);
 *   3. every span's outputs from its start state S_in(p).
 * The result equals gdn_chunk_fwd's up to rounding (passes 1 and 3 run the
 * same chunk arithmetic; pass 2 adds a rounding per span).  Passes 1 and 3 hold
 * (Dk + 2 Dv) / Dv times the state columns of one plain scan, spread over the
 * spans in parallel: it pays when B H Dv / 16 is well below the CU count, and
 * for long sequences that fill the device with few units (gdn_chunk_fwd's cost
 * model decides; see gdn_chunk_fwd_auto_span_chunks).
 * Arguments as gdn_chunk_fwd for a fixed-length batch (no cu_seqlens), plus:
 *  span_chunks  chunks per span (>= 1); the last span of a sequence may be
 *               shorter;
 *  workspace    at least gdn_chunk_fwd_split_workspace_bytes(...) bytes;
 *  kernel_ms    NULL, or a HOST array of 4 floats: then the call BLOCKS and
 *               returns the device milliseconds of [prep, pass 1, pass 2, pass 3].
 * Compiled for C = 64 with bf16 Dk = Dv = 128, fp32 Dk = Dv = 64 and fp32
 * Dk = Dv = 128 (GDN_ERR_UNSUPPORTED otherwise).  Errors: as gdn_chunk_fwd;
 * GDN_ERR_SHAPE also for span_chunks < 1 or more than 65535 spans in the batch. */
size_t gdn_chunk_fwd_split_workspace_bytes(int B, int T, int H, int Dk, int Dv, int C,
                                           int span_chunks, gdn_dtype dt);
/* Span length in chunks that gdn_chunk_fwd splits a call of these sizes into
 * on the current device (the cost model in gdn_chunk_fwd's description), or 0
 * when it runs the plain scan (also for sizes gdn_chunk_fwd rejects).
 * n_seqs > 0 (a packed batch) always gives 0. */
int gdn_chunk_fwd_auto_span_chunks(int B, int T, int H, int Dk, int Dv, int C, int n_seqs,
                                   gdn_dtype dt);
gdn_status gdn_chunk_fwd_split(const void *q, const void *k, const void *v,
                               const float *log_alpha, const float *beta, const float *S0,
                               void *O, float *S_T,
                               int B, int T, int H, int Dk, int Dv, int C, gdn_dtype dt,
                               int span_chunks, void *workspace, size_t workspace_bytes,
                               void *stream, float *kernel_ms);

/* Measurement variant of gdn_chunk_fwd: same arguments and result, plus
 * kernel_ms, a HOST array of 4 floats that receives the device time in
 * milliseconds of each kernel of this call, taken with HIP events recorded
 * on `stream` around every launch: [0] packed-batch chunk table (0 when
 * cu_seqlens is NULL), [1] prep (0 when there are no tokens), [2] scan (which
 * also writes O), [3] reserved, always 0.  Unlike gdn_chunk_fwd it BLOCKS until the call's
 * work on `stream` has finished.  Errors: as gdn_chunk_fwd, plus GDN_ERR_NULL
 * when kernel_ms is NULL. */
gdn_status gdn_chunk_fwd_profiled(const void *q, const void *k, const void *v,
                                  const float *log_alpha, const float *beta, const float *S0,
                                  const int32_t *cu_seqlens, int n_seqs,
                                  void *O, float *S_T,
                                  int B, int T, int H, int Dk, int Dv, int C, gdn_dtype dt,
                                  void *workspace, size_t workspace_bytes, void *stream,
                                  float *kernel_ms);

/* Chunked forward of the scalar-gated linear recurrence without the delta
 * rule's erase term (Mamba2 with a write strength beta):
 *     S_t = alpha_t S_{t-1} + beta_t v_t k_t^T,   o_t = S_t q_t
 * Definition: the Qiita article by Nyysyyan on the Linear Attention lineage,
 * section "Mamba2" (update of S_i, read h_i = S_i q_i; its closed form
 * H = S_0 Q D_gamma + V (Gamma o K^T Q)), here with V D_beta in place of V;
 * chunked as in that article's section "Chunk Computation" (Mamba2 case: the
 * chunk output from the chunk-start state and the in-chunk decays, then the
 * state handed to the next chunk).  It is the "GLA (scalar gate)" row of the
 * form table in LinearAttention系列解读(六)'s summary; with log_alpha NULL it is
 * plain linear attention (the Qiita article's section "Linear attention").
 * Arguments, layouts, ownership, asynchrony and errors as gdn_chunk_fwd, except:
 *  beta   [B][T][H] fp32, or NULL for beta = 1;
 *  workspace  at least gdn_rule_workspace_bytes(GDN_RULE_MAMBA2, ...) bytes;
 *  supported sizes: gdn_rule_supported(GDN_RULE_MAMBA2, ...). */
gdn_status gdn_mamba2_chunk_fwd(const void *q, const void *k, const void *v,
                                const float *log_alpha, const float *beta, const float *S0,
                                const int32_t *cu_seqlens, int n_seqs,
                                void *O, float *S_T,
                                int B, int T, int H, int Dk, int Dv, int C, gdn_dtype dt,
                                void *workspace, size_t workspace_bytes, void *stream);

/* Chunked forward of the linear recurrence with a per-channel (vector) gate,
 * without the erase term (vector-gated GLA with a write strength beta):
 *     S_t = S_{t-1} diag(alpha_t) + beta_t v_t k_t^T,   o_t = S_t q_t
 * where alpha_t = exp(log_alpha_t) holds one gate per key channel and scales
 * column c of S = [Dv][Dk] (the channel of k and q it multiplies).
 * Definition: LinearAttention系列解读(六)：DeltaNet的Chunkwise Form推导, section 1
 * (引言): the vector-gated GLA's state transition is a diagonal matrix that
 * scales each state element on its own, by an amount fixed by the gate, so in
 * the chunk form that scaling is split onto both sides of the causal mask.
 * The chunk form (derived from unrolling the update; the per-channel version
 * of the Qiita article's "Chunk Computation", Mamba2 case): with b_i the
 * in-chunk cumulative log-gate per channel,
 *     O = (Q o e^b) S^T + P diag(beta) V,   P_is = sum_d q_id k_sd e^{b_id - b_sd} (s <= i)
 *     S <- S diag(e^{b_n}) + V^T diag(beta) (K o e^{b_n - b}).
 * Arguments, layouts, ownership, asynchrony and errors as gdn_chunk_fwd, except:
 *  log_alpha  [B][T][H][Dk] fp32, one gate per key channel, each <= 0
 *             (alpha in (0, 1]); NULL means alpha = 1;
 *  beta       [B][T][H] fp32, or NULL for beta = 1;
 *  workspace  at least gdn_rule_workspace_bytes(GDN_RULE_GLA, ...) bytes (it
 *             holds decayed copies of q and k besides the per-chunk data);
 *  supported sizes: gdn_rule_supported(GDN_RULE_GLA, ...); GDN_ERR_SHAPE also
 *             when one chunk of log_alpha, C * H * Dk * 4 bytes, passes 2^31-1.
 * Any gate in range is handled exactly (a chunk whose decay across 16 tokens
 * passes e^64 on some channel takes a slower exact path for that block). */
gdn_status gdn_gla_chunk_fwd(const void *q, const void *k, const void *v,
                             const float *log_alpha, const float *beta, const float *S0,
                             const int32_t *cu_seqlens, int n_seqs,
                             void *O, float *S_T,
                             int B, int T, int H, int Dk, int Dv, int C, gdn_dtype dt,
                             void *workspace, size_t workspace_bytes, void *stream);

/* gdn_chunk_fwd_profiled for the entry point of `rule` (same arguments as
 * that entry point, then kernel_ms; kernel_ms[1] is the per-chunk preparation
 * of that rule: prep for GDN_RULE_DELTA, the gates kernel for
 * GDN_RULE_MAMBA2 (0 where the scan forms the gate rows itself, as it does
 * for the 64-column bf16 slices and for fp32 with C = 64), the GLA prep
 * kernel for GDN_RULE_GLA).  Blocks until the call's work has finished. */
gdn_status gdn_rule_chunk_fwd_profiled(gdn_rule rule, const void *q, const void *k, const void *v,
                                       const float *log_alpha, const float *beta, const float *S0,
                                       const int32_t *cu_seqlens, int n_seqs,
                                       void *O, float *S_T,
                                       int B, int T, int H, int Dk, int Dv, int C, gdn_dtype dt,
                                       void *workspace, size_t workspace_bytes, void *stream,
                                       float *kernel_ms);

/* One token per sequence (decoding).  Updates the state in place and reads it:
 *     S <- alpha S (I - beta k k^T) + beta v k^T,   o = S q     (same section).
 *  q, k [N][H][Dk] in dt; v [N][H][Dv] in dt; log_alpha (nullable: alpha = 1)
 *  and beta [N][H] fp32; S [N][H][Dv][Dk] fp32, read and written in place;
 *  o [N][H][Dv] in dt.  S must be 16-byte aligned (its rows are read and
 *  written as 16-byte pieces; GDN_ERR_SHAPE otherwise).
 * Supported (Dk, Dv): any with Dk, Dv in {16, 64, 128, 256}, both dtypes.
 * Errors: GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_UNSUPPORTED, GDN_ERR_HIP. */
gdn_status gdn_recurrent_step(const void *q, const void *k, const void *v,
                              const float *log_alpha, const float *beta,
                              float *S, void *o,
                              int N, int H, int Dk, int Dv, gdn_dtype dt, void *stream);

/* Static English text for a status code (never NULL). */
const char *gdn_status_string(gdn_status s);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
