/*
 * mdn.h -- C ABI of the MI355X (gfx950) Momentum DeltaNet hot path.
 *
 * Operation (pages about "MDN: Parallelizing Stepwise Momentum for Delta
 * Linear Attention"; the MDN summary at paper.rainbus.top, method
 * walk-through step 1, and the ijyty.com article on MDN, section 3):
 *
 *     vtilde_t = v_t - S_{t-1}^T (alpha_t k_t)
 *     M_t      = mu_t M_{t-1} - eta_t k_t vtilde_t^T
 *     S_t      = alpha_t S_{t-1} - beta_t M_t
 *     o_t      = S_t^T q_t
 *
 * mdn_chunk_fwd evaluates this over a whole sequence with the chunkwise
 * parallel algorithm (summary, steps 2-5: log-domain coefficients, the
 * unit-lower T = (I + (P K^T) o Gamma^-)^{-1}, vtilde = U - Y S + Z M, the
 * intra-chunk term ((Q K^T) o Gamma) vtilde) and returns O, the final states
 * and the materialised vtilde (summary, step 7; article, section 6).
 * mdn_step is the one-token recurrent form used for generation (article,
 * section 6).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers are DEVICE pointers owned by the caller (e.g. torch tensors).
 *   The library allocates nothing, keeps no pointer after returning and has
 *   no mutable global state, so calls are reentrant.
 * - Every tensor is contiguous, row-major, in the layout stated per
 *   argument, and 16-byte aligned.
 * - dtype (mdn_dtype) is the element type of q, k, v, O, vtilde and o.
 *   Gates and the states S, M are always fp32.  In the bf16 path the
 *   matrix products take bf16 operands with fp32 accumulation; states,
 *   coefficients and every accumulation stay fp32.
 * - Gate preconditions (documented, not checked on the device): alpha, mu in
 *   (0, 1]; beta, eta >= 0 and finite.  The coefficients are formed from
 *   logarithms of alpha and mu, so a gate of exactly 0 is outside the
 *   contract (the results are undefined, not an error).
 * - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *   the call returns without synchronising.  Arguments are validated on the
 *   host before any HIP call; a failed validation enqueues nothing.
 *   Launch failures return MDN_ERR_HIP; device faults surface at the
 *   caller's next synchronisation.
 * - Return value: an mdn_status (0 = success).
 */
#ifndef MDN_H
#define MDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mdn_status {
    MDN_OK = 0,
    MDN_ERR_NULL_ARG = 1,    /* a required pointer is NULL */
    MDN_ERR_BAD_SHAPE = 2,   /* negative size, or sizes whose product overflows */
    MDN_ERR_UNSUPPORTED = 3, /* dtype / head dim / chunk size outside the compiled set */
    MDN_ERR_ALIAS = 4,       /* an output overlaps an input (other than the allowed aliases) */
    MDN_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required */
    MDN_ERR_ALIGN = 6,       /* a pointer is not 16-byte aligned */
    MDN_ERR_HIP = 7,         /* a HIP launch or runtime call failed */
    MDN_ERR_TOO_LARGE = 8    /* mdn_chunk_fwd_noalloc: workspace need above MDN_NOALLOC_SCRATCH_BYTES */
} mdn_status;

typedef enum mdn_dtype {
    MDN_F32 = 0,             /* fp32 q, k, v, outputs; fp32 matrix-core products */
    MDN_BF16 = 1             /* bf16 q, k, v, outputs; bf16 operands, fp32 accumulation */
} mdn_dtype;

/* Rows of the per-chunk coefficient block written by mdn_chunk_coef (and
 * kept in the workspace of mdn_chunk_fwd).  Each row holds C fp32 values
 * indexed by the chunk-local token r = 0..C-1.  Definitions (summary, steps 2
 * and 5; every cumulative quantity restarts at each chunk):
 *   LA    Lambda_alpha_r = sum_{s<=r} log alpha_s        (cumsum of logs)
 *   LM    Lambda_mu_r    = sum_{s<=r} log mu_s
 *   LOGC  log c_r = logcumsumexp_{j<=r}(log beta_j + LM_j - LA_j)
 *   ABAR  abar_r = exp(LA_r)
 *   B     b_r = exp(LA_r + LOGC_r) = sum_{j<=r} beta_j (abar_r/abar_j) mubar_j
 *   ABP   alpha_r * b_{r-1} (b_{-1} = 0): the momentum weight of the error term
 *   GS    Gamma_{C-1,i}: weight of k_i vtilde_i^T in the end-of-chunk S
 *   GM    eta_i mubar_{C-1}/mubar_i: weight of k_i vtilde_i^T in the end-of-chunk M
 * Tokens past the end of a ragged last chunk are padded with alpha = mu = 1,
 * beta = eta = 0 and zero q, k, v, which leaves every quantity unchanged. */
enum {
    MDN_COEF_ABAR = 0, MDN_COEF_ABP = 1, MDN_COEF_B = 2, MDN_COEF_GS = 3,
    MDN_COEF_GM = 4, MDN_COEF_LA = 5, MDN_COEF_LM = 6, MDN_COEF_LOGC = 7,
    MDN_COEF_ROWS = 8
};

/* Bytes of workspace mdn_chunk_fwd needs for these sizes (0 if none).
 * Returns (size_t)-1 when the sizes are invalid or unsupported.
 * Layout (documented for diagnostics; NT = ceil(T / C)):
 *   [B*H*NT][C][C]  T matrices   (dtype)
 *   [B*H*NT][C][C]  (Q K^T) o Gamma, zero above the diagonal (dtype)
 *   [B*H*NT][MDN_COEF_ROWS][C]  coefficients (fp32)
 * each section starting on a 256-byte boundary.  Both matrices are lower
 * triangular; for bf16 at C = 64 and fp32 at C >= 32 their upper-right
 * C/2 x C/2 quadrant (all zero) is not written, and nothing reads it.  For
 * a widened bf16 call (dk = 16 or C = 16, see mdn_chunk_fwd) the layout is
 * that of the fp32 call, followed by fp32 copies of q, k, v, O and Vtilde.
 * Where mdn_chunk_fwd would cut the sequences into segments (bf16, dk = dv
 * in {64, 128}, C = 64, few heads with long sequences; see
 * mdn_chunk_fwd_split) the size is mdn_chunk_fwd_split_workspace_bytes()
 * for that segment count, which depends on the current device's compute
 * units: query it with the device current that the call will run on. */
size_t mdn_chunk_fwd_workspace_bytes(int64_t B, int64_t H, int64_t T,
                                     int dk, int dv, int C, int dtype);

/* Chunkwise-parallel forward over a whole sequence.
 *   B, H, T     batch, heads, sequence length (any T >= 0; a last chunk
 *               shorter than C is handled by neutral padding; B*H == 0 or
 *               T == 0 is valid: with T == 0 only S_T, M_T are written,
 *               as copies of S0, M0).
 *   dk, dv      head dims: dk == dv, in {16, 32, 64, 128}.
 *   C           chunk size: {16, 32, 64}.
 *               The bf16 kernels contract in steps of 32 (the bf16 matrix
 *               op), so a bf16 call with dk = 16 or C = 16 is widened: q, k,
 *               v are copied to fp32 in the workspace (exactly), the fp32
 *               kernels run, and O, Vtilde are rounded to bf16 (nearest
 *               even).  Its arithmetic is the fp32 path's.
 *   q, k        [B][H][T][dk]  (dtype); every k_t is used as given.
 *   v           [B][H][T][dv]  (dtype)
 *   alpha, mu, beta, eta   [B][H][T] fp32, linear (not log) gates.
 *   S0, M0      [B][H][dk][dv] fp32 initial states, or NULL for zero.
 *   O           [B][H][T][dv]  (dtype) out: o_t = S_t^T q_t.
 *   S_T, M_T    [B][H][dk][dv] fp32 out: states after token T.  S_T may be
 *               exactly S0 and M_T exactly M0 (in-place update); any other
 *               overlap with an input is MDN_ERR_ALIAS.
 *   Vtilde      [B][H][T][dv]  (dtype) out: the materialised vtilde_t.
 *   workspace   device scratch of at least mdn_chunk_fwd_workspace_bytes();
 *               must not overlap any other argument.  Its contents on return
 *               follow the layout above.  Where that size includes the
 *               sequence split's state slots and the workspace holds them,
 *               the call runs mdn_chunk_fwd_split with the segment count the
 *               query chose (same results up to rounding); a workspace of
 *               only the single pass's size runs the single pass.
 *   stream      hipStream_t.
 */
int mdn_chunk_fwd(int64_t B, int64_t H, int64_t T, int dk, int dv, int C, int dtype,
                  const void* q, const void* k, const void* v,
                  const float* alpha, const float* mu, const float* beta, const float* eta,
                  const float* S0, const float* M0,
                  void* O, float* S_T, float* M_T, void* Vtilde,
                  void* workspace, size_t workspace_bytes, void* stream);

/* The whole forward in one kernel, without a workspace: the same arguments,
 * results and errors as mdn_chunk_fwd (up to rounding: it computes the
 * off-diagonal blocks of T with bf16 operands, where the two-kernel forward
 * keeps T in fp32), for
 *   dtype == MDN_BF16, C == 64, dk == dv in {64, 128};
 * any other size returns MDN_ERR_UNSUPPORTED.  The per-chunk quantities of
 * the summary's steps 2-5 (coefficients, Gamma, T, (Q K^T) o Gamma) stay on
 * chip, so HBM carries q, k, v, the gates, O, Vtilde and the states only.
 * On MI355X it is slower than mdn_chunk_fwd at these sizes (0.26 against
 * 0.21 ms on B8 H8 T4096 d128): each of a head's four workgroups computes
 * the head's whole intra-chunk stage.  Use it where no workspace can be
 * given or HBM bandwidth is shared. */
int mdn_chunk_fwd_fused(int64_t B, int64_t H, int64_t T, int dk, int dv, int C, int dtype,
                        const void* q, const void* k, const void* v,
                        const float* alpha, const float* mu, const float* beta, const float* eta,
                        const float* S0, const float* M0,
                        void* O, float* S_T, float* M_T, void* Vtilde, void* stream);

/* Chunkwise forward with each sequence cut into nseg segments that run side
 * by side, for batches with few heads and long sequences, whose single
 * serial pass over the chunks leaves most compute units idle.  The result
 * is that of mdn_chunk_fwd (up to rounding), on the same arguments plus
 * nseg; supported sizes are the natively compiled ones (fp32: dk = dv in
 * {16, 32, 64, 128}, C in {16, 32, 64}; bf16: dk = dv in {32, 64, 128},
 * C in {32, 64}); others, and nseg outside [2, MDN_SPLIT_MAX_SEGMENTS],
 * return MDN_ERR_UNSUPPORTED.
 *
 * Why it is exact: each chunk's update of the state pair [S; M] (summary,
 * steps 2 and 4: S' = abar S - b M + K^T Diag(gS) vtilde, M' = mubar M -
 * K^T Diag(gM) vtilde, with vtilde = T (V - Diag(abar) K S + Diag(alpha
 * b_prev) K M)) is affine in [S; M], with the same 2dk x 2dk linear part
 * for every state column.  A run of chunks therefore maps its start state
 * to its end state by one linear map Phi plus an offset.
 *   - Segment p holds chunks [p NT / nseg, (p + 1) NT / nseg), NT = ceil(T/C).
 *   - Pass 1: segment 0 from S0, M0 (its O and Vtilde are final); for each
 *     middle segment 1 .. nseg-2, the data from a zero state (the offset)
 *     and, with V = 0, the states S = I, M = 0 and S = 0, M = I (the
 *     columns of Phi).
 *   - Combine: the start state of segment p is Phi_{p-1} [S; M]_{p-1} +
 *     offset_{p-1}, in fp32, in order of p.
 *   - Pass 2: segments 1 .. nseg-1 from their start states.
 * The extra arithmetic is about 3x the state work of the middle segments.
 *   workspace   at least mdn_chunk_fwd_split_workspace_bytes(); the
 *               mdn_chunk_fwd layout, then the state slots (fp32).
 * Errors as mdn_chunk_fwd. */
#define MDN_SPLIT_MAX_SEGMENTS 64
size_t mdn_chunk_fwd_split_workspace_bytes(int64_t B, int64_t H, int64_t T,
                                           int dk, int dv, int C, int dtype, int nseg);
int mdn_chunk_fwd_split(int64_t B, int64_t H, int64_t T, int dk, int dv, int C, int dtype, int nseg,
                        const void* q, const void* k, const void* v,
                        const float* alpha, const float* mu, const float* beta, const float* eta,
                        const float* S0, const float* M0,
                        void* O, float* S_T, float* M_T, void* Vtilde,
                        void* workspace, size_t workspace_bytes, void* stream);

/* mdn_chunk_fwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, semantics and errors as mdn_chunk_fwd, without the
 * workspace: it uses a static device array of MDN_NOALLOC_SCRATCH_BYTES
 * instead, which every GPU the library runs on holds until the process
 * ends.  The call itself allocates nothing (no hipMalloc, no hipFree).
 *   - Problems whose mdn_chunk_fwd_workspace_bytes() exceeds
 *     MDN_NOALLOC_SCRATCH_BYTES return MDN_ERR_TOO_LARGE and enqueue
 *     nothing.  At dk = dv = 128, C = 64 in bf16 a chunk tile needs 18 KiB,
 *     so 80 MiB holds 4551 tiles: e.g. B*H = 64 heads of 4096 tokens, or
 *     16 heads of 16384 (4096 tiles each).
 *   - Every call on one GPU shares that GPU's array: calls that overlap in
 *     time on one GPU (two streams, two host threads) race and give
 *     undefined results.  Calls ordered on one stream are safe.
 *   - The first call on a device looks up the array's device address once
 *     (hipGetSymbolAddress, with that device current) and keeps it: this
 *     entry point is the one exception to "no mutable global state". */
#define MDN_NOALLOC_SCRATCH_BYTES (80ll << 20)
int mdn_chunk_fwd_noalloc(int64_t B, int64_t H, int64_t T, int dk, int dv, int C, int dtype,
                          const void* q, const void* k, const void* v,
                          const float* alpha, const float* mu, const float* beta, const float* eta,
                          const float* S0, const float* M0,
                          void* O, float* S_T, float* M_T, void* Vtilde, void* stream);

/* The two stages of mdn_chunk_fwd, exposed separately so that each kernel
 * can be timed or checked on its own.  mdn_chunk_fwd(args) is exactly
 * mdn_chunk_intra(args) followed by mdn_chunk_inter(args) on one stream.
 *
 * mdn_chunk_intra: coefficients (summary, step 5), T = (I + (P K^T) o
 *   Gamma^-)^{-1} and (Q K^T) o Gamma (steps 3-4) for every chunk, written to
 *   `workspace` (layout above).  Reads q, k and the gates only; same
 *   validation as mdn_chunk_fwd for the arguments it takes.
 * mdn_chunk_inter: the sequential inter-chunk stage: vtilde = T W, O and the
 *   S/M carry (step 4 and the closed form of step 2).  Takes the arguments of
 *   mdn_chunk_fwd and reads the workspace mdn_chunk_intra left for the same
 *   q, k and gates; the gates themselves are validated but not read.
 * Both take the natively compiled shapes only: a bf16 call with dk = 16 or
 * C = 16 (widened inside mdn_chunk_fwd) returns MDN_ERR_UNSUPPORTED. */
int mdn_chunk_intra(int64_t B, int64_t H, int64_t T, int dk, int dv, int C, int dtype,
                    const void* q, const void* k,
                    const float* alpha, const float* mu, const float* beta, const float* eta,
                    void* workspace, size_t workspace_bytes, void* stream);

int mdn_chunk_inter(int64_t B, int64_t H, int64_t T, int dk, int dv, int C, int dtype,
                    const void* q, const void* k, const void* v,
                    const float* alpha, const float* mu, const float* beta, const float* eta,
                    const float* S0, const float* M0,
                    void* O, float* S_T, float* M_T, void* Vtilde,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Backward of mdn_chunk_fwd: the gradients of a scalar loss L with respect
 * to every input, given dL/dO, dL/dS_T and dL/dM_T.  The pages print only
 * the forward; this is the chain rule applied to its chunk equations (the
 * summary, steps 2-5, in the form W = V - Diag(abar) K S + Diag(alpha_r
 * b_{r-1}) K M, vtilde = T W).  The chunk-start states are rebuilt from the
 * forward's materialised vtilde (the reason the forward stores it: summary,
 * step 7; article, section 6 and the Q&A), so v itself is not needed.
 *   B, H, T, dk, dv, C, dtype   as for mdn_chunk_fwd, with the same
 *               supported sizes (bf16 at dk = 16 or C = 16 widened to fp32
 *               in the workspace the same way: q, k, Vtilde, dO copied in,
 *               dq, dk_out, dv_out rounded back).
 *   q, k, alpha, mu, beta, eta, S0, M0   the forward's inputs (S0/M0 NULL
 *               for zero).
 *   Vtilde      [B][H][T][dv] (dtype): the forward's vtilde for these inputs.
 *   dO          [B][H][T][dv] (dtype): dL/dO.
 *   dS_T, dM_T  [B][H][dk][dv] fp32: dL/dS_T, dL/dM_T, or NULL for zero.
 *   dq, dk_out  [B][H][T][dk] (dtype) out;  dv_out [B][H][T][dv] (dtype) out.
 *   dalpha, dmu, dbeta, deta   [B][H][T] fp32 out.
 *   dS0, dM0    [B][H][dk][dv] fp32 out: dL/dS0, dL/dM0 (written whether or
 *               not S0, M0 were given).
 *   workspace   at least mdn_chunk_bwd_workspace_bytes(); no output may
 *               overlap an input or another output.
 * Gates must be positive and finite (the coefficients use their logs).
 * Errors as for mdn_chunk_fwd. */
size_t mdn_chunk_bwd_workspace_bytes(int64_t B, int64_t H, int64_t T,
                                     int dk, int dv, int C, int dtype);

int mdn_chunk_bwd(int64_t B, int64_t H, int64_t T, int dk, int dv, int C, int dtype,
                  const void* q, const void* k,
                  const float* alpha, const float* mu, const float* beta, const float* eta,
                  const float* S0, const float* M0, const void* Vtilde,
                  const void* dO, const float* dS_T, const float* dM_T,
                  void* dq, void* dk_out, void* dv_out,
                  float* dalpha, float* dmu, float* dbeta, float* deta, float* dS0, float* dM0,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Packed variable-length batch: nseq independent sequences of any lengths,
 * laid end to end along the token axis of every head, each starting from
 * its own state.  Each sequence computes exactly what mdn_chunk_fwd computes
 * for it alone (the recurrence of the summary, step 1, restarted at every
 * sequence start; chunked as in steps 2-5, with chunks that begin at the
 * sequence start and a short last chunk per sequence).  The packing is the
 * usual serving layout and is not itself on the pages.
 *   H, T        heads and packed length (sum of the sequence lengths);
 *               T <= INT32_MAX.
 *   nseq        number of sequences (0 is valid: nothing is written).
 *   cu_seqlens  [nseq + 1] int32, DEVICE memory, 4-byte aligned: sequence i
 *               is tokens [cu_seqlens[i], cu_seqlens[i+1]) of every head.
 *               Required: cu_seqlens[0] == 0, nondecreasing, cu_seqlens[nseq]
 *               == T.  This is not checked (the bounds live on the device);
 *               the kernels clamp every bound into [0, T], so a table that
 *               breaks it gives unspecified values but no access outside the
 *               arguments.  Empty sequences are allowed: their S_T, M_T are
 *               copies of S0, M0 (or zero).
 *   dk, dv, C, dtype   as for mdn_chunk_fwd.
 *   q, k        [H][T][dk] (dtype);  v, O, Vtilde  [H][T][dv] (dtype)
 *   alpha, mu, beta, eta   [H][T] fp32
 *   S0, M0      [nseq][H][dk][dv] fp32, or NULL for zero
 *   S_T, M_T    [nseq][H][dk][dv] fp32 out (exact aliases of S0, M0 allowed)
 *   workspace   at least mdn_chunk_fwd_varlen_workspace_bytes(); its layout
 *               is that of mdn_chunk_fwd with NT = T / C + nseq tile slots per
 *               head (sequence i owns slots from cu_seqlens[i] / C + i on),
 *               followed by a [NT][2] int32 slot table and the [nseq] int32
 *               dispatch order (sequences by length, longest first: their
 *               inter-chunk carries start first), each on a 256-byte
 *               boundary.
 * Errors as for mdn_chunk_fwd; a NULL cu_seqlens with nseq > 0 is
 * MDN_ERR_NULL_ARG, a misaligned one MDN_ERR_ALIGN. */
size_t mdn_chunk_fwd_varlen_workspace_bytes(int64_t H, int64_t T, int64_t nseq,
                                            int dk, int dv, int C, int dtype);

int mdn_chunk_fwd_varlen(int64_t H, int64_t T, int64_t nseq, const int32_t* cu_seqlens,
                         int dk, int dv, int C, int dtype,
                         const void* q, const void* k, const void* v,
                         const float* alpha, const float* mu, const float* beta, const float* eta,
                         const float* S0, const float* M0,
                         void* O, float* S_T, float* M_T, void* Vtilde,
                         void* workspace, size_t workspace_bytes, void* stream);

/* One recurrent decode step for every (batch, head), states updated in place
 * (article, section 6: generation runs the recurrence token by token).
 *   q, k        [B][H][dk] (dtype);  v [B][H][dv] (dtype)
 *   alpha, mu, beta, eta   [B][H] fp32
 *   S, M        [B][H][dk][dv] fp32, read and overwritten with S_t, M_t.
 *   o           [B][H][dv] (dtype) out.
 *   dk == dv in {16, 32, 64, 128} for both dtypes.
 * S and M must not overlap each other or any other argument. */
int mdn_step(int64_t B, int64_t H, int dk, int dv, int dtype,
             const void* q, const void* k, const void* v,
             const float* alpha, const float* mu, const float* beta, const float* eta,
             float* S, float* M, void* o, void* stream);

/* Measurement reference for mdn_step (not part of the method): reads every
 * fp32 of `buf` and writes it back multiplied by `scale`, in place, with the
 * decode step's access pattern (16-byte non-temporal loads, then stores,
 * 64 KiB per workgroup).  Over a buffer the size of the decode states it
 * gives the HBM bandwidth an in-place read-write stream attains, the
 * ceiling the decode step is compared with.
 *   buf     device buffer, 16-byte aligned; bytes a multiple of 16 (>= 0).
 *   scale   factor applied to every element (1 leaves the buffer unchanged).
 * Errors: MDN_ERR_BAD_SHAPE (bytes negative, not a multiple of 16, or beyond
 * 2^47), MDN_ERR_NULL_ARG, MDN_ERR_ALIGN, MDN_ERR_HIP. */
int mdn_stream_rw(void* buf, int64_t bytes, float scale, void* stream);

/* Diagnostic: the log-domain coefficient stage alone (summary, step 5), as
 * used inside mdn_chunk_fwd.
 *   alpha, mu, beta, eta   [B][H][T] fp32;  C in {16, 32, 64}.
 *   coef   out [B][H][NT][MDN_COEF_ROWS][C] fp32 (rows as defined above).
 *   gamma  out [B][H][NT][C][C] fp32: Gamma_{r,i} = eta_i gamma_{r,i} for
 *          i <= r, 0 above the diagonal; or NULL to skip. */
int mdn_chunk_coef(int64_t B, int64_t H, int64_t T, int C,
                   const float* alpha, const float* mu, const float* beta, const float* eta,
                   float* coef, float* gamma, void* stream);

/* Gate pre-operation and query correction: the elementwise step between a
 * layer's projections and the recurrence (summary, steps 6 and 7; article,
 * sections 5 and 8).  For every (b, h, t):
 *   eta   = tanh(x) + 1
 *   theta = arctan(s * eta),  alpha_max = cos^2 theta,  beta_max = sin^2 theta
 *   alpha = alpha_max * sigmoid(a),  beta = beta_max * sigmoid(b)
 *           (so alpha + beta <= 1: the stable-gating constraint)
 *   mu    = exp(clamp(mu_log, mu_log_min, 0))
 * and, when q_out is not NULL, the output correction of the query
 *   q_out[b][h][t][:] = q[b][h][t][:] - d[h] * k[b][h][t][:]
 * in fp32, rounded to dtype (round to nearest even for bf16).
 *   x, a, b, mu_log        [B][H][T] fp32 in (finite).
 *   alpha, mu, beta, eta   [B][H][T] fp32 out; they must not overlap each
 *                          other or any input.
 *   s                      scale inside arctan: finite and > 0 (1 in the
 *                          workloads here).
 *   mu_log_min             lower clamp of log mu: finite and <= 0 (-2 on the
 *                          pages).
 *   q, k                   [B][H][T][dk] (dtype) in, d [H] fp32 in, q_out
 *                          [B][H][T][dk] (dtype) out; either all four are
 *                          NULL (no correction) or none.  q_out may be
 *                          exactly q (in place); any other overlap is
 *                          MDN_ERR_ALIAS.  dk in {16, 32, 64, 128}.
 * A bad s or mu_log_min returns MDN_ERR_BAD_SHAPE. */
int mdn_gates(int64_t B, int64_t H, int64_t T, int dk, int dtype, float s, float mu_log_min,
              const float* x, const float* a, const float* b, const float* mu_log,
              float* alpha, float* mu, float* beta, float* eta,
              const void* q, const void* k, const float* d, void* q_out, void* stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* mdn_status_string(int status);

/* ABI revision of this header (incremented on any signature change). */
int mdn_abi_version(void);

#define MDN_ABI_VERSION 8

#ifdef __cplusplus
}
#endif

#endif /* MDN_H */
