/*
 * gdn.h -- C ABI of the gated delta rule layer core for MI355X (gfx950).
 *
 * The operation (Gated Delta Networks paper, section 3.1, eq. (10)):
 *
 *     S_t = S_{t-1} ( alpha_t (I - beta_t k_t k_t^T) ) + beta_t v_t k_t^T
 *     o_t = S_t q_t                      S_t in R^{dv x dk},  alpha_t = exp(log_alpha_t)
 *
 * evaluated two ways:
 *   gdn_chunk_fwd    -- chunkwise-parallel prefill over whole sequences
 *                       (paper section 3.3, the WY/UT chunk algorithm with the
 *                       decay mask; paper-notes blog, "Hardware-Efficient
 *                       Chunkwise Training", summary (4)), optionally packed
 *                       with cu_seqlens, from an initial state, returning the
 *                       final state.
 *   gdn_decode_step  -- one token of the recurrence for a batch of resident
 *                       states, updated in place (tutorial page, decode
 *                       recursion S_t = S_{t-1} A_t + B_t).
 * and differentiated:
 *   gdn_chunk_bwd    -- gradients of gdn_chunk_fwd's outputs with respect to
 *                       all of its inputs (for training).
 * gdn_chunk_fwd_noalloc is gdn_chunk_fwd for callers that cannot allocate
 * device memory: it uses a scratch array of the library instead of a
 * workspace argument.
 *
 * Both return the same numbers as the recurrence up to floating-point
 * rounding.  Chunked, single-step and save-then-resume evaluations agree
 * (tutorial: the three paths must line up; independent samples reset the
 * state, a continued request does not).
 *
 * CONVENTIONS (all calls)
 *   - Every pointer argument except `stream` is a DEVICE pointer (HBM) unless
 *     stated otherwise.  Tensors are dense, row-major, last index fastest.
 *   - The caller owns every buffer.  The library keeps no pointer after the
 *     call returns and allocates no device memory on these paths (the one
 *     device array it owns is gdn_chunk_fwd_noalloc's scratch array, which
 *     exists while the library is loaded).
 *   - Work is enqueued on `stream` (NULL = the default stream) and the call
 *     returns without waiting.  Buffers must stay valid until the stream
 *     reaches that point.  A kernel fault shows up at the caller's next
 *     synchronisation, as for any HIP launch.
 *   - All argument checks run before anything is enqueued: a call that
 *     returns an error status has launched nothing and written nothing.
 *     gdn_last_error_message() then describes the failure (thread-local).
 *   - q, k, v, o, the state buffers and the workspace must be 16-byte
 *     aligned; log_alpha, beta and cu_seqlens 4-byte aligned
 *     (GDN_ERR_ALIGN otherwise).
 *   - Calls are reentrant and may run concurrently on different streams with
 *     disjoint buffers.
 *   - Preconditions that are documented but NOT checked on the device:
 *     finite inputs; log_alpha <= 0; beta in [0, 1] (any finite beta is
 *     computed as given); q and k normalised upstream (the paper normalises
 *     them in the token-mixing block, section 3.4).  With 16-bit inputs the
 *     matrix-core operands are fp16, so |q|, |k|, |v| and the state entries
 *     must stay below 65504.  Outside that range nothing reports an error:
 *     bf16 q, k and v reach their fp16 operands through a round-toward-zero
 *     conversion and saturate silently at +-65504, and a state entry that is
 *     rounded to an fp16 operand (round to nearest) becomes infinite.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 5

typedef enum {
    GDN_OK = 0,
    GDN_ERR_NULL = 1,         /* a required pointer is NULL                       */
    GDN_ERR_SHAPE = 2,        /* sizes negative, zero where not allowed, or
                                 inconsistent                                     */
    GDN_ERR_DTYPE = 3,        /* unknown dtype code                               */
    GDN_ERR_ALIGN = 4,        /* a device pointer is misaligned (see CONVENTIONS) */
    GDN_ERR_UNSUPPORTED = 5,  /* well-formed but not built (head dims, chunk size,
                                 dtype combination)                               */
    GDN_ERR_WORKSPACE = 6,    /* workspace NULL or smaller than required          */
    GDN_ERR_HIP = 7,          /* a HIP runtime call or launch failed              */
    GDN_ERR_ALIAS = 8,        /* an output overlaps an input it may not overlap   */
    GDN_ERR_DEVICE_INPUT = 9  /* device-side validation failed (gdn_chunk_fwd_check) */
} gdn_status;

typedef enum {
    GDN_FP32 = 0,
    GDN_BF16 = 1,
    GDN_FP16 = 2
} gdn_dtype;

/*
 * Options of gdn_chunk_fwd (gdn_chunk_desc.flags) and gdn_decode_step.
 *   GDN_QK_L2NORM  q and k are L2-normalised per (token, head) inside the
 *                  kernels, q / ||q||_2 and k / ||k||_2, as the Gated
 *                  DeltaNet paper's token-mixing block does before the delta
 *                  rule (section 3.4, "Token mixer block"; the paper notes
 *                  list it for training stability).  The input buffers are
 *                  not modified.  An all-zero vector stays zero.
 */
typedef enum {
    GDN_QK_L2NORM = 1
} gdn_flags;

/*
 * Shape of one gdn_chunk_fwd call.
 *   batch     B  >= 1: batch rows.  Must be 1 when cu_seqlens is given.
 *   seqlen    T  >= 0: tokens per batch row (packed batch: total tokens).
 *   heads     H  >= 1.
 *   dk           key/query head dim: 32, 64, 128 or 256 (fp32 inputs: <= 128).
 *   dv           value head dim: a multiple of 16, 16..1024.
 *   num_seqs  N: number of sequences.  Without cu_seqlens it must equal B
 *                (row b is sequence b); with cu_seqlens, N >= 1 and the
 *                cu_seqlens array holds N+1 offsets.
 *   chunk     C: chunk length; 64 is the supported value.
 *   in_dtype     dtype of q, k, v (FP32, BF16 or FP16).  BF16/FP16 inputs run
 *                the matrix products on fp16 operands with fp32 accumulation
 *                and an fp32 state; FP32 inputs run them on fp32 operands.
 *   out_dtype    dtype of o (FP32, BF16 or FP16).
 *   flags        bitwise OR of gdn_flags (0: none).
 */
typedef struct {
    int32_t batch;
    int32_t seqlen;
    int32_t heads;
    int32_t dk;
    int32_t dv;
    int32_t num_seqs;
    int32_t chunk;
    int32_t in_dtype;   /* gdn_dtype */
    int32_t out_dtype;  /* gdn_dtype */
    int32_t flags;      /* gdn_flags */
} gdn_chunk_desc;

/* ABI version of the loaded library (GDN_ABI_VERSION at build time). */
int gdn_abi_version(void);

/* Static, human-readable name of a status code. */
const char *gdn_status_string(gdn_status status);

/* Detail of the last failed call on this thread ("" if none).  The pointer is
 * valid until the next gdn_* call on the same thread. */
const char *gdn_last_error_message(void);

/*
 * Workspace for gdn_chunk_fwd, in bytes, written to *bytes (host pointer).
 * Depends only on the descriptor (and on GDN_SEG_CHUNKS, below).  The
 * workspace holds the chunk table built from cu_seqlens and, per (chunk,
 * head), the UT-transform matrix T diag(beta), the decay-masked Q K^T block
 * and the chunk's decay factors (exp of the cumulative log-decay from the
 * chunk start, and to the chunk end).  When the state pass is segmented (a
 * batch with too few (sequence, head) pairs to fill the GPU: each sequence's
 * chunks are cut into segments whose affine state maps S -> S F + G are
 * formed in parallel and then chained, the algebra of the paper's chunk-level
 * state recurrence, section 3.3, applied to runs of chunks) it also holds the
 * segment table and, per (segment, head), the map [G; F] ((dv + dk) x dk
 * fp32) and the segment's incoming state (dv x dk fp32).  The environment
 * variable GDN_SEG_CHUNKS, read at every call, fixes the segment length in
 * chunks (0 = never segment); unset, the library chooses.  The workspace
 * need not be initialised and may be reused by later calls that are ordered
 * after this one on the stream.
 * Errors: GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_DTYPE, GDN_ERR_UNSUPPORTED.
 */
gdn_status gdn_chunk_fwd_workspace_size(const gdn_chunk_desc *desc, size_t *bytes);

/*
 * Chunkwise-parallel forward pass (prefill).
 *
 *   q           [B, T, H, dk]  in_dtype
 *   k           [B, T, H, dk]  in_dtype
 *   v           [B, T, H, dv]  in_dtype
 *   log_alpha   [B, T, H]      fp32, log of the forget gate alpha_t
 *   beta        [B, T, H]      fp32, write strength beta_t
 *   init_state  [N, H, dv, dk] fp32 or NULL (zeros).  S[n,h] maps keys to
 *                              values, row index = value dim (paper 2.1).
 *   cu_seqlens  int32 [N+1] or NULL.  Packed batch (B == 1): sequence n is
 *               tokens cu[n] .. cu[n+1]-1 of the T axis; cu[0] = 0,
 *               non-decreasing, cu[N] = T.  Empty sequences are allowed
 *               (their final state equals their initial state).  The state
 *               restarts from init_state[n] at every sequence start, and
 *               chunks restart there too (the last chunk of a sequence may
 *               be partial).  The array is checked on the device; a
 *               malformed one makes the kernels write nothing and is
 *               reported by gdn_chunk_fwd_check.
 *   o           [B, T, H, dv]  out_dtype (written)
 *   final_state [N, H, dv, dk] fp32 or NULL (not returned).  May be the
 *               same pointer as init_state (in-place continuation): each
 *               state tile is read before it is written and tiles are
 *               disjoint.  Partial overlap with init_state is not allowed.
 *   workspace   device buffer of at least gdn_chunk_fwd_workspace_size bytes
 *   stream      HIP stream the kernels are launched on
 *
 * Evaluation: when the call averages more than 16 tokens per sequence
 * (B*T > 16*N) it runs the chunkwise algorithm (paper section 3.3) with
 * 64-token chunks.  Otherwise each (sequence, head) state is read and
 * written once by one kernel: for 16-bit inputs with dk <= 128 the same
 * chunkwise algorithm with 16-token chunks on the matrix cores, else the
 * recurrence itself token by token; either is cheaper for a few tokens per
 * sequence.  The environment variable GDN_SMALL_CHUNKS=0, read at every
 * call, sends such calls to the token-by-token kernel.  All compute eq. (10)
 * with fp32 state and accumulation and meet the same bounds; bit-identical
 * results are guaranteed between calls that take the same branch.
 *
 * o must not overlap any input or the state buffers (GDN_ERR_ALIAS).
 * Errors: GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_DTYPE, GDN_ERR_ALIGN,
 * GDN_ERR_UNSUPPORTED, GDN_ERR_WORKSPACE, GDN_ERR_ALIAS, GDN_ERR_HIP.
 */
gdn_status gdn_chunk_fwd(const gdn_chunk_desc *desc,
                         const void *q, const void *k, const void *v,
                         const float *log_alpha, const float *beta,
                         const float *init_state, const int32_t *cu_seqlens,
                         void *o, float *final_state,
                         void *workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * gdn_chunk_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, semantics and errors as gdn_chunk_fwd, without the
 * workspace: the library's own scratch array stands in for it, a
 * GDN_NOALLOC_SCRATCH_BYTES device array per GPU that exists from the moment
 * the library is loaded until the process ends.  Its device address is
 * looked up (hipGetSymbolAddress) on the first call on each device; the call
 * itself allocates nothing.
 *   - A call whose gdn_chunk_fwd_workspace_size exceeds
 *     GDN_NOALLOC_SCRATCH_BYTES returns GDN_ERR_WORKSPACE and writes nothing
 *     (64 MiB covers, e.g., B = 4, T = 4096, H = 16, dk = dv = 128 with
 *     16-bit inputs).
 *   - Every call on a GPU uses that GPU's one array.  Calls that may overlap
 *     in time on one GPU (different streams, or different host threads
 *     without ordering) race on it and must not be issued; calls ordered on
 *     one stream are safe.  Nothing in the array has to start at a known
 *     value: each call writes every part of it that it reads.
 *   - A malformed cu_seqlens makes the kernels write nothing, as in
 *     gdn_chunk_fwd, but is not reported (gdn_chunk_fwd_check needs the
 *     workspace pointer).
 */
#define GDN_NOALLOC_SCRATCH_BYTES (64u << 20)
gdn_status gdn_chunk_fwd_noalloc(const gdn_chunk_desc *desc,
                                 const void *q, const void *k, const void *v,
                                 const float *log_alpha, const float *beta,
                                 const float *init_state, const int32_t *cu_seqlens,
                                 void *o, float *final_state, hipStream_t stream);

/*
 * Workspace for gdn_chunk_bwd, in bytes, written to *bytes (host pointer).
 * Depends only on the descriptor.  Besides the chunk table it holds, per
 * (chunk, head), the fp32 UT-transform matrix T = (I + A)^{-1}, the
 * decay-masked Q K^T and K K^T blocks and the decay vectors (49 KiB at
 * C = 64), the
 * state and the state's gradient at every chunk boundary (2 * dv * dk * 4
 * bytes) and three C x dv fp32 chunk intermediates.  Prefill with B = 4,
 * T = 4096, H = 16, dk = dv = 128 needs about 1 GiB.  With GDN_QK_L2NORM
 * in desc->flags it also holds the normalised q and k and v as fp32 rows and
 * the two normalisation factors, (2 dk + dv + 2) * 4 bytes per (token, head).
 * Errors: GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_DTYPE, GDN_ERR_UNSUPPORTED.
 */
gdn_status gdn_chunk_bwd_workspace_size(const gdn_chunk_desc *desc, size_t *bytes);

/*
 * Backward pass of gdn_chunk_fwd: given the gradients of a loss with respect
 * to o and to the final state, the gradients with respect to every input.
 * The pages call the chunkwise algorithm a training method (paper section
 * 3.3) but give no gradient formulas; these follow from differentiating the
 * recurrence of eq. (10), evaluated on the chunked form.  The forward pass
 * is recomputed from the inputs (nothing from gdn_chunk_fwd is kept).
 *
 *   desc, q, k, v, log_alpha, beta, init_state, cu_seqlens
 *               as for gdn_chunk_fwd (desc->out_dtype is not used)
 *   d_o            [B, T, H, dv]  fp32, dL/do
 *   d_final_state  [N, H, dv, dk] fp32 or NULL (zeros): dL/d final state
 *   dq, dk         [B, T, H, dk]  fp32 (written)
 *   dv             [B, T, H, dv]  fp32 (written)
 *   dlog_alpha     [B, T, H]      fp32 (written), dL/d log_alpha
 *   dbeta          [B, T, H]      fp32 (written)
 *   d_init_state   [N, H, dv, dk] fp32 or NULL (not returned): dL/d init_state
 *                  (with init_state NULL it is the gradient at a zero state)
 *   workspace      at least gdn_chunk_bwd_workspace_size bytes
 *
 * Supported: dk 32, 64 or 128; dv a multiple of 16 up to 1024; flags 0 or
 * GDN_QK_L2NORM.  With GDN_QK_L2NORM the gradients are those of the call
 * that normalised q and k (paper section 3.4, token mixer block): the
 * backward kernels run on q^ = q / ||q||, k^ = k / ||k|| (fp32 rows in the
 * workspace) and dq, dk are carried back through the normalisation,
 * dx = (dx^ - x^ (x^ . dx^)) / ||x||, zero for an all-zero row.  All
 * gradient arithmetic has fp32 precision for every input dtype (products
 * with a 16-bit q or k factor may run on the 16-bit matrix cores with the
 * other factor split exactly into three bf16 terms).  Tokens past a
 * sequence's end are not written.  With cu_seqlens the array is checked on
 * the device as in gdn_chunk_fwd; a malformed one makes the kernels write
 * nothing and gdn_chunk_fwd_check(workspace, ...) reports it.
 * The outputs must not overlap each other, any input or the workspace
 * (GDN_ERR_ALIAS).
 * Errors: GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_DTYPE, GDN_ERR_ALIGN,
 * GDN_ERR_UNSUPPORTED, GDN_ERR_WORKSPACE, GDN_ERR_ALIAS, GDN_ERR_HIP.
 */
gdn_status gdn_chunk_bwd(const gdn_chunk_desc *desc,
                         const void *q, const void *k, const void *v,
                         const float *log_alpha, const float *beta,
                         const float *init_state, const int32_t *cu_seqlens,
                         const float *d_o, const float *d_final_state,
                         float *dq, float *dk, float *dv,
                         float *dlog_alpha, float *dbeta, float *d_init_state,
                         void *workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * Result of the device-side cu_seqlens check of the last gdn_chunk_fwd (or
 * packed gdn_chunk_bwd) that used `workspace`.  Synchronises `stream`, then writes 0 (valid) or a
 * non-zero code (1: cu[0] != 0, 2: decreasing offsets, 3: cu[N] != T) to
 * *code (host pointer).  Returns GDN_ERR_DEVICE_INPUT when the code is
 * non-zero, GDN_OK otherwise.
 */
gdn_status gdn_chunk_fwd_check(const void *workspace, hipStream_t stream, int32_t *code);

/*
 * One decode step for N resident states, in place.
 *
 *   state      [N, H, dv, dk] fp32, read and overwritten with S_t
 *   q, k       [N, H, dk]     in_dtype
 *   v          [N, H, dv]     in_dtype
 *   log_alpha  [N, H]         fp32
 *   beta       [N, H]         fp32
 *   o          [N, H, dv]     out_dtype, o = S_t q (read after the update)
 *
 * Per (n, h) it computes, reading each state row once and writing it once:
 *   Sbar = alpha S;  u = beta (v - Sbar k);  S_t = Sbar + u k^T;
 *   o = alpha (S q) + u (k . q)
 * (tutorial page: forget first, then correct the error of the decayed
 * memory).  flags: 0 or GDN_QK_L2NORM (q and k normalised first).
 * dk: 32, 64, 128 or 256.  dv: 1..4096.
 * o must not overlap state.
 * Errors: GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_DTYPE, GDN_ERR_ALIGN,
 * GDN_ERR_UNSUPPORTED, GDN_ERR_ALIAS, GDN_ERR_HIP.
 */
gdn_status gdn_decode_step(int32_t N, int32_t H, int32_t dk, int32_t dv,
                           int32_t in_dtype, int32_t out_dtype, int32_t flags,
                           float *state,
                           const void *q, const void *k, const void *v,
                           const float *log_alpha, const float *beta,
                           void *o, hipStream_t stream);

/*
 * Per-kernel timing for measurement harnesses (host-side bookkeeping only;
 * kernels are unchanged).  While enabled, every launch made by this library
 * is bracketed by a pair of HIP events recorded on the launch stream.
 *   gdn_profile_enable(1) clears previous records and starts recording;
 *   gdn_profile_enable(0) stops recording.
 *   gdn_profile_read synchronises the recorded events and reports, for the
 *   i-th distinct kernel name (0 <= i < count), its name (static string),
 *   the number of recorded launches and their summed duration in ms.
 * gdn_profile_read(i, ...) with i >= count returns GDN_ERR_SHAPE.
 */
gdn_status gdn_profile_enable(int32_t on);
gdn_status gdn_profile_count(int32_t *count);
gdn_status gdn_profile_read(int32_t index, const char **name, int64_t *launches,
                            double *total_ms);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
