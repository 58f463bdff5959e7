/*
 * la.h -- C ABI of liblinattn, normalized kernelized linear attention on AMD MI355X (gfx950).
 *
 * The operation (all three entry points), with the feature map phi(x) = ELU(x) + 1 (alpha = 1)
 * applied element-wise to q and k:
 *
 *     o_i = phi(q_i)^T S_i / phi(q_i)^T z_i,   S_i = sum_{j in W(i)} phi(k_j) v_j^T,
 *                                              z_i = sum_{j in W(i)} phi(k_j)
 *
 *   causal  W(i) = {j <= i} (token i sees itself: the state is updated, then read)
 *           -- "Linear Attention Math", section "The recurrent form: a running KV state";
 *              "Linear Attention: Accumulating KV in a Fixed-Size State", section
 *              "Summarize state updates and reads with equations".
 *   global  W(i) = all tokens -- "Linear Attention Math", section "The associativity trick,
 *              written out"; "线性注意力从头到尾讲清楚", section 5 (matrix form).
 *   decode  one step of the causal recurrence on a caller-held state
 *           -- "Linear Attention Math", section "The recurrent form" (O(1) per token);
 *              "线性注意力从头到尾讲清楚", section 7 (only S_t and z_t are kept).
 * No epsilon is added to the denominator ("Linear Attention: From Pairwise Reads to a
 * Recurrent State", section "The reassociation that works—and the one that does not": a clamp
 * changes the operation).
 *
 * Layout: every tensor is contiguous, row-major, in device memory.
 *   q, k  [B, H, N, d]       dtype given by `dtype`
 *   v     [B, H, N, d_v]     dtype given by `dtype`
 *   out   [B, H, N, d_v]     dtype given by `dtype` (rounded to nearest even for bf16)
 *   S     [B, H, d, d_v]     float32; rows are key features, columns value components
 *   z     [B, H, d]          float32
 * Arithmetic is float32 throughout (bf16 operands of matrix-core products, float32 accumulation
 * and state). d and d_v must each be one of 16, 32, 64, 128. Pointers must be 16-byte aligned.
 * q, k and v must not overlap out; S and z must not overlap each other or q, k, v, out.
 *
 * Ownership and concurrency: all memory passed in belongs to the caller; the library never
 * frees or retains a caller pointer past the call. Work is enqueued on `stream` (NULL = the
 * null stream) and the call returns without waiting; the results are ready when the stream
 * reaches that point. Calls on different streams may run concurrently.
 * Scratch: the causal and global forms need temporary device memory for per-segment partial
 * states (size: la_workspace_bytes()).
 *   - la_causal_fwd_ws and la_global_fwd_ws take it from the caller (`ws`, `ws_bytes`): they
 *     allocate nothing, never wait on the host and keep no state between calls. The caller
 *     must not reuse or free `ws` before the stream has passed the call; calls running at the
 *     same time need workspaces of their own.
 *   - Every other entry point (the convenience forms) takes it from blocks the library caches
 *     per device until la_release_cache() or the end of the process. A call takes any free
 *     block large enough and makes its stream wait, on the device, for that block's last use
 *     (an event recorded after the kernels of the call that used it last); the host does not
 *     wait. When no free block is large enough, a new one is allocated with hipMalloc (which
 *     may wait for the device). Under stream capture the memory comes from the device's
 *     default stream-ordered pool instead (hipMallocAsync / hipFreeAsync: allocation nodes in
 *     the graph).
 *
 * Errors: every call validates all arguments before enqueuing anything and returns a status.
 *   LA_OK       enqueued
 *   LA_EINVAL   a required pointer is NULL or misaligned, a size is <= 0, decode with N != 1,
 *               dtype unknown, or buffers overlap as forbidden above; nothing was enqueued
 *   LA_ENOTSUP  valid but unsupported: d or d_v not in {16, 32, 64, 128}, chunk not accepted
 *               for this shape/dtype (see la_causal_fwd), or a size whose index arithmetic
 *               would overflow
 *   LA_EHIP     the HIP runtime reported an error (allocation or launch); work enqueued before
 *               the failure may have run
 *   LA_ENOSPACE la_causal_fwd_noalloc only: the call needs more scratch than the library's
 *               static array holds; nothing was enqueued
 * Nothing aborts, exits or throws across this interface.
 */
#ifndef LINATTN_LA_H
#define LINATTN_LA_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { LA_F32 = 0, LA_BF16 = 1 } la_dtype;

enum { LA_OK = 0, LA_EINVAL = 1, LA_ENOTSUP = 2, LA_EHIP = 3, LA_ENOSPACE = 4 };

/*
 * Variant flags of the *_ex entry points (bitwise or; any other bit set: LA_EINVAL).
 *   LA_PHI_IDENTITY  q and k are taken as already-mapped features: phi(x) = x. This is the
 *                    convention of the pages' worked examples ("Linear Attention:
 *                    Accumulating KV in a Fixed-Size State", section "Store Values according
 *                    to Key components") and the form that attention over precomputed
 *                    features (la_rf_features) takes. Features that are not positive can make
 *                    a denominator zero or negative; nothing is clamped.
 *   LA_UNNORMALIZED  out = phi(q_i)^T S_i, the weighted sum before the division by the score
 *                    sum (same page, sections "Read the state with a Query" and "Divide by
 *                    the sum of scores"). z is still accumulated and returned as part of the
 *                    state, so a state can be read both ways.
 */
enum { LA_PHI_IDENTITY = 1, LA_UNNORMALIZED = 2 };

/*
 * Causal prefill: out[b,h,i] = phi(q_i)^T S_i / phi(q_i)^T z_i over tokens j <= i, starting
 * from an optional carried state.
 *   S, z   both NULL: start from the zero state; the final state is not returned.
 *          both non-NULL: read as the state before token 0 (zero-fill them for a fresh
 *          sequence) and overwritten with the state after token N-1, so a long sequence can
 *          be processed in pieces and handed to la_decode_step. One NULL and one not: LA_EINVAL.
 *   chunk  tokens per intra-chunk tile: 0 lets the library choose (64 and the matrix-core
 *          kernel for bf16 with d = d_v in {64, 128}, 32 and the float32 matrix-core kernel for
 *          float32 with d = d_v in {64, 128}, else the vector-ALU kernel with chunk 16 for the
 *          causal forms -- a sequence of at most 64 tokens with d, d_v in {16, 32} and no decay
 *          as one chunk -- and 32 for the global form); 64 selects the matrix-core kernel for bf16
 *          with d = d_v in {64, 128}, 32 the float32 matrix-core kernel for float32 with
 *          d = d_v in {64, 128}; otherwise 16, 32, 64 or 128
 *          select the vector-ALU kernel (any supported d, d_v, either dtype) when its working
 *          set, 4 (d d_v + d + chunk (2 d + d_v) + chunk^2 + chunk) bytes, fits the 160 KiB of
 *          LDS of a workgroup (chunk 128 at d, d_v <= 32 or so). Other values, or a working set
 *          that does not fit: LA_ENOTSUP. Results are the same within rounding for every
 *          accepted chunk.
 * Defined by the recurrence S_i = S_{i-1} + phi(k_i) v_i^T, z_i = z_{i-1} + phi(k_i) of
 * "Linear Attention Math", section "The recurrent form: a running KV state"; the chunked
 * evaluation (within-chunk part plus the state carried from earlier chunks) is the one that
 * "Linear Attention: From Pairwise Reads to a Recurrent State", section "A recurrence need
 * not force token-serial training", describes.
 */
int la_causal_fwd(const void *q, const void *k, const void *v, void *out, float *S, float *z,
                  int B, int H, int N, int d, int d_v, int chunk, la_dtype dtype,
                  hipStream_t stream);

/*
 * Same as la_causal_fwd with an explicit sequence split: each (b, h) is cut into segments of
 * `seg_len` tokens (a positive multiple of the chunk in use) that run in parallel, joined by
 * an exclusive prefix over segment states. seg_len = 0 lets the library choose (what
 * la_causal_fwd does). A seg_len that is not a positive multiple of the chunk: LA_ENOTSUP.
 */
int la_causal_fwd_seg(const void *q, const void *k, const void *v, void *out, float *S,
                      float *z, int B, int H, int N, int d, int d_v, int chunk, int seg_len,
                      la_dtype dtype, hipStream_t stream);

/*
 * la_causal_fwd_seg with the initial and the final state in separate arguments:
 *   S0, z0 the state before token 0, read only; both NULL: the zero state (nothing is read,
 *          so a fresh sequence needs no zero-filled buffers).
 *   S, z   receive the state after token N-1; both NULL: not returned.
 * S0, z0 may be the same buffers as S, z (then this is la_causal_fwd_seg) or must not
 * overlap them; neither may overlap q, k, v, out. One of a pair NULL and the other not,
 * misalignment or a forbidden overlap: LA_EINVAL.
 * Same definition and citations as la_causal_fwd ("Linear Attention Math", section "The
 * recurrent form": S_0 = 0, z_0 = 0 for a fresh sequence).
 */
int la_causal_fwd_state(const void *q, const void *k, const void *v, void *out, const float *S0,
                        const float *z0, float *S, float *z, int B, int H, int N, int d, int d_v,
                        int chunk, int seg_len, la_dtype dtype, hipStream_t stream);

/*
 * la_causal_fwd_state with variant flags (LA_PHI_IDENTITY, LA_UNNORMALIZED; 0 gives
 * la_causal_fwd_state itself). Arguments, layout, ownership and errors as there.
 */
int la_causal_fwd_ex(const void *q, const void *k, const void *v, void *out, const float *S0,
                     const float *z0, float *S, float *z, int B, int H, int N, int d, int d_v,
                     int chunk, int seg_len, int flags, la_dtype dtype, hipStream_t stream);

/*
 * Causal prefill with a per-head decay of the carried state, the retention recurrence of
 * "Linear Attention Math", section "The kernel cousins: SSMs and RetNet" (linear attention plus an
 * explicit decay gamma < 1 of the state, scalar or per head):
 *     S_i = gamma_h S_{i-1} + phi(k_i) v_i^T,   z_i = gamma_h z_{i-1} + phi(k_i),
 *     out_i = phi(q_i)^T S_i / phi(q_i)^T z_i    (LA_UNNORMALIZED: phi(q_i)^T S_i)
 * RetNet's retention as stated there is flags = LA_PHI_IDENTITY | LA_UNNORMALIZED (its gated
 * normalisation is a separate learned layer, not part of this call). Equivalently, token j
 * reaches the read of token i with weight gamma^(i - j) (the parallel form); the chunked
 * evaluation applies that mask within a chunk and gamma^(i + 1 - t0) to the carried state.
 *   gamma  device memory, H float32 values (one per head, shared by the batch), 4-byte
 *          aligned, read only; values in [0, 1] (0 keeps only the current token, 1 is
 *          la_causal_fwd_ex). Values are not inspected on the host; one above 1 can overflow.
 *          A negative or NaN value makes every output and the state of its head NaN, in this
 *          form and in la_decode_step_decay alike (nothing is clamped).
 *          NULL, misaligned, or overlapping out, S or z: LA_EINVAL.
 * Every other argument, the layout, ownership and errors as for la_causal_fwd_ex (S0, z0: the
 * state before token 0; S, z: the state after token N-1, both in the decayed recurrence).
 */
int la_causal_fwd_decay(const void *q, const void *k, const void *v, void *out, const float *S0,
                        const float *z0, float *S, float *z, const float *gamma, int B, int H,
                        int N, int d, int d_v, int chunk, int seg_len, int flags, la_dtype dtype,
                        hipStream_t stream);

/*
 * Global (non-causal): S = phi(K)^T V and z = phi(K)^T 1 per (b, h) over all N tokens, then
 * out[b,h,i] = phi(q_i)^T S / phi(q_i)^T z for every token.
 *   S, z   required; written (not read) with the full-sequence state.
 *   q, out may both be NULL: only S and z are computed (a state summary of a context).
 *   chunk  as for la_causal_fwd (0, 16, 32, 64).
 * "Linear Attention Math", section "The associativity trick, written out";
 * "线性注意力从头到尾讲清楚", section 5, O = Phi(Q)(Phi(K)^T V) / Phi(Q)(Phi(K)^T 1).
 */
int la_global_fwd(const void *q, const void *k, const void *v, void *out, float *S, float *z,
                  int B, int H, int N, int d, int d_v, int chunk, la_dtype dtype,
                  hipStream_t stream);

/* la_global_fwd with variant flags (as for la_causal_fwd_ex; 0 gives la_global_fwd). */
int la_global_fwd_ex(const void *q, const void *k, const void *v, void *out, float *S, float *z,
                     int B, int H, int N, int d, int d_v, int chunk, int flags, la_dtype dtype,
                     hipStream_t stream);

/*
 * One recurrent decode step for B*H heads: N must be 1; q, k [B,H,1,d], v, out [B,H,1,d_v].
 *   S, z   required; read as the state before this token and updated in place:
 *          S <- S + phi(k) v^T, z <- z + phi(k); then out = phi(q)^T S / phi(q)^T z.
 *   chunk  ignored.
 * "Linear Attention Math", section "The recurrent form" (update, then read; constant time
 * and memory per token).
 */
int la_decode_step(const void *q, const void *k, const void *v, void *out, float *S, float *z,
                   int B, int H, int N, int d, int d_v, int chunk, la_dtype dtype,
                   hipStream_t stream);

/* la_decode_step with variant flags (as for la_causal_fwd_ex; 0 gives la_decode_step). */
int la_decode_step_ex(const void *q, const void *k, const void *v, void *out, float *S, float *z,
                      int B, int H, int N, int d, int d_v, int flags, la_dtype dtype,
                      hipStream_t stream);

/*
 * One decode step of the decayed recurrence (as for la_causal_fwd_decay): S <- gamma_h S +
 * phi(k) v^T, z <- gamma_h z + phi(k), then the read. gamma as for la_causal_fwd_decay; the
 * other arguments as for la_decode_step_ex.
 */
int la_decode_step_decay(const void *q, const void *k, const void *v, void *out, float *S, float *z,
                         const float *gamma, int B, int H, int N, int d, int d_v, int flags,
                         la_dtype dtype, hipStream_t stream);

/*
 * Profiling form of la_causal_fwd_ex: the same call enqueued `reps` times back to back on
 * `stream` (with S0 == S each call reads the state the previous one left; the work per call
 * is identical either way), with a HIP event recorded on that stream before and after each of
 * every call's kernels. The function then waits for the last event and writes the average
 * device time in milliseconds of each phase to ms[0..2]:
 *   ms[0] segment sums (segments 0..P-2), ms[1] exclusive scan over segment states,
 *   ms[2] causal outputs and final state; a phase the call did not launch gets 0 (about 0):
 *   with P = 1 the first two, on the bf16 matrix-core path (d = d_v in {64, 128}, chunk 64)
 *   the scan, since each causal segment adds up the sums before it itself.
 *   reps   1..4096; ms host array of 3 floats. reps out of range or ms NULL -> LA_EINVAL.
 * Blocks the calling thread until the work is done; for measurement, not for pipelines.
 * Errors as for la_causal_fwd_ex; a failure while creating or reading events -> LA_EHIP.
 */
int la_causal_fwd_profiled(const void *q, const void *k, const void *v, void *out,
                           const float *S0, const float *z0, float *S, float *z, int B, int H,
                           int N, int d, int d_v, int chunk, int seg_len, int flags,
                           la_dtype dtype, hipStream_t stream, int reps, float *ms);

/*
 * Positive random features: for rows x_i [rows, d] and projections W [m, d] (rows w_r),
 *     f[i][r] = exp(w_r . x_i - |x_i|^2 / 2) / sqrt(m),      f [rows, m]
 * so that f(q) . f(k) is an unbiased estimate of exp(q . k) when the w_r are drawn standard
 * normal ("Linear Attention Math", section "Feature maps: elu+1 and positive random
 * features"; "线性注意力从头到尾讲清楚", section 9, Performer's FAVOR+). The caller draws W
 * (seeded, orthogonalised or not): the library draws no random numbers. Attention over the
 * features is la_causal_fwd_ex / la_global_fwd_ex / la_decode_step_ex with LA_PHI_IDENTITY
 * and d = m (q and k both mapped with the same W).
 *   x, W, f  device memory, contiguous row-major, all of `dtype`; 16-byte aligned; f must not
 *            overlap x or W. For B*H*N tokens of a [B, H, N, d] tensor, rows = B*H*N.
 *   Arithmetic: float32 dots (bf16 operands of matrix-core products for bf16 with d in
 *   {64, 128} and m in {64, 128, 256}), float32 exponent, output rounded to nearest even.
 * Errors: NULL or misaligned pointer, rows, d or m <= 0, unknown dtype or a forbidden overlap:
 * LA_EINVAL; d > 256, m > 4096 or rows > 2^31 - 1: LA_ENOTSUP; launch failure: LA_EHIP.
 * Asynchronous on `stream` like the other entry points; no temporary memory.
 */
int la_rf_features(const void *x, const void *W, void *f, long rows, int d, int m,
                   la_dtype dtype, hipStream_t stream);

/*
 * Causal prefill over positive random features (Performer's FAVOR+ form, "Linear Attention
 * Math", section "Feature maps: elu+1 and positive random features"): with f as for
 * la_rf_features (one projection matrix W for q and k),
 *     out_i = f(q_i)^T S_i / f(q_i)^T z_i,  S_i = sum_{j <= i} f(k_j) v_j^T,  z_i = sum f(k_j)
 * (LA_UNNORMALIZED: f(q_i)^T S_i). Equal to la_rf_features on q and k followed by
 * la_causal_fwd_ex with LA_PHI_IDENTITY and d = m.
 *   q, k   [B, H, N, d];  v, out [B, H, N, d_v];  W [m, d] (rows = projections); all of dtype
 *   S0, z0 / S, z   the state over the m features: [B, H, m, d_v] and [B, H, m] float32, with
 *          the rules of la_causal_fwd_state (NULL pairs allowed as there)
 *   flags  0 or LA_UNNORMALIZED (LA_PHI_IDENTITY, or any other bit: LA_EINVAL)
 *   chunk, seg_len  as for la_causal_fwd_seg, for the attention over m features
 * When m == d == d_v in {64, 128}, dtype is bf16 and the matrix-core chunk applies, the map runs
 * inside the attention kernels' staging (W in LDS; no feature tensor is written to memory);
 * otherwise the features of q and k are written to scratch memory (2 B H N m elements of
 * dtype, taken as described at the top of this file) and read back.
 * Errors: as for la_causal_fwd_state (with S, z sized by m), plus W NULL, misaligned or
 * overlapping out or the state: LA_EINVAL; d > 256, or m, d_v not in {16, 32, 64, 128}:
 * LA_ENOTSUP.
 */
int la_causal_fwd_rf(const void *q, const void *k, const void *v, void *out, const void *W,
                     const float *S0, const float *z0, float *S, float *z, int B, int H, int N,
                     int d, int d_v, int m, int chunk, int seg_len, int flags, la_dtype dtype,
                     hipStream_t stream);

/*
 * Causal prefill with a caller-supplied workspace: la_causal_fwd_ex (gamma = NULL) or
 * la_causal_fwd_decay (gamma non-NULL: the per-head decay of the carried state, as there), with
 * the segment states in `ws` instead of library memory. Same definition, citations, arguments,
 * layout and results as those two calls.
 *   ws        device memory of at least la_workspace_bytes(0, B, H, N, d, d_v, chunk, seg_len,
 *             dtype) bytes, 16-byte aligned, owned by the caller; no part of it needs any
 *             initial value (every byte the call reads it first writes). May be NULL when that
 *             size is 0 (one segment per head).
 *   ws_bytes  its size in bytes.
 * The call allocates nothing, does not wait on the host and keeps no state: it is reentrant,
 * and usable under stream capture (the graph then holds kernel nodes only). `ws` belongs to
 * the call until the stream has passed it.
 * Errors: as for la_causal_fwd_ex / la_causal_fwd_decay, plus LA_EINVAL when the workspace is
 * needed and is NULL, misaligned, smaller than required, or overlaps q, k, v, out, S0, z0, S,
 * z or gamma.
 */
int la_causal_fwd_ws(const void *q, const void *k, const void *v, void *out, const float *S0,
                     const float *z0, float *S, float *z, const float *gamma, int B, int H, int N,
                     int d, int d_v, int chunk, int seg_len, int flags, la_dtype dtype, void *ws,
                     size_t ws_bytes, hipStream_t stream);

/*
 * Global form with a caller-supplied workspace: la_global_fwd_ex with the per-segment partial
 * sums in `ws` (la_workspace_bytes(1, B, H, N, d, d_v, chunk, 0, dtype) bytes; rules for `ws`,
 * `ws_bytes` and the errors as for la_causal_fwd_ws). Same definition and citations as
 * la_global_fwd ("Linear Attention Math", section "The associativity trick, written out").
 */
int la_global_fwd_ws(const void *q, const void *k, const void *v, void *out, float *S, float *z,
                     int B, int H, int N, int d, int d_v, int chunk, int flags, la_dtype dtype,
                     void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * la_causal_fwd_ex for callers that cannot allocate device memory (code under stream capture
 * that must not record allocation nodes, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments, definition and results, with the segment states in a static device
 * array of the library instead of allocated scratch. The call allocates nothing (no hipMalloc,
 * hipMallocAsync or pool memory; no host wait).
 *   Limit: 64 MiB of scratch per device, enough for every split the library chooses for the
 *   matrix-core kernels (bf16, d = d_v in {64, 128}); a call needing more
 *   (la_workspace_bytes(0, ...) > 64 MiB, e.g. a small explicit seg_len over many heads) returns
 *   LA_ENOSPACE and enqueues nothing.
 *   Sharing: every call on one device uses that device's one array, which keeps the last call's
 *   contents (no part of it needs an initial value: every byte a call reads it first writes).
 *   Calls that overlap in time on one device -- on different streams, or from several threads
 *   -- race on it: callers serialise them (e.g. one stream). The array is held until the
 *   process ends.
 * Errors: as for la_causal_fwd_ex, plus LA_ENOSPACE.
 */
int la_causal_fwd_noalloc(const void *q, const void *k, const void *v, void *out,
                          const float *S0, const float *z0, float *S, float *z, int B, int H,
                          int N, int d, int d_v, int chunk, int seg_len, int flags, la_dtype dtype,
                          hipStream_t stream);

/*
 * Frees the scratch blocks the convenience entry points cached, each after the work that last
 * used it has finished (this waits on the host). Blocks held by a call running on another
 * thread at that moment are kept. Returns LA_OK, or LA_EHIP if the runtime reported an error
 * (a block that could not be freed stays cached).
 */
int la_release_cache(void);

/* Bytes of scratch device memory a causal (form = 0) or global (form = 1)
 * call with these arguments takes (0 when none). seg_len as in la_causal_fwd_seg (0 = auto).
 * Returns 0 for invalid or unsupported arguments as well. */
size_t la_workspace_bytes(int form, int B, int H, int N, int d, int d_v, int chunk,
                          int seg_len, la_dtype dtype);

/* Segments per (b, h) head that a causal (form = 0) or global (form = 1) call with these
 * arguments splits the sequence into (they run in parallel; see la_causal_fwd_seg). Returns 0
 * for invalid or unsupported arguments. */
int la_segments(int form, int B, int H, int N, int d, int d_v, int chunk, int seg_len,
                la_dtype dtype);

/* Static, NUL-terminated description of a status code; never NULL. */
const char *la_strerror(int status);

/* Library version as (major << 16) | (minor << 8) | patch. */
int la_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LINATTN_LA_H */
