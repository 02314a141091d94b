/*
 * libkda -- Kimi Delta Attention (KDA) operator for AMD Instinct MI355X (gfx950).
 *
 * The operator is the per-head gated delta-rule recurrence defined in the
 * "Kimi K3 Technical Report review" (jw9603.github.io), sections 3.2-3.3:
 *
 *     Sbar_{t-1} = Diag(alpha_t) S_{t-1}            (key channel i kept at rate alpha_t[i])
 *     S_t        = Sbar_{t-1} + beta_t k_t (v_t - Sbar_{t-1}^T k_t)^T
 *     o_t        = S_t^T q_t                          (read from the updated state)
 *
 * with S_t in R^{d_k x d_v}.  Decay is applied before the write.  There is no
 * readout scale and keys are used as given (the library does not normalise them).
 *
 * Conventions shared by every call:
 *  - All tensor pointers are DEVICE pointers (HIP global memory) owned by the
 *    caller.  The bf16 prefill with d_k in {64, 128} (kda_chunk_fwd, its
 *    snapshot, packed-batch and gated forms, and a split of one part) keeps its
 *    per-chunk intermediates ("chunk records", about 1 KB per token and head) in
 *    device memory it takes from a memory pool the library creates on each
 *    device at first use and keeps: allocated and freed in stream order on
 *    `stream` around the call, at most 1 GiB of records per buffer (2 GiB when a
 *    long batch's blocks overlap); when that memory cannot be had, or a packed
 *    batch's records exceed the cap, the call runs a kernel that needs none.
 *    kda_chunk_fwd_split_noalloc never allocates.  Beyond that pool the library
 *    keeps, per device, its compute-unit count and the address of the
 *    allocation-free call's array, and a thread-local copy of the last HIP
 *    error.  Calls are reentrant.
 *  - `stream` is the hipStream_t the work is enqueued on (NULL = the default
 *    stream).  Each call only enqueues work on that stream and returns without
 *    synchronising; a device-side fault surfaces at the caller's next
 *    synchronisation.
 *  - Layouts are dense, row-major, token-major: [B][T][H][d] for per-token
 *    tensors and [B][H][d_k][d_v] for states.
 *  - Every pointer must be 16-byte aligned.
 *  - Arguments are validated before any HIP call; on error nothing is enqueued
 *    and no output is touched.  Calls never abort and never throw.
 *  - Supported sizes: d_k, d_v in {16, 32, 64, 128}, for bf16 and fp32 q/k/v.
 *  - Arithmetic.  The state is carried in fp32 and every product accumulates in
 *    fp32.  With fp32 q/k/v all matrix-core operands are fp32.  With bf16 q/k/v
 *    the matrix-core operands are fp16: the decayed keys and queries, the
 *    factors of the intra-chunk key products (each bounded by |k| or |q|: every
 *    decay ratio inside a chunk is split at a power-of-two block boundary into
 *    two products of decays; the single-kernel form used without a workspace
 *    takes inverse-decayed keys, at most e^10 |k|, and processes a chunk whose
 *    decay would exceed that as shorter exact segments), and the state and
 *    values rescaled by a power of two per state column, so their magnitude is
 *    not restricted.  q and k entries should stay below 6.5e4 in magnitude.
 *    (Head sizes served by the generic kernel form the intra-chunk key products
 *    from bf16 high/low pairs instead, about 16 significant bits.)
 *  - Input domain: alpha in [exp(-5), 1] (the lower-bounded decay of section 3.5
 *    of the same page); results outside it are not guaranteed, except that the
 *    bf16 prefill with d_k in {64, 128} on its chunk-record path accepts any
 *    alpha in [0, 1].  beta may be any finite value (it is not clamped).
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>

#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KDA_F32 = 0,  /* IEEE binary32 */
  KDA_BF16 = 1  /* bfloat16; outputs are rounded to nearest even */
} kda_dtype;

typedef enum {
  KDA_OK = 0,
  KDA_ERR_NULL = 1,        /* a required pointer is NULL */
  KDA_ERR_SHAPE = 2,       /* B, H < 1, T < 0, or a size overflows 2^31 elements per row index */
  KDA_ERR_DTYPE = 3,       /* qkv_dtype or o_dtype is not a kda_dtype */
  KDA_ERR_UNSUPPORTED = 4, /* d_k/d_v not in {16,32,64,128} or chunk not in {16,32,64} */
  KDA_ERR_MISALIGNED = 5,  /* a pointer is not 16-byte aligned */
  KDA_ERR_ALIAS = 6,       /* an output overlaps an input it may not overlap */
  KDA_ERR_HIP = 7          /* the launch failed; kda_last_hip_error() holds the hipError_t */
} kda_status;

/*
 * Chunkwise-parallel prefill over T tokens for B sequences and H heads.
 *
 * The sequence is cut into chunks of `chunk` tokens (the chunkwise form of the
 * second page, "Kimi 모델 분석", rlaope.github.io, section on putting the
 * recurrence on the GPU: chunk size 64, WY representation, UT transform, only
 * the state carried between chunks).  The result equals the token recurrence
 * above up to rounding, for any chunk size.
 *
 *   q, k   : [B][T][H][d_k]  qkv_dtype          (read)
 *   v      : [B][T][H][d_v]  qkv_dtype          (read)
 *   alpha  : [B][T][H][d_k]  fp32, per-channel retention   (read)
 *   beta   : [B][T][H]       fp32, write strength          (read)
 *   S0     : [B][H][d_k][d_v] fp32 initial state, or NULL for zeros   (read)
 *   o      : [B][T][H][d_v]  o_dtype, o_t for every token             (written)
 *   o_dtype: KDA_F32 or KDA_BF16 (the q/k/v dtype is the usual choice).  A
 *            bf16 o is exactly the fp32 result rounded to nearest even; that
 *            rounding alone can reach 2^-8 of |o_t|, so an fp32 o keeps the full
 *            accuracy of the fp32 state.
 *   S_T    : [B][H][d_k][d_v] fp32 final state, or NULL to skip       (written)
 *   chunk  : 16, 32 or 64 (64 is the size the second page names).  The chunk
 *            size a call actually runs: 32 for chunk 32 or 64 with bf16 q/k/v,
 *            d_k in {64, 128} and d_v a multiple of 32 (the pipelined kernel,
 *            whose stage rings of 64-token chunks would not fit the 160 KB of
 *            LDS), and for chunk 64 with fp32 q/k/v and d_k in {64, 128} (same
 *            reason); the requested size otherwise.  The result does not depend
 *            on the chunk size beyond rounding.
 *
 * S0 == S_T (the same buffer) is allowed and updates the state in place; any
 * other overlap between an output and an input returns KDA_ERR_ALIAS.
 * T == 0 writes S_T = S0 (zeros when S0 is NULL) and touches nothing else.
 * Any T >= 1 is accepted; a partial last chunk is masked.
 */
kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                         const float* alpha, const float* beta, const float* S0,
                         void* o, kda_dtype o_dtype, float* S_T,
                         int B, int T, int H, int d_k, int d_v, int chunk, hipStream_t stream);

/*
 * The chunk size a kda_chunk_fwd call with these arguments runs (see `chunk`
 * above), written to *run_chunk.  Host only: enqueues nothing and touches no
 * device.  Errors: KDA_ERR_DTYPE, KDA_ERR_SHAPE (H < 1), KDA_ERR_UNSUPPORTED
 * (a size or chunk that kda_chunk_fwd would refuse), KDA_ERR_NULL.
 */
kda_status kda_chunk_fwd_run_chunk(kda_dtype qkv_dtype, int H, int d_k, int d_v, int chunk, int* run_chunk);

/* Most positions one kda_chunk_fwd_snapshots call records. */
#define KDA_MAX_SNAPSHOTS 128

/*
 * kda_chunk_fwd that also records the state at caller-chosen positions, for
 * prefix caching.  A KDA layer keeps no per-token keys and values: resuming a
 * shared prompt prefix needs the state at exactly that position, and saving it
 * at every token is too costly, so a server saves it at positions it selects --
 * at a fixed interval, or where a prompt ends (the second page, "Kimi 모델
 * 분석", section on prefix caching breaking and its parts on separating block
 * size from caching granularity and on where to store the summaries).
 *
 * Every argument of kda_chunk_fwd keeps its meaning; in addition:
 *   snap_tokens: HOST array of n_snap token counts, strictly increasing, each
 *                in [1, T] and a multiple of `chunk` or equal to T.  Entry j
 *                asks for the state after the first snap_tokens[j] tokens of
 *                every sequence, S_{snap_tokens[j]} (read during the call only).
 *   n_snap     : 0 .. KDA_MAX_SNAPSHOTS (0: identical to kda_chunk_fwd).
 *   snaps      : [B][H][n_snap][d_k][d_v] fp32, device (written).  Snapshot j
 *                of (b, h) is the same value kda_chunk_fwd's S_T would hold for
 *                the first snap_tokens[j] tokens with the same S0 (bit for bit:
 *                the chunks before it are computed identically).
 *
 * Errors, in addition to kda_chunk_fwd's: KDA_ERR_SHAPE for n_snap outside
 * [0, KDA_MAX_SNAPSHOTS] or a position list that breaks the rules above;
 * KDA_ERR_NULL for a NULL snap_tokens or snaps with n_snap > 0;
 * KDA_ERR_MISALIGNED / KDA_ERR_ALIAS for snaps as for the other outputs.
 */
kda_status kda_chunk_fwd_snapshots(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                                   const float* alpha, const float* beta, const float* S0,
                                   void* o, kda_dtype o_dtype, float* S_T,
                                   const int* snap_tokens, int n_snap, float* snaps,
                                   int B, int T, int H, int d_k, int d_v, int chunk, hipStream_t stream);

/*
 * One batched decode step: one new token for each of B sequences and H heads,
 * i.e. exactly one step of the recurrence, applied to the state in place.
 *
 *   q, k   : [B][H][d_k] qkv_dtype        v: [B][H][d_v] qkv_dtype   (read)
 *   alpha  : [B][H][d_k] fp32             beta: [B][H] fp32          (read)
 *   S      : [B][H][d_k][d_v] fp32, read and overwritten with S_t    (in place)
 *   o      : [B][H][d_v] o_dtype (KDA_F32 or KDA_BF16), o_t         (written)
 *
 * Each state is streamed once from HBM and written back once.  o must not
 * overlap S or any input (KDA_ERR_ALIAS).
 */
kda_status kda_decode_step(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                           const float* alpha, const float* beta, float* S, void* o, kda_dtype o_dtype,
                           int B, int H, int d_k, int d_v, hipStream_t stream);

/*
 * kda_chunk_fwd over a packed batch of N sequences of different lengths (for
 * serving: prompts of a batch are concatenated along the token axis).  Sequence
 * b covers token rows [cu_seqlens[b], cu_seqlens[b+1]) and is an independent
 * recurrence with its own initial and final state.
 *
 *   q, k, alpha: [total_T][H][d_k]   v, o: [total_T][H][d_v]   beta: [total_T][H]
 *                (dtypes as in kda_chunk_fwd)
 *   S0, S_T    : [N][H][d_k][d_v] fp32 (S0 may be NULL; S_T may be NULL or S0)
 *   cu_seqlens : [N + 1] int32, DEVICE memory, non-decreasing from 0 to total_T.
 *                The kernels clamp each offset to [0, total_T] and each length
 *                to >= 0, so no offset can make them access memory out of
 *                range; o rows not covered by any sequence are not written.
 *   N          : >= 1 sequences;  total_T >= 0.
 *
 * Validation and errors as kda_chunk_fwd (cu_seqlens must be non-NULL and
 * 16-byte aligned, and may not overlap an output).  A sequence's results equal
 * kda_chunk_fwd run on that sequence alone up to rounding.
 */
kda_status kda_chunk_fwd_varlen(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                                const float* alpha, const float* beta, const float* S0,
                                void* o, kda_dtype o_dtype, float* S_T,
                                const int* cu_seqlens, int N, int total_T,
                                int H, int d_k, int d_v, int chunk, hipStream_t stream);

/*
 * kda_chunk_fwd with the gate fused in: instead of alpha, the caller passes the
 * gate pre-activation z and a per-head log-scale A, and the kernels form the
 * lower-bounded retention of section 3.5 of the first page,
 *     alpha_t[i] = exp(-5 * sigmoid(exp(A_h) * z_t[i]))      (in (e^-5, 1)),
 * in fp32 as they read z, so no fp32 alpha tensor is stored or read: the
 * per-token-head input shrinks from 4*d_k to 2*d_k bytes with bf16 z.
 *
 *   z : [B][T][H][d_k] in qkv_dtype (read)        A : [H] fp32, device (read)
 * Every other argument as kda_chunk_fwd.  The result equals kda_chunk_fwd with
 * alpha = the formula above evaluated in fp32 (the exponentials and the
 * reciprocal use the hardware's approximations, within a few fp32 ulps).
 */
kda_status kda_chunk_fwd_gated(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                               const void* z, const float* A, const float* beta, const float* S0,
                               void* o, kda_dtype o_dtype, float* S_T,
                               int B, int T, int H, int d_k, int d_v, int chunk, hipStream_t stream);

/*
 * Prefill with each sequence split into parts that run side by side: for few
 * long sequences (small B*H) the single-pass kernel has one workgroup per
 * (sequence, head, 32 state columns) and leaves most of the GPU idle.  Between
 * chunks only the state is carried (the second page, on putting the recurrence
 * on the GPU), and a run of tokens maps its incoming state S to M S + N with a
 * d_k x d_k transition M (section 3.3 of the first page: each token applies
 * (I - beta k k^T) Diag(alpha) to every state column and adds beta k v^T), so:
 * pass 1 computes N and M of every part but the last, in parallel; a combine
 * step chains S_in(j+1) = M_j S_in(j) + N_j in fp32 (from 9 parts on, as a tree
 * over the part maps: log2 levels of pairwise compositions, then one product
 * with S0); pass 2 reruns every part from its S_in and writes o and S_T.  Parts
 * are whole 32-token chunks.
 *
 *   parts     : 0 = the library's choice (a step-count model of the launches
 *               on num_cus compute units against the single pass the call would
 *               otherwise run; 1 part when splitting does not pay);
 *               1 = the single pass (kda_chunk_fwd); >= 2 = that many parts, or
 *               fewer when T has fewer 32-token chunks.
 *   num_cus   : compute units for the model; 0 = those of the current device.
 *   workspace : device memory of workspace_bytes bytes, 16-byte aligned, used
 *               for the transitions and incoming states; its contents on entry
 *               do not matter and are overwritten.  May be NULL when the
 *               resulting split has 1 part.  kda_chunk_fwd_split_plan gives the
 *               part count and the bytes needed:
 *               4 * B * H * d_k * (c * (P - 1) * (d_v + d_k) + P * d_v) for P
 *               parts, with c = 1 below 9 parts and c = 2 from 9 parts on.
 * Every other argument as kda_chunk_fwd.  Splitting is built for the pipelined
 * kernel's shapes (bf16 q/k/v, d_k in {64, 128}, d_v a multiple of 32, chunk 32
 * or 64); parts >= 2 for another shape returns KDA_ERR_UNSUPPORTED.  Errors:
 * as kda_chunk_fwd, plus KDA_ERR_NULL (workspace NULL when needed),
 * KDA_ERR_SHAPE (workspace_bytes too small, parts or num_cus < 0),
 * KDA_ERR_ALIAS (workspace overlaps an input or output), KDA_ERR_HIP (the
 * device's compute units could not be queried).  The result equals
 * kda_chunk_fwd up to rounding (the state entering each part goes through one
 * fp32 product with M instead of the chunk recurrence).  Three kernels are
 * enqueued on `stream` below 9 parts; from 9 parts on, 3 + ceil(log2(P - 1)).
 */
kda_status kda_chunk_fwd_split_plan(kda_dtype qkv_dtype, int B, int T, int H, int d_k, int d_v, int chunk,
                                    int parts, int num_cus, int* parts_out, size_t* workspace_bytes);
kda_status kda_chunk_fwd_split(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                               const float* alpha, const float* beta, const float* S0,
                               void* o, kda_dtype o_dtype, float* S_T,
                               int B, int T, int H, int d_k, int d_v, int chunk,
                               int parts, int num_cus, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of device scratch kda_chunk_fwd_split_noalloc holds on each GPU (64 MiB). */
#define KDA_SPLIT_SCRATCH_BYTES ((size_t)64 << 20)

/*
 * kda_chunk_fwd_split for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.  The
 * same split prefill, with its workspace in a fixed device array of
 * KDA_SPLIT_SCRATCH_BYTES that the library holds on each GPU it runs on (from
 * when the library's code is loaded on that GPU until the process ends).  The
 * call allocates nothing; the caller still passes every input and output.
 *
 *   parts : 0 = the library's choice among part counts whose workspace fits
 *           the scratch (1, the single pass, needs none); >= 2 = that many
 *           parts (or fewer, as kda_chunk_fwd_split), KDA_ERR_SHAPE when
 *           their workspace (kda_chunk_fwd_split_plan) exceeds
 *           KDA_SPLIT_SCRATCH_BYTES.
 * Every call on one GPU uses that GPU's one array and overwrites what the last
 * call left there: calls that overlap on one GPU (on other streams or from
 * other threads) race and must be ordered by the caller.  Every other argument
 * and error as kda_chunk_fwd_split; KDA_ERR_HIP also when the array's device
 * address cannot be obtained (kda_last_hip_error() holds the hipError_t).
 */
kda_status kda_chunk_fwd_split_noalloc(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                                       const float* alpha, const float* beta, const float* S0,
                                       void* o, kda_dtype o_dtype, float* S_T,
                                       int B, int T, int H, int d_k, int d_v, int chunk,
                                       int parts, int num_cus, hipStream_t stream);

/*
 * kda_decode_step with the gate fused in (as kda_chunk_fwd_gated):
 *   z : [B][H][d_k] in qkv_dtype (read)           A : [H] fp32, device (read)
 */
kda_status kda_decode_step_gated(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                                 const void* z, const float* A, const float* beta, float* S, void* o,
                                 kda_dtype o_dtype, int B, int H, int d_k, int d_v, hipStream_t stream);

/* Most draft tokens one speculative step may verify. */
#define KDA_MAX_DRAFT 16

/*
 * Speculative decoding, pass 1 of 2: verify K draft tokens of each of B
 * sequences without changing the state.  Each decode step overwrites the state
 * in place, so a rejected draft token could not be taken back afterwards (the
 * second page, "Kimi 모델 분석", serving section on speculative decoding; the
 * first page, section 13, on restoring the state after rejected draft tokens).
 * This call reads S once and gives what K kda_decode_step calls would (the
 * same recurrence, restated, in fp32): S is multiplied once by every draft's
 * key and query, each decayed to the draft's position, and the drafts' effect
 * on one another is resolved on those products with coefficients formed from
 * k, q and alpha alone.  It stores what the commit pass needs instead of the
 * state.
 *
 *   q, k   : [B][K][H][d_k] qkv_dtype     v: [B][K][H][d_v] qkv_dtype   (read)
 *   alpha  : [B][K][H][d_k] fp32          beta: [B][K][H] fp32          (read)
 *   S      : [B][H][d_k][d_v] fp32, the state before the drafts (read only)
 *   o      : [B][K][H][d_v] o_dtype: o_t as if tokens 1..t were accepted (written)
 *   u      : [B][H][K][d_v] fp32: the write vectors u_t = beta_t (v_t - Sbar^T k_t)
 *            of the K updates S_t = Diag(alpha_t) S_{t-1} + k_t u_t^T   (written)
 *   K      : 1 .. KDA_MAX_DRAFT
 *
 * o and u may overlap nothing else (KDA_ERR_ALIAS).  Other rules as for
 * kda_decode_step.
 */
kda_status kda_decode_verify(const void* q, const void* k, const void* v, kda_dtype qkv_dtype,
                             const float* alpha, const float* beta, const float* S,
                             void* o, kda_dtype o_dtype, float* u,
                             int B, int K, int H, int d_k, int d_v, hipStream_t stream);

/*
 * Speculative decoding, pass 2 of 2: advance the state over the accepted
 * prefix.  For sequence b, j = n_accept[b] (clamped to [0, K]) tokens were
 * accepted; S becomes the state after them,
 *     S_j = Diag(P_j) S + sum_{t<j} Diag(P_j / P_{t+1}) k_t u_t^T,
 *     P_m = prod_{s<m} alpha_s   (per key channel; products only, no division),
 * the closed form of j steps of the recurrence, in one read and one write of
 * each state (none when j = 0).  k, alpha and u are the arguments and output
 * of the kda_decode_verify call for the same drafts.
 *
 *   n_accept: [B] int32, DEVICE memory (read)
 *   S       : [B][H][d_k][d_v] fp32, updated in place
 *
 * S may overlap none of the inputs (KDA_ERR_ALIAS).
 */
kda_status kda_decode_commit(const void* k, kda_dtype qkv_dtype, const float* alpha, const float* u,
                             const int* n_accept, float* S,
                             int B, int K, int H, int d_k, int d_v, hipStream_t stream);

/* Human-readable text for a status code (static storage; never NULL). */
const char* kda_status_string(kda_status s);

/* The hipError_t of the last failed launch on the calling thread (0 if none). */
int kda_last_hip_error(void);

/* Library version, major * 10000 + minor * 100 + patch. */
int kda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H */
