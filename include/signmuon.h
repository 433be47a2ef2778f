/*
 * signmuon.h - C ABI of libsignmuon.so: the Sign-Muon optimizer step on
 * AMD Instinct MI355X (gfx950), written as HIP kernels.
 *
 * Method: "SignMuon: Communication-Efficient Distributed Muon Optimization"
 * (Mishra, Trivedi, Kumar; arXiv 2605.16311).  Algorithm 1 gives one
 * worker's step (weight decay, momentum EMA, PolarNS, entrywise sign,
 * update); Algorithm 2 and Figure 1 give the distributed step (each worker
 * sends its signs, an integer sum across workers is thresholded by sign,
 * every worker applies the same update).  The first author's blog ("SignMuon:
 * Matrix Directions, Majority Votes, and the Actual Bytes Sent") fixes the
 * tie policy (a tied vote gives 0) and the 1-bit payload of d/8 bytes.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every array pointer is a DEVICE pointer unless stated otherwise; the
 *   caller owns all memory.  The library allocates no device memory: scratch
 *   space is a caller workspace (the *_workspace queries give its size).
 *   The only host objects it creates are those of an executor
 *   (signmuon_executor_create), which the caller owns and destroys; besides
 *   that, the first call on a device sets the matrix-core kernels' LDS size
 *   attribute once.  Calls that use different workspaces (and executors)
 *   are independent and may run concurrently; calls that share a workspace
 *   must be ordered on one stream.
 * - Work is enqueued asynchronously on the caller's stream (NULL = the null
 *   stream) and never synchronises, except signmuon_get_status and
 *   signmuon_executor_destroy.  Without an executor, and while the caller's
 *   stream is being captured into a HIP graph, every kernel of a call is
 *   enqueued on the caller's stream and nothing else: such calls can be
 *   captured.
 * - Matrices are row-major and contiguous.  A parameter set is one flat
 *   array per quantity (G, W, Mom) holding every matrix back to back at
 *   sm_matrix.elem_off.
 * - Packed signs: flat index j of a matrix lives in bit (j % 32) of word
 *   j / 32 of that matrix's segment (little-endian uint32), and the bit is 1
 *   exactly when the value is negative (so 0 and -0 pack as the +1 bit).
 *   Tail bits past the last entry are written as 0 and ignored on input.
 * - Argument errors return SM_EINVAL (or SM_ERANGE / SM_EWORKSPACE) before
 *   anything is enqueued.  A failed launch returns SM_EHIP.  Faults inside
 *   kernels surface at the caller's next synchronisation.
 * - Floating-point work never uses atomics: results are deterministic and
 *   bit-reproducible run to run.
 */
#ifndef SIGNMUON_H
#define SIGNMUON_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sm_status {
  SM_OK = 0,
  SM_EINVAL = -1,        /* bad argument; nothing enqueued */
  SM_EWORKSPACE = -2,    /* workspace missing or too small; nothing enqueued */
  SM_EHIP = -3,          /* a HIP launch or runtime call failed */
  SM_ENONFINITE = -4,    /* a step saw a non-finite G, W or momentum */
  SM_ERANGE = -5,        /* worker count or size outside the supported range */
  SM_EUNSUPPORTED = -6   /* valid request this build does not implement */
} sm_status;

typedef enum sm_dtype { SM_F32 = 0, SM_BF16 = 1 } sm_dtype;

/* Arithmetic of the Newton-Schulz products.  BF16: bfloat16 operands with
 * float32 accumulation.  BF16X3: each operand split into hi + lo bfloat16
 * parts, products hi*hi + hi*lo + lo*hi (near-float32 accuracy at three
 * times the matrix-core work).  F32: float32 operands and accumulation. */
typedef enum sm_ns_precision {
  SM_NS_F32 = 0, SM_NS_BF16 = 1, SM_NS_BF16X3 = 2
} sm_ns_precision;

/* Pre-scale of PolarNS (paper, section 4): X0 = Mom / (s + eps) with
 * s = ||Mom||_F (FRO) or s = an estimate of sigma_max(Mom) from P steps of
 * power iteration on the smaller Gram matrix (SPECTRAL): u <- A u / |A u|,
 * s = sqrt(|A u|) at the last step. */
typedef enum sm_scale { SM_SCALE_FRO = 0, SM_SCALE_SPECTRAL = 1 } sm_scale;

/* Encoding of the worker sign buffers of signmuon_step and
 * signmuon_worker_pipeline.  PACKED: 1 bit per entry (the blog's d/8-byte
 * payload), bit = 1 for a negative value, so a zero travels as +1.
 * TERNARY: one int8 per entry in {-1, 0, +1} (section 3: sign(0) = 0;
 * Algorithm 2 and Figure 1 exchange int8 signs), so an exact zero adds
 * nothing to the vote. */
typedef enum sm_sign_encoding {
  SM_SIGNS_PACKED = 0, SM_SIGNS_TERNARY = 1
} sm_sign_encoding;

/* Hyper-parameters: the inputs of Algorithm 1 (eta, beta, lambda, K, eps,
 * scale, P) plus the Newton-Schulz coefficients, the product precision, the
 * tie policy and the sign encoding.  One Newton-Schulz step is X <- a X + (b A + c A^2) X with
 * A = X X^T for a wide matrix (rows <= cols), and X <- a X + X (b A + c A^2)
 * with A = X^T X for a tall one; the cubic of section 4 is (1.5, -0.5, 0). */
typedef struct sm_hparams {
  float eta;             /* step size of this call, any finite value */
  float beta;            /* momentum, 0 <= beta < 1 */
  float lambda;          /* weight decay, >= 0 */
  float eps;             /* pre-scale stability constant, > 0 */
  int32_t K;             /* Newton-Schulz steps, 0 <= K <= 64 */
  int32_t scale;         /* sm_scale */
  int32_t P;             /* power-iteration steps, 1..256 when SPECTRAL */
  float ns_a, ns_b, ns_c;
  int32_t ns_precision;  /* sm_ns_precision */
  int32_t tie_value;     /* value of a tied vote: 0 (default) or 1 */
  int32_t sign_encoding; /* sm_sign_encoding (steps only; else ignored) */
} sm_hparams;

/* One matrix of a parameter set. */
typedef struct sm_matrix {
  int64_t rows, cols;    /* both in [1, 2^20]; with rows and cols rounded up
                            to multiples of 128, rows*cols < 2^31 (2^30 when
                            hp->ns_precision is SM_NS_F32), else SM_EINVAL */
  int64_t elem_off;      /* element offset in the flat G / W / Mom arrays */
  int64_t word_off;      /* word offset of its packed signs in a worker buffer */
} sm_matrix;

/* Largest worker count: vote sums are kept in int16 (the blog notes that an
 * int8 accumulator overflows once more than 127 workers agree). */
#define SM_MAX_WORKERS 32767

const char *signmuon_strerror(int status);
int32_t signmuon_abi_version(void);

/*
 * Momentum (Algorithm 1 and 2, weight-decay and momentum lines):
 *   Mom[i] <- beta * Mom[i] + (1 - beta) * (G[i] + lambda * W[i]),
 * in float32, for i < n.  G, Mom: float32[n]; W: float32 or bfloat16[n]
 * (w_dtype).  Mom is updated in place; G and W are read only.  n = 0 is a
 * no-op.
 */
sm_status signmuon_momentum(const float *G, const void *W, int32_t w_dtype,
                            float *Mom, int64_t n, float beta, float lambda,
                            hipStream_t stream);

/*
 * PolarNS of one matrix (Algorithm 1 polar line; section 4): pre-scale by
 * hp->scale, then hp->K Newton-Schulz steps with (ns_a, ns_b, ns_c) in
 * hp->ns_precision.  X: float32[rows*cols] input, U: float32[rows*cols]
 * output (must not alias X).  u0: float32[min(rows, cols)] start vector of
 * the power iteration, or NULL for the all-ones vector; ignored for FRO.
 * ws: device workspace of at least signmuon_polar_ns_workspace() bytes,
 * 256-byte aligned; its contents on entry do not matter.  eta, beta, lambda
 * and tie_value are ignored.
 */
size_t signmuon_polar_ns_workspace(int64_t rows, int64_t cols,
                                   const sm_hparams *hp);
sm_status signmuon_polar_ns(const float *X, float *U, int64_t rows,
                            int64_t cols, const sm_hparams *hp,
                            const float *u0, void *ws, size_t ws_bytes,
                            hipStream_t stream);

/*
 * signmuon_polar_ns without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The same kernels run with their
 * scratch space in an array of SM_STATIC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends; it calls no
 * allocator.  A matrix whose signmuon_polar_ns_workspace() exceeds that size
 * returns SM_ERANGE (with bfloat16 products and the Frobenius scale, shapes
 * up to about 1024 x 4096 fit); other arguments and errors as for
 * signmuon_polar_ns.  Every such call on one GPU uses the same array:
 * calls that overlap in time on one GPU (two streams, two threads) race and
 * must be ordered by the caller.
 */
#define SM_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
sm_status signmuon_polar_ns_static(const float *X, float *U, int64_t rows,
                                   int64_t cols, const sm_hparams *hp,
                                   const float *u0, hipStream_t stream);

/*
 * Entrywise sign with 1-bit packing (section 3 sign; section 6 packing):
 * bits[j/32] bit (j%32) = (U[j] < 0) for j < n; ceil(n/32) words written,
 * tail bits 0.  U: float32[n].
 */
sm_status signmuon_sign_pack(const float *U, uint32_t *bits, int64_t n,
                             hipStream_t stream);

/*
 * Majority vote (Algorithm 2 sum all-reduce and local threshold; blog tie
 * rule): for j < n, sum_j = sum over m < M of (bit_{m,j} ? -1 : +1) and
 * D[j] = sign(sum_j), a zero sum giving tie_value.  Worker m's buffer starts
 * at bits + m * worker_stride_words (worker_stride_words >= ceil(n/32)).
 * D: int8[n] output; sums: int16[n] output or NULL.  1 <= M <= 32767 else
 * SM_ERANGE.
 */
sm_status signmuon_majority_vote(const uint32_t *bits,
                                 int64_t worker_stride_words, int32_t M,
                                 int64_t n, int32_t tie_value, int8_t *D,
                                 int16_t *sums, hipStream_t stream);

/*
 * Ternary sign buffers, the one-byte encoding that keeps sign(0) = 0
 * (section 3 of the paper defines sign(0) = 0; Algorithm 2, Figure 1 and
 * section 6 describe signs exchanged as int8).  For callers that exchange
 * int8 signs instead of the 1-bit packed buffers.
 *
 * signmuon_sign_ternary: S[j] = +1, -1 or 0 for U[j] > 0, < 0, or zero / NaN.
 *   U: float32[n], S: int8[n] (device).  0 <= n <= 2^36 else SM_EINVAL.
 * signmuon_majority_vote_ternary: sum_j = sum over m < M of S_m[j] (exact;
 *   |sum| <= M <= 32767), D[j] = sign(sum_j) with a zero sum giving
 *   tie_value (0 or 1).  Worker m's buffer starts at S + m * worker_stride
 *   bytes (worker_stride >= n when M > 1).  D: int8[n]; sums: int16[n] or
 *   NULL.  1 <= M <= 32767 else SM_ERANGE.  Buffer starts and a stride that
 *   are multiples of 16 bytes take the 16-byte access path.
 */
sm_status signmuon_sign_ternary(const float *U, int8_t *S, int64_t n,
                                hipStream_t stream);
sm_status signmuon_majority_vote_ternary(const int8_t *S, int64_t worker_stride,
                                         int32_t M, int64_t n, int32_t tie_value,
                                         int8_t *D, int16_t *sums,
                                         hipStream_t stream);

/*
 * Update (Algorithm 1 and 2, last line): W[i] <- W[i] - eta * D[i] with the
 * product and the difference each rounded to float32 (no fused
 * multiply-add) and, for a bfloat16 W, the result rounded to nearest even.
 * Exactly one of D (int8[n], values -1/0/+1) and Df (float32[n]) is
 * non-NULL.
 */
sm_status signmuon_apply(void *W, int32_t w_dtype, const int8_t *D,
                         const float *Df, float eta, int64_t n,
                         hipStream_t stream);

/*
 * Executor: caller-owned host resources that let signmuon_step,
 * signmuon_worker_pipeline and signmuon_step_profiled run the PolarNS work
 * of disjoint groups of matrices as up to three concurrent chains (three
 * non-blocking HIP streams on the device current at creation, forked from
 * and joined back into the caller's stream with the executor's own events;
 * each of the at most two PolarNS passes of a step has its own events; the
 * chain with the most matrices runs on the caller's stream itself).
 * Passing NULL instead runs everything on the caller's stream (a few percent
 * slower on large sets).  An executor may be passed only on its own device
 * (else SM_EINVAL) and by one thread at a time (calls lock it while they
 * enqueue).  signmuon_executor_destroy waits for the executor's streams,
 * then frees it; NULL is a no-op.
 */
typedef struct sm_executor sm_executor;
sm_status signmuon_executor_create(sm_executor **ex);
sm_status signmuon_executor_destroy(sm_executor *ex);

/*
 * One fused Sign-Muon step for the local worker over a parameter set, with
 * the M workers' packed sign buffers resident on this GPU (they stand for
 * this GPU's copy after an exchange of sign buffers).
 *
 * post_vote = 0 (Algorithm 2): for every matrix, momentum (in place in
 *   Mom), PolarNS of the new momentum, its signs packed into worker buffer
 *   local_worker; then the vote over all M buffers and
 *   W <- W - eta * majority.
 * post_vote = 1 (the variant with the polar step after the vote): the signs
 *   of the new momentum go to buffer local_worker; the majority matrix S of
 *   each matrix is voted, U = PolarNS(S), and W <- W - eta * U.
 * post_vote = 2 (both: the optional local polar step of the abstract on the
 *   sota2.com paper record, read as an extra PolarNS of the voted matrix on
 *   top of Algorithm 2): the local worker's pipeline of post_vote = 0, then
 *   the vote and update of post_vote = 1.  Both PolarNS passes use the same
 *   hyper-parameters and start vectors.
 * post_vote = 3 (the spectral-norm normalized sign step under which the
 *   abstract states its O(1/sqrt(T)) rate; section 4 normalizes D_t in the
 *   analysis and estimates spectral norms by power iteration, locally): the
 *   local worker's pipeline of post_vote = 0, then the majority matrix D of
 *   each matrix, s = an estimate of ||D||_2 from hp->P power-iteration steps
 *   on its smaller Gram matrix (start vectors u0, as for the spectral
 *   pre-scale), and W <- W - eta * D / (s + eps).  Needs 1 <= hp->P <= 256
 *   whatever hp->scale is.
 * Any other post_vote value is SM_EINVAL (the workspace query returns 0).
 *
 * mats[n_mats]: HOST array of matrix descriptors (1 <= n_mats <= 65536);
 * matrices must not overlap in the flat arrays or in a worker buffer.
 * G, Mom: float32 flat arrays; W: w_dtype flat array.  bits: M worker
 * buffers, worker m at bits + m * worker_stride_words.  With
 * hp->sign_encoding = SM_SIGNS_TERNARY, bits points to int8 buffers instead:
 * worker m at (int8_t *)bits + m * worker_stride_words (then a count of
 * bytes), matrix i's signs at its elem_off (word_off is ignored), and
 * elem_off + rows * cols <= worker_stride_words.  u0: float32, the
 * concatenation of every matrix's min(rows, cols) power-iteration start
 * vector, or NULL (all ones).  ws: workspace of signmuon_step_workspace()
 * bytes, 256-byte aligned.  Before its first call a step workspace must be
 * zero-filled or passed to signmuon_reset_status: its first 8 bytes carry
 * the non-finite flags from call to call (below); the rest is scratch
 * whose contents on entry do not matter.
 *
 * ex: an executor for the concurrent chains, or NULL (see above).
 *
 * If any G, W or new momentum value is non-finite the update of W is
 * skipped (Mom and the local buffer are still written) and the next
 * signmuon_get_status on the same workspace returns SM_ENONFINITE.  The
 * same holds for a non-finite value met by any signmuon_worker_pipeline
 * call on the same workspace enqueued since the previous step: a step
 * starts by taking over those flags, so the vote skips the update when any
 * worker's pipeline of the step saw a non-finite value.
 */
size_t signmuon_step_workspace(const sm_matrix *mats, int32_t n_mats,
                               const sm_hparams *hp, int32_t post_vote);
sm_status signmuon_step(const sm_matrix *mats, int32_t n_mats,
                        const sm_hparams *hp, const float *G, void *W,
                        int32_t w_dtype, float *Mom, uint32_t *bits,
                        int64_t worker_stride_words, int32_t M,
                        int32_t local_worker, int32_t post_vote,
                        const float *u0, void *ws, size_t ws_bytes,
                        sm_executor *ex, hipStream_t stream);

/*
 * The per-worker half of signmuon_step for worker `worker` (Algorithm 2's
 * local computation up to the packed signs, for every matrix of the set):
 * post_vote = 0 or 2: momentum (in place in Mom), PolarNS of the new
 * momentum and its signs packed into buffer `worker`; post_vote = 1:
 * momentum and the signs of the new momentum packed into buffer `worker`.  No vote, and W is
 * only read.  Arguments, validation and workspace as for signmuon_step (same
 * workspace size); a non-finite G, W or momentum value is recorded in the
 * workspace (it never clears a flag): signmuon_get_status reports it, and
 * the next signmuon_step on the workspace skips its update.  Calling it for
 * workers 1..M-1 and then signmuon_step for worker 0, with one workspace on
 * one stream, runs every worker's pipeline of one step on this GPU.
 */
sm_status signmuon_worker_pipeline(const sm_matrix *mats, int32_t n_mats,
                                   const sm_hparams *hp, const float *G,
                                   const void *W, int32_t w_dtype, float *Mom,
                                   uint32_t *bits, int64_t worker_stride_words,
                                   int32_t M, int32_t worker, int32_t post_vote,
                                   const float *u0, void *ws, size_t ws_bytes,
                                   sm_executor *ex, hipStream_t stream);

/*
 * Instrumented step: identical work to signmuon_step, plus a hipEventRecord
 * on `stream` after each phase so a caller can time the kernels of one step
 * (events[i] closes the phase kinds[i]; the first event opens the step).
 * Matrix-core launches outside the concurrent chains, the momentum pass
 * (sweep, or momentum + signs) and every vote launch take two events that
 * the kernel itself sets to its start and stop time (hipExtLaunchKernel):
 * the first closes an SM_PHASE_GAP interval, the second the kernel's own
 * duration (SM_PHASE_GRAM / SQUARE / UPDATE / MOMENTUM / VOTE).
 * events[capacity]: caller-created events (HOST array of handles);
 * kinds[capacity]: HOST array receiving the phase of each event
 * (SM_PHASE_*); *count receives the number of events recorded.  If the
 * capacity is too small, recording stops and *count == capacity.
 */
typedef enum sm_phase {
  SM_PHASE_START = 0,     /* opening event */
  SM_PHASE_MOMENTUM = 1,  /* momentum sweep (+ signs in the post-vote form) */
  SM_PHASE_PRESCALE = 2,  /* Frobenius finalize / power iteration */
  SM_PHASE_GEMM = 3,      /* the concurrent PolarNS chains (closed at their
                             join), or an elementwise Newton-Schulz launch */
  SM_PHASE_PACK = 4,      /* unfused sign packing */
  SM_PHASE_VOTE = 5,      /* vote (+ apply, or majority matrix) */
  /* single Newton-Schulz matrix-core launches (only recorded outside the
     concurrent chains: without an executor, or for sets run as one chain) */
  SM_PHASE_GRAM = 6,      /* Gram or raw Gram S S^T */
  SM_PHASE_SQUARE = 7,    /* symmetric Rp x Rp product (Gram-space steps,
                             quintic square) */
  SM_PHASE_UPDATE = 8,    /* update B S, or the final product Q_K S_0 */
  SM_PHASE_GAP = 9        /* the interval before a kernel with its own start
                             and stop events starts (launch gap; a split-k
                             reduction; before the momentum pass, the status
                             launch; before the post-vote vote, the padding
                             launch) */
} sm_phase;
typedef struct sm_profile {
  hipEvent_t *events;
  int32_t *kinds;
  int32_t capacity;
  int32_t count;
} sm_profile;
sm_status signmuon_step_profiled(const sm_matrix *mats, int32_t n_mats,
                                 const sm_hparams *hp, const float *G, void *W,
                                 int32_t w_dtype, float *Mom, uint32_t *bits,
                                 int64_t worker_stride_words, int32_t M,
                                 int32_t local_worker, int32_t post_vote,
                                 const float *u0, void *ws, size_t ws_bytes,
                                 sm_profile *prof, sm_executor *ex,
                                 hipStream_t stream);

/*
 * Status of workspace ws: waits for the stream, then returns SM_ENONFINITE
 * if the last signmuon_step on ws, or a signmuon_worker_pipeline call on ws
 * enqueued after it, saw a non-finite value; else SM_OK.  SM_EHIP if the
 * copy fails, or if the one-launch power iteration of a spectral scale
 * (sets whose raw Grams have at most 4096 rows in all, none wider than
 * 768) found its blocks not all resident within its bounded wait (then the
 * step's update is skipped, as for a non-finite value).  Reading the status
 * clears nothing.
 */
sm_status signmuon_get_status(const void *ws, hipStream_t stream);

/*
 * Clears the non-finite flags of step workspace ws (enqueued on the stream,
 * a kernel, so it can be captured): for a new workspace that is not
 * zero-filled, or to drop the flags of worker pipelines whose step is
 * abandoned.
 */
sm_status signmuon_reset_status(void *ws, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* SIGNMUON_H */
