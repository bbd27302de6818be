/*
 * matopt.h - C ABI of libmatopt.so: the owner-local Muon step and the Sign-Muon
 * tail on one AMD Instinct MI355X (gfx950), in hand-written HIP kernels.
 *
 * Sources (web pages, cited by title and section):
 *   "Riassunto Tecnico: MatrixFSDP" (gist.science, paper 2607.05895),
 *     "Metodologia: MatrixFSDP", item 1 (owner-shaped placement): one owner rank
 *     holds each 2D weight matrix whole and, after the gradient reduction, runs the
 *     Newton-Schulz update on it locally with no matrix communication.  The list of
 *     whole matrices one owner holds is the batch these calls take.
 *   "Riepilogo Tecnico: SignMuon" (gist.science, paper 2605.16311), section 2:
 *     momentum -> Newton-Schulz polar direction -> elementwise sign -> 1-bit
 *     packing -> integer-sum majority vote with a sign threshold.
 *
 * Readings where the pages are silent (stated once here, used throughout):
 *   momentum      M <- beta*M + G (heavy-ball, one fp32 buffer), one fused
 *                 multiply-add per element;
 *   scaling       X0 = M / (||M||_F + eps), per matrix;
 *   iteration     X <- a X + (b A + c A^2) X with A = X X^T, applied `iters` times
 *                 on the orientation with rows <= cols (a tall matrix is processed
 *                 as its transpose and the result is returned in the caller's
 *                 orientation);
 *   sign          bit = (u >= 0): +0 and -0 give +1, NaN gives -1;
 *   bit layout    flat row-major element i -> word i/32, bit i%32 (LSB first),
 *                 1 means +1, unused bits of the last word are 0;
 *   vote          sum_i = 2*count_i - M, out bit = (sum_i >= 0): ties give +1.
 *
 * Conventions for every call:
 *   - All buffer pointers are DEVICE pointers on the current HIP device, owned by
 *     the caller.  The library allocates no device memory and no pinned host
 *     memory on these calls; scratch comes from the caller's `workspace` (size
 *     from muon_workspace_bytes), whose head receives the per-call descriptor
 *     table through the kernel arguments of small copy kernels.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream), so that
 *     callers need no HIP header; the Newton-Schulz parameters are passed by
 *     pointer (read before return).  Work is enqueued and the
 *     call returns without waiting for the GPU.  `mats` is read before return.
 *     With profiling on (mo_profile_begin), calls also create and record HIP
 *     events.
 *   - Return value 0 (MO_OK) or a negative MO_ERR_* code.  Argument errors are
 *     found on the host before anything is launched; mo_last_error() then returns
 *     a message (thread-local).  Faults inside kernels surface at the caller's
 *     next synchronisation.
 *   - Calls that share a workspace must be ordered on one stream.
 *   - muon_step_batched, muon_step_apply and ns_orthogonalize may run half of
 *     their Newton-Schulz products on a second stream of the library's own (one
 *     per device, created on first use with the default priority and kept for the
 *     life of the process): they do so when a product's launch holds fewer than
 *     64 rounds of 256x256 tiles per CU, not while `stream` is being captured
 *     into a graph, and never in muon_step_batched_noalloc.  That stream waits
 *     for everything enqueued on `stream` before the call, and `stream` waits for
 *     it before anything enqueued after the call, so the ordering seen from
 *     `stream` is the same as with one stream.  Results do not depend on it: each
 *     matrix is computed by the same kernels tile by tile either way.
 */
#ifndef MATOPT_H
#define MATOPT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MATOPT_VERSION 112

/* element types */
enum { MO_F32 = 0, MO_BF16 = 1 };

/* return codes */
enum {
  MO_OK = 0,
  MO_ERR_INVALID = -1,     /* bad shape, null pointer, bad scalar, bad count       */
  MO_ERR_UNSUPPORTED = -2, /* dtype combination not provided                       */
  MO_ERR_WORKSPACE = -3,   /* workspace pointer null or smaller than required      */
  MO_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed           */
};

/* Newton-Schulz parameters: the quintic coefficients, the step count (>= 0; 0
 * returns the Frobenius-scaled input) and the epsilon of the scaling. */
typedef struct {
  float a, b, c;
  int32_t iters;
  float eps;
} mo_ns_params;

/* One owned matrix: rows x cols, row-major, contiguous (leading dimension = cols).
 * rows, cols >= 1.  Unused pointers may be NULL. */
typedef struct {
  int64_t rows, cols;
  const void *grad;  /* muon_step_batched: gradient, rows*cols of grad_dtype        */
  float *momentum;   /* muon_step_batched: fp32 momentum, updated in place          */
  const void *x;     /* ns_orthogonalize: input, rows*cols of in_dtype              */
  void *out;         /* both: the orthogonalised U, rows*cols of out_dtype          */
} mo_matrix;

/* Bytes of device workspace muon_step_batched / ns_orthogonalize need for this
 * list with this compute dtype (MO_F32 or MO_BF16): the scratch of the owner's local
 * update of every whole matrix it holds ("Riassunto Tecnico: MatrixFSDP",
 * Metodologia item 1).  Returns 0 if the list is invalid (then mo_last_error() says
 * why).  The workspace holds, per matrix, two
 * copies of the iterate X (ping-pong), A and B, each padded to multiples of 256 in
 * both dimensions, plus the per-call descriptor table and the per-matrix norm
 * partial sums. */
size_t muon_workspace_bytes(const mo_matrix *mats, int32_t count, int32_t compute_dtype);

/* The owner-local Muon step on `count` matrices, batched ("Riassunto Tecnico:
 * MatrixFSDP", Metodologia item 1: the owner of a whole matrix runs the
 * Newton-Schulz update locally; "Riepilogo Tecnico: SignMuon", section 2, core
 * mechanism item 1 and distributed flow item 1: the local momentum update, then its
 * Newton-Schulz polar direction; section 4, nanoGPT: Frobenius scaling).  For each
 * matrix
 *   M <- beta*M + G            (fp32, in place)
 *   X <- M / (||M||_F + eps)   (oriented so that rows <= cols)
 *   repeat ns->iters times: A = X X^T; B = b A + c A A; X <- a X + B X
 *   out <- X                   (caller's orientation, out_dtype)
 * grad_dtype: MO_F32 or MO_BF16.  compute_dtype: MO_F32 (fp32 operands) or MO_BF16
 * (bf16 operands X, A, B with fp32 accumulation; A is rounded to bf16 once, and the
 * polynomial matrix a*I + b*A + c*A^2 is formed from that same rounded A and rounded
 * to bf16 once, so that each step is the single product X <- (a*I + b*A + c*A^2) X).
 * The scale s = 1 / (||M||_F + eps) enters through the first iteration's products
 * (s^2 on X X^T, s on the update), with the first X being M itself in the compute
 * dtype: the same in exact arithmetic, one HBM pass fewer.  Where ||M||_F lies
 * outside [2^-20, 2^40], X is scaled before the first product instead, so fp32
 * accumulation never overflows or underflows.
 * out_dtype: MO_F32 or MO_BF16.
 * out must not overlap grad or momentum.  Deterministic: identical inputs give
 * bit-identical outputs, and a matrix's result does not depend on the rest of
 * the batch. */
int32_t muon_step_batched(const mo_matrix *mats, int32_t count, int32_t grad_dtype,
                          int32_t compute_dtype, int32_t out_dtype, float beta,
                          const mo_ns_params *ns, void *workspace, size_t workspace_bytes,
                          void *stream);

/* Scratch held by each GPU for muon_step_batched_noalloc: 256 MiB, enough for one
 * 4096 x 11008 matrix in bf16 (about 236 MiB) or for sets of smaller ones. */
#define MO_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)

/* For callers that cannot allocate (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same step as muon_step_batched,
 * with the same arguments and bit-identical results, but without a caller
 * workspace.  Its scratch is a file-scope device array of MO_NOALLOC_SCRATCH_BYTES
 * that every GPU the library runs on holds until the process ends; the call
 * allocates nothing (no hipMalloc, no pinned staging: the descriptor table goes up
 * through kernel arguments) and records no profiling events.  A list whose
 * muon_workspace_bytes exceeds MO_NOALLOC_SCRATCH_BYTES is rejected with
 * MO_ERR_WORKSPACE before anything is launched.  Every call on one GPU shares that
 * GPU's scratch: calls that overlap on one GPU (two streams, two threads) race and
 * must be ordered by the caller; the scratch keeps the last call's contents, and
 * nothing in it needs to start at zero. */
int32_t muon_step_batched_noalloc(const mo_matrix *mats, int32_t count, int32_t grad_dtype,
                                  int32_t compute_dtype, int32_t out_dtype, float beta,
                                  const mo_ns_params *ns, void *stream);

/* Frobenius scaling and Newton-Schulz only (no momentum): out <- NS(x / (||x|| + eps))
 * ("Riepilogo Tecnico: SignMuon", section 2, core mechanism item 1: the polar
 * direction of a worker's momentum; Flusso Algoritmico item 5: the optional polar
 * step on the voted signs).  in_dtype: MO_F32 or MO_BF16.  x == out is allowed.
 * Same arguments, conventions and workspace as muon_step_batched otherwise. */
int32_t ns_orthogonalize(const mo_matrix *mats, int32_t count, int32_t in_dtype,
                         int32_t compute_dtype, int32_t out_dtype, const mo_ns_params *ns,
                         void *workspace, size_t workspace_bytes, void *stream);

/* Elementwise sign and 1-bit packing ("Riepilogo Tecnico: SignMuon", section 2,
 * core mechanism item 2 and distributed flow items 2-3; "Efficienza di
 * Comunicazione": one bit per element).  u: numel values of dtype (MO_F32 or
 * MO_BF16) in flat order; packed: ceil(numel/32) uint32 words (written whole,
 * pad bits 0).  numel >= 1. */
int32_t sign_pack(const void *u, int32_t dtype, int64_t numel, uint32_t *packed, void *stream);

/* sign_pack for M workers in one launch ("Riepilogo Tecnico: SignMuon", section 2,
 * core mechanism item 2 and distributed flow items 2-3: every worker packs the signs
 * of its own direction).  Worker w's numel values (dtype MO_F32 or MO_BF16) start at
 * element w * u_stride of u (u_stride >= numel when M > 1; ignored when M == 1); its
 * ceil(numel/32) words go to packed + w * ceil(numel/32), so packed receives the
 * [M][ceil(numel/32)] stack sign_vote reads.  Same bits as M calls of sign_pack.
 * 1 <= M <= 65535, numel >= 1. */
int32_t sign_pack_batched(const void *u, int32_t dtype, int32_t M, int64_t numel, int64_t u_stride,
                          uint32_t *packed, void *stream);

/* Majority vote over M packed sign buffers ("Riepilogo Tecnico: SignMuon",
 * section 2, core mechanism item 3 and distributed flow item 4: integer sum of the
 * signs, then a sign threshold).  packed: [M][ceil(numel/32)] uint32, worker-major
 * (the layout an all-gather of packed buffers produces).  out_packed:
 * ceil(numel/32) words, bit = (sum >= 0), pad bits 0.  out_sum: NULL, or numel
 * int8 values sum_i = 2*count_i - M (needs M <= 127).  1 <= M <= 65535. */
int32_t sign_vote(const uint32_t *packed, int32_t M, int64_t numel, uint32_t *out_packed,
                  int8_t *out_sum, void *stream);

/* The step with the weight update fused in: the same computation as
 * muon_step_batched, but the last Newton-Schulz product (or, for iters == 0, the
 * scaled copy) updates the caller's weight in place instead of writing U:
 *   W <- W - lr * U
 * formed in fp32 from the unrounded U and stored in weight_dtype (MO_F32 or
 * MO_BF16).  mats[i].out is W, rows*cols of weight_dtype, read and written; it must
 * not overlap grad or momentum.  lr is finite (any sign).  The update form follows
 * "Riepilogo Tecnico: SignMuon", Flusso Algoritmico item 4 (W - eta * direction),
 * with the raw polar factor U as the direction: the pages give Muon no other
 * scaling.  ("Riassunto Tecnico: MatrixFSDP", Metodologia item 1: the owner runs
 * the update locally.) */
int32_t muon_step_apply(const mo_matrix *mats, int32_t count, int32_t grad_dtype, int32_t compute_dtype,
                        int32_t weight_dtype, float beta, const mo_ns_params *ns, float lr, void *workspace,
                        size_t workspace_bytes, void *stream);

/* Inverse of sign_pack, for the optional local polar step on the voted signs
 * ("Riepilogo Tecnico: SignMuon", Flusso Algoritmico item 5): out[i] = +1 where bit
 * i of packed is set, -1 elsewhere; then ns_orthogonalize(out).  packed:
 * ceil(numel/32) words; out: numel values of dtype (MO_F32 or MO_BF16).  numel >= 1. */
int32_t sign_unpack(const uint32_t *packed, int64_t numel, int32_t dtype, void *out, void *stream);

/* The Sign-Muon parameter update ("Riepilogo Tecnico: SignMuon", Flusso
 * Algoritmico item 4): W <- W - lr * S, S[i] = +1 where bit i of packed (the voted
 * signs) is set, -1 elsewhere.  The difference is formed in fp32 and stored in
 * dtype (MO_F32 or MO_BF16).  weight: numel values, updated in place; lr finite. */
int32_t sign_apply(const uint32_t *packed, int64_t numel, int32_t dtype, void *weight, float lr,
                   void *stream);

/* Owner planner, host only ("Riassunto Tecnico: MatrixFSDP", Metodologia, the
 * MatrixShard metadata and global planner item: owners are chosen to balance
 * resident bytes and optimizer work).  Work of matrix i is its algorithmic
 * Newton-Schulz flops, iters * (3 m^2 n + m^3) with m = min(rows, cols),
 * n = max(rows, cols); its bytes are rows*cols*bytes_per_element.  Matrices are
 * taken in decreasing order of work (ties: more bytes first, then lower index) and
 * each goes to the rank with the least work so far (ties: fewest bytes, then
 * lowest rank).  owner: count entries in [0, ranks).  rank_work, rank_bytes:
 * NULL or ranks entries each, the per-rank totals.  count >= 0, ranks >= 1, iters
 * >= 0, bytes_per_element finite and >= 0. */
int32_t mo_plan_owners(const int64_t *rows, const int64_t *cols, int32_t count, int32_t ranks, int32_t iters,
                       double bytes_per_element, int32_t *owner, double *rank_work, double *rank_bytes);

/* Message for the last non-zero return on this thread ("" if none). */
const char *mo_last_error(void);

/* MATOPT_VERSION of the built library. */
int32_t mo_version(void);

/* Per-kernel timing for measurement.  mo_profile_begin() makes the calls above
 * record a HIP event pair around every kernel they launch (on the stream it runs
 * on: the call's, or the library's second stream for half of a split product, whose
 * records then overlap in time with the other half's);
 * mo_profile_end() waits for those events and fills up to `max` records, one per
 * kernel kind, returning how many kinds were seen (or a negative code).
 * Profiling state is process-wide and guarded by a lock, so calls from several
 * threads may interleave; the records then mix every thread's launches. */
typedef struct {
  char name[32];     /* kernel kind, e.g. "ns_syrk"                               */
  int64_t launches;  /* launches recorded                                          */
  double total_ms;   /* sum of event-measured durations                            */
  double busy_ms;    /* time with at least one launch of this kind running: the
                        union of their event intervals on one timeline (equal to
                        total_ms when they never overlap; when the records span
                        more than one device, total_ms)                          */
} mo_kernel_time;

int32_t mo_profile_begin(void);
int32_t mo_profile_end(mo_kernel_time *out, int32_t max);

#ifdef __cplusplus
}
#endif

#endif /* MATOPT_H */
