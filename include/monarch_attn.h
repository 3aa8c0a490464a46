/*
 * monarch_attn.h -- C ABI of MonarchAttention for AMD MI355X (gfx950): the
 * forward (square layer, or a chunk of frames against cached keys; fixed
 * iteration count or early stop) and its gradient.
 *
 * The operation (MonarchRT pages):
 *   Video self-attention over N = f*h*w tokens is approximated by a Monarch
 *   matrix M = P^T L P R: P is the fixed reshape-transpose permutation of the
 *   token index, L and R are block-diagonal factors (yunpan.plus MonarchRT
 *   article, section "Monarch matrices: a unified structured approximation
 *   tool").  The factors are computed from Q and K by alternating block
 *   softmax steps (MonarchAttention; same section, Fig. 3), with blocks
 *   aligned to the video as (b1, b2) = (f*h, w) ("Innovation 1: block
 *   alignment"), optionally split into independently factorised tiles along
 *   the f*h axis ("Innovation 2: tiled Monarch parameterisation"), for a given
 *   number of iterations ("Innovation 3: finetuning and efficient kernels").
 *   The output is Y = M V, computed without forming the N x N matrix.
 *
 * Exact definition used (readings of points the pages leave open):
 *   token n = a1*b2 + a2, key m = c1*b2 + c2, s = 1/sqrt(d);
 *   tile g of a1: [floor(g*b1/t), floor((g+1)*b1/t));
 *   R starts uniform; one iteration = L-step then R-step:
 *     L-step: L[a2][a1,:] = softmax_c1( s<q_n, Kt[g,c1,a2]> + H(R[g,c1,a2,:]) ),
 *             Kt[g,c1,a2] = sum_c2 R[g,c1,a2,c2] k_(c1,c2);
 *     R-step: R[g,c1,a2,:] = softmax_c2( s<Qh[g,c1,a2], k_(c1,c2)> ),
 *             Qh[g,c1,a2] = sum_(a1 in g) L[a2][a1,c1] q_(a1,a2) / sum_(a1 in g) L[a2][a1,c1]
 *             (Qh = 0 when that sum is 0);
 *   y_(a1,a2) = sum_c1 L[a2][a1,c1] sum_c2 R[g(a1),c1,a2,c2] v_(c1,c2).
 *
 * Layout: q, k, v, out are [B, H, N, d] contiguous, token order
 *   n = (fi*h + hi)*w + wi (column fastest).  bf16 entry points take raw bf16
 *   storage (2 bytes per element); f32 entry points take float.  All pointers
 *   are DEVICE pointers owned by the caller; the library never frees or keeps
 *   them past the call.  Everything is enqueued on `stream` (a hipStream_t;
 *   NULL = the null stream) and the call returns without synchronising: the
 *   caller keeps the buffers alive until the stream has run the work.
 *
 * Graph capture: the entry points that take a caller's workspace or state
 *   (monarch_attn_fwd_ws, monarch_attn_fwd_kv_ws, monarch_attn_fwd_adaptive_ws
 *   and its _kv form, monarch_attn_fwd_train and its _kv form) allocate
 *   nothing, record no memset and never synchronise, so a caller may capture
 *   them in a HIP graph and replay it (with per-kernel timing off: timing
 *   records HIP events around each launch).  The entry points without a workspace
 *   argument, and the backward, allocate their scratch memory stream-ordered
 *   (hipMallocAsync / hipFreeAsync on `stream`).
 *
 * Errors: every entry point returns a monarch_status.  Arguments are checked
 *   before any GPU call; on MONARCH_EINVAL / MONARCH_EUNSUPPORTED nothing is
 *   launched and `out` is untouched.  MONARCH_EHIP reports a HIP runtime
 *   failure; monarch_attn_last_hip_error() gives its code.  The library never
 *   prints or aborts.  NaN/Inf in the inputs propagate to the output.
 *
 * Supported envelope: d in {16, 32, 64, 128}; 1 <= b2 <= 16384; any b1 >= 1;
 *   b1*b2 == f*h*w; 1 <= tiles <= b1; iters >= 1; tiles*N*d < 2^31.
 *   Key blocks longer than 128 tokens, e.g. whole frames, (b1, b2) =
 *   (f, h*w) (the spatio-temporal factorisation of the VMonarch abstract,
 *   listed on the same pages), run an R-step that takes the block softmax
 *   online, forward and backward.
 */
#ifndef MONARCH_ATTN_H
#define MONARCH_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MONARCH_OK = 0,
    MONARCH_EINVAL = -1,        /* bad argument (NULL, aliasing, dims, blocks, tiles, iters) */
    MONARCH_EUNSUPPORTED = -2,  /* valid but outside the kernels' envelope (d, b2, sizes) */
    MONARCH_EHIP = -3,          /* a HIP runtime call failed */
    MONARCH_ENOMEM = -4,        /* workspace allocation failed or workspace too small */
} monarch_status;

typedef enum {
    MONARCH_BF16 = 0,           /* bf16 I/O; bf16 MFMA with fp32 accumulation and softmax */
    MONARCH_F32 = 1,            /* fp32 I/O and fp32 arithmetic throughout */
} monarch_dtype;

/* Y = M V for bf16 q, k, v, out ([B,H,N,d], N = f*h*w).  (b1, b2) are the
 * Monarch block sizes (b1*b2 == N; the aligned choice is (f*h, w)), `tiles`
 * the number of tiles per aligned block along the f*h axis, `iters` the
 * number of (L-step, R-step) iterations.  Allocates its workspace
 * stream-ordered (hipMallocAsync/hipFreeAsync on `stream`). */
int monarch_attn_fwd(const void* q, const void* k, const void* v, void* out,
                     int B, int H, int f, int h, int w, int d,
                     int b1, int b2, int tiles, int iters, void* stream);

/* Same operation with float I/O and float arithmetic. */
int monarch_attn_fwd_f32(const float* q, const float* k, const float* v, float* out,
                         int B, int H, int f, int h, int w, int d,
                         int b1, int b2, int tiles, int iters, void* stream);

/* Bytes of device workspace monarch_attn_fwd_ws needs for these arguments
 * (0 if the arguments are invalid or unsupported). */
size_t monarch_attn_workspace_bytes(int B, int H, int f, int h, int w, int d,
                                    int b1, int b2, int tiles, int iters, int dtype);

/* Same operation for either dtype with a caller-provided device workspace of
 * at least monarch_attn_workspace_bytes(...) bytes (256-byte aligned).  The
 * workspace must not overlap q, k, v or out; its contents on entry are
 * ignored and on return are unspecified.  Returns MONARCH_ENOMEM when
 * workspace_bytes is too small. */
int monarch_attn_fwd_ws(const void* q, const void* k, const void* v, void* out,
                        int B, int H, int f, int h, int w, int d,
                        int b1, int b2, int tiles, int iters, int dtype,
                        void* workspace, size_t workspace_bytes, void* stream);

/* ---- a forward that allocates nothing ----
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * operation and arguments as monarch_attn_fwd_ws without the workspace:
 * the intermediates live in one static device array of the library,
 * MONARCH_SCRATCH_BYTES (128 MiB) per GPU, allocated with the library's code
 * on that GPU and held until the process ends.  A call whose workspace
 * (monarch_attn_workspace_bytes) exceeds it returns MONARCH_ENOMEM and
 * launches nothing: it covers, e.g., the 3-frame 480p chunk (12 heads,
 * 15 MB) and the 21-frame 480p clip (12 heads, 101 MB), not the 40-head
 * 720p latent.  The first call on a device looks up the array's device
 * address (hipGetSymbolAddress) with that device current.  Every call on one
 * GPU uses the same array: calls that overlap on one GPU (two host threads,
 * or two streams whose work runs concurrently) race and give undefined
 * results; calls on one stream are ordered and safe.  Nothing in the array
 * needs clearing between calls (every intermediate is written before it is
 * read). */
#define MONARCH_SCRATCH_BYTES ((size_t)128 << 20)
int monarch_attn_fwd_scratch(const void* q, const void* k, const void* v, void* out,
                             int B, int H, int f, int h, int w, int d,
                             int b1, int b2, int tiles, int iters, int dtype, void* stream);

/* ---- iterating until the factors converge ----
 * Without finetuning the pages run about ten iterations (yunpan.plus
 * MonarchRT article, "Innovation 3: finetuning and efficient kernels",
 * Fig. 4 right) and give no stopping rule.  monarch_attn_fwd_adaptive_ws runs
 * up to max_iters iterations and stops each (batch, head) on its own: after
 * the L-step of iteration i the objective of the current factors is
 * F_i = sum_n log-sum-exp of that L-step's logits (nats; the L-step is the
 * exact maximiser), and the head stops after iteration i when i == max_iters
 * or when i >= 2 and (F_i - F_(i-1)) / N <= tol (gain per token).  Its last
 * R-step then gives U = R V and the apply uses that iteration's L and R: the
 * output equals monarch_attn_fwd_ws with iters = iters_used[head].
 * iters_used is a DEVICE array of B*H ints written on `stream` (the count of
 * iterations each head ran, 1..max_iters).  The workspace
 * (monarch_attn_adaptive_workspace_bytes) holds every head at once.  tol NaN or
 * iters_used NULL: MONARCH_EINVAL; otherwise errors as monarch_attn_fwd_ws. */
size_t monarch_attn_adaptive_workspace_bytes(int B, int H, int f, int h, int w, int d,
                                             int b1, int b2, int tiles, int max_iters, int dtype);
int monarch_attn_fwd_adaptive_ws(const void* q, const void* k, const void* v, void* out,
                                 int B, int H, int f, int h, int w, int d,
                                 int b1, int b2, int tiles, int max_iters, float tol, int dtype,
                                 int* iters_used, void* workspace, size_t workspace_bytes,
                                 void* stream);
/* The same for a chunk of fq frames against all f frames (see
 * monarch_attn_fwd_kv below): the objective sums the chunk's Nq = fq*h*w
 * query rows and the gain is taken per query token. */
size_t monarch_attn_adaptive_kv_workspace_bytes(int B, int H, int fq, int f, int h, int w, int d,
                                                int b1, int b2, int tiles, int max_iters, int dtype);
int monarch_attn_fwd_adaptive_kv_ws(const void* q, const void* k, const void* v, void* out,
                                    int B, int H, int fq, int f, int h, int w, int d,
                                    int b1, int b2, int tiles, int max_iters, float tol, int dtype,
                                    int* iters_used, void* workspace, size_t workspace_bytes,
                                    void* stream);

/* ---- chunked queries against cached keys ----
 * Autoregressive video generation produces a chunk of frames at a time; the
 * chunk's queries attend to the cached keys and values of earlier frames plus
 * the chunk's own (yunpan.plus MonarchRT article, on autoregressive,
 * frame-by-frame real-time generation).  Here q and out are [B, H, Nq, d]
 * with Nq = fq*h*w (the chunk: fq frames), k and v are [B, H, N, d] with
 * N = f*h*w (all f frames the chunk attends to, its own included).  (b1, b2)
 * block the keys (b1*b2 == N); the queries form b1q = Nq/b2 blocks of the same
 * b2 (Nq must be a multiple of b2).  The definition is the one above with the
 * query block index a1 in [b1q] and the key block index c1 in [b1]; tiles
 * split the query blocks (1 <= tiles <= b1q).  With fq == f this is exactly
 * monarch_attn_fwd_ws; a chunk of the last fq frames gives the rows of the
 * full layer over all frames whose tiles cover the chunk with the same bounds.
 * Errors and workspace rules as for monarch_attn_fwd_ws (out must not overlap
 * q, k or v). */
size_t monarch_attn_kv_workspace_bytes(int B, int H, int fq, int f, int h, int w, int d,
                                       int b1, int b2, int tiles, int iters, int dtype);
int monarch_attn_fwd_kv(const void* q, const void* k, const void* v, void* out,
                        int B, int H, int fq, int f, int h, int w, int d,
                        int b1, int b2, int tiles, int iters, int dtype, void* stream);
int monarch_attn_fwd_kv_ws(const void* q, const void* k, const void* v, void* out,
                           int B, int H, int fq, int f, int h, int w, int d,
                           int b1, int b2, int tiles, int iters, int dtype,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ---- training: the forward that keeps its factors, and its gradient ----
 * The pages' deployed regime is one iteration after finetuning the video
 * model with this attention in place (yunpan.plus MonarchRT article,
 * "Innovation 3: finetuning and efficient kernels", Fig. 4 right), which
 * needs the gradient of the layer; several iterations (iters >= 1, the
 * same refinement as monarch_attn_fwd) are differentiated too.
 *
 * monarch_attn_fwd_train computes the same out as monarch_attn_fwd_ws and
 * also leaves in `state` (a caller-owned device buffer of at least
 * monarch_attn_train_state_bytes(...) bytes, 256-byte aligned, not
 * overlapping q, k, v or out) what the backward pass reads: the block-mean
 * keys; per iteration the L-row log-sum-exps, the column masses beta and the
 * aggregated queries Qh of every tile; U = R V of the last R-step; and for
 * every R-step but the last the keys R k and entropies H(R) it hands to the
 * next L-step; with b2 > 128 also every R-step's row log-sum-exps.  Its
 * size is, with e = element bytes and T = iters,
 *   B*H*(b1*d*e + 4*b1 + T*(4*N + 4*t*N + t*N*d*e) + t*N*d*e
 *        + (T-1)*(t*N*d*e + 4*t*N) + [b2 > 128] T*4*t*N)  (+ alignment).
 *
 * monarch_attn_bwd takes the same q, k, v, the out and state of a
 * monarch_attn_fwd_train call with the same arguments, and dout = dLoss/dout,
 * and writes dq, dk, dv = dLoss/dq, dLoss/dk, dLoss/dv ([B,H,N,d], same
 * dtype).  Definition: the chain rule through every step of the forward as
 * monarch_attn_fwd computes it: with R starting uniform the first L-step's
 * keys are the block means Kbar[c1] = mean_c2 k_(c1,c2); each L-step
 * L = softmax(s q Kt^T + H) with the keys Kt = R k and entropies H of the
 * R-step before; Qh = sum L q / beta (0 where beta == 0);
 * R = softmax(s Qh k^T); U = R V of the last R-step and y = L U on the
 * permuted index.
 * dq, dk, dv must not overlap each other or any input (state included).
 * It allocates a workspace stream-ordered (about 2*t*N*d*e + 16*t*N +
 * N*roundup(b1, 256)*e bytes per head, plus 4*t*N + 8*N*d for T > 1).  The
 * supported envelope is the forward's.  State from another shape, iteration
 * count or dtype gives undefined results. */
size_t monarch_attn_train_state_bytes(int B, int H, int f, int h, int w, int d,
                                      int b1, int b2, int tiles, int iters, int dtype);
int monarch_attn_fwd_train(const void* q, const void* k, const void* v, void* out,
                           int B, int H, int f, int h, int w, int d,
                           int b1, int b2, int tiles, int iters, int dtype,
                           void* state, size_t state_bytes, void* stream);
int monarch_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                     const void* dout, void* dq, void* dk, void* dv,
                     int B, int H, int f, int h, int w, int d,
                     int b1, int b2, int tiles, int iters, int dtype,
                     void* state, size_t state_bytes, void* stream);

/* ---- training for a chunk of frames against cached keys ----
 * The training forward and backward of monarch_attn_fwd_kv: fq query frames
 * (q, out, dout, dq: [B,H,fq*h*w,d]) against all f key frames (k, v, dk, dv:
 * [B,H,f*h*w,d]), same definitions as monarch_attn_fwd_train /
 * monarch_attn_bwd with a1 over the chunk's fq*h*w/b2 query blocks (tiles
 * split those) and c1 over the b1 key blocks.  The gradient of a chunk is
 * the one of the square layer over all frames, with tiles that cover the
 * chunk with the same bounds, restricted to dy = 0 outside the chunk.  State
 * size as for the square layer with 4*Nq instead of 4*N per iteration for
 * the log-sum-exps; the backward's workspace has Nq rows on its query side.
 * fq == f is the square layer (same results as the calls above). */
size_t monarch_attn_train_state_bytes_kv(int B, int H, int fq, int f, int h, int w, int d,
                                         int b1, int b2, int tiles, int iters, int dtype);
int monarch_attn_fwd_train_kv(const void* q, const void* k, const void* v, void* out,
                              int B, int H, int fq, int f, int h, int w, int d,
                              int b1, int b2, int tiles, int iters, int dtype,
                              void* state, size_t state_bytes, void* stream);
int monarch_attn_bwd_kv(const void* q, const void* k, const void* v, const void* out,
                        const void* dout, void* dq, void* dk, void* dv,
                        int B, int H, int fq, int f, int h, int w, int d,
                        int b1, int b2, int tiles, int iters, int dtype,
                        void* state, size_t state_bytes, void* stream);

/* ---- the factors themselves (test-only export) ----
 * monarch_attn_debug_factors_f32 runs the fp32 forward of monarch_attn_fwd_f32
 * (square layer) and writes the factors of its last iteration, the L and R
 * that the output y = P^T L P R v applies (MonarchRT article, "Monarch
 * matrices"), as fp32 device arrays the caller owns:
 *   L_out [B,H,b2,b1,b1]:   L[a2][a1][c1], each row a1 sums to 1 over c1;
 *   R_out [B,H,t,b1,b2,b2]: R[g][c1][a2][c2], each row sums to 1 over c2.
 * For parity tests of the factors on small shapes: the counts B*H*b2*b1*b1
 * and B*H*t*N*b2 must each be at most 2^28 (else MONARCH_EUNSUPPORTED); the
 * outputs must not overlap the inputs or each other (MONARCH_EINVAL).  It
 * allocates a temporary training state stream-ordered and is not tuned. */
int monarch_attn_debug_factors_f32(const float* q, const float* k, const float* v, float* L_out, float* R_out,
                                   int B, int H, int f, int h, int w, int d,
                                   int b1, int b2, int tiles, int iters, void* stream);

/* Static text for a status code (never NULL). */
const char* monarch_attn_status_string(int status);

/* hipError_t of the last MONARCH_EHIP on the calling thread (0 if none). */
int monarch_attn_last_hip_error(void);

/* ---- per-kernel timing (benchmarking aid; not thread-safe) ----
 * While enabled, each kernel launch is bracketed by HIP events recorded on
 * the launch stream.  monarch_attn_profile_collect waits for those events,
 * adds each kernel's elapsed milliseconds and launch count into ms[i] and
 * launches[i] for kernel id i < n, and forgets them.  Kernel ids:
 * 0 block-mean keys, 1 L-row log-sum-exp, 2 R-side aggregation through L,
 * 3 R-step block softmax (+ R V or next keys/entropy), 4 L-apply;
 * backward: 5 dU per tile column, 6 R-step per key block (G, statistics),
 * 7 row pass (dq), 8 block-mean key gradient (product over tokens),
 * 9 its reduction, 10 dv and dk per key block; 11 objective and early-stop
 * decision per head; 12 (backward, several iterations) gradient of the
 * aggregated keys and entropies per tile column.  Each id covers every form
 * of its step that the library picks by shape (key blocks over 128 tokens,
 * tile columns of at most 32 rows and keys). */
#define MONARCH_NUM_KERNELS 13
int monarch_attn_profile_enable(int on);
int monarch_attn_profile_collect(double* ms, long* launches, int n);
const char* monarch_attn_kernel_name(int id);

#ifdef __cplusplus
}
#endif

#endif /* MONARCH_ATTN_H */
