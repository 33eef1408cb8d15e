/*
 * dpg.h -- C ABI of the deterministic BF16 projection GEMM library for AMD
 * MI355X (gfx950).
 *
 * The operations are the dense projection GEMM family and the FP32 router GEMM
 * described on the pages
 *   "plan the 4096 -> 12288 input gradient with the row-half-release program
 *    at T-exact keys" (description: BF16-operand forward, input gradient and
 *    weight gradient; FP32 accumulation; BF16 or FP32 output),
 *   "restore the K1 weight-gradient routes that meet the deterministic
 *    package's absolute FP64 budgets" (description: the weight gradient reduces
 *    over the token count T in 64-token K blocks, with one or two K splits), and
 *   "cache the router entry points' calls by their own tensors" (description:
 *    an FP32 router GEMM with 256 experts computed by BF16x3 emulation, and
 *    deterministic=True as the default).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every matrix is row-major with a leading dimension `ld*` counted in
 *   elements (ld >= number of columns).  All data pointers are DEVICE pointers
 *   owned by the caller; the library keeps no pointer after a call returns.
 * - `T` is the token count, `N` the output features, `K` the input features
 *   (the pages write a projection as "K -> N", e.g. 4096 -> 12288).
 * - Alignment: every base pointer is 16-byte aligned, every `ld * sizeof(elt)`
 *   is a multiple of 16 bytes, and the contiguous extent of every matrix
 *   (its number of columns) is a multiple of 8 elements.  Otherwise the call
 *   returns DPG_ERR_ALIGNMENT.  T (the row count of X, dY, Y and dX) may be any
 *   value >= 0, including odd counts of 64-token blocks.
 * - Row strides of 2^22 elements or more are supported; such calls run a
 *   slower kernel with 64-bit addressing (the pipelined kernels address a tile
 *   through 32-bit buffer offsets).
 * - Outputs are written only in [rows, cols]; elements of a padded row beyond
 *   `cols` are never touched.  Outputs are overwritten, never read.
 * - An empty output (a zero extent) is a no-op.  An empty reduction (K = 0 for
 *   the forward pass, N = 0 for the input gradient, T = 0 for the weight
 *   gradient) writes zeros.
 * - `deterministic` != 0 (the default of the Python binding) selects the
 *   deterministic plan: the K partition and the in-tile accumulation order are
 *   a fixed function of (pass, T, N, K, output dtype, split_k) alone -- never of
 *   the device, its CU count or the cache state -- so the bits are reproducible
 *   on any MI355X.  deterministic == 0 selects the split-K plan, which may also
 *   use the device's CU count to pick the K split.  `split_k` = 0 lets the
 *   planner choose; 1..64 forces min(split_k, B) K splits in either mode, B
 *   being the number of 64-element blocks of the reduction (K for the forward
 *   pass, N for the input gradient, 64-token blocks of T for the weight
 *   gradient).  S splits partition the blocks evenly: with q = B / S and
 *   r = B % S the first r splits take q + 1 blocks and the others q (split s
 *   starts at block s*q + min(s, r); for S = 2: [0, ceil(B/2)) and the rest).
 *   In BOTH
 *   modes every reduction runs in a fixed order with no atomics, so repeated
 *   calls with the same arguments on one device give bitwise-identical
 *   outputs; different plans may differ from each other in the last bits.
 * - Split partials go to the caller's `workspace`, which must hold at least
 *   dpg_workspace_size(...) bytes for the same shape and flags (it may be NULL
 *   when that size is 0).  The library never allocates and never synchronizes;
 *   all work is enqueued on `stream` (0 = the null stream), so calls may be
 *   captured into a HIP graph.
 * - All validation happens before the first launch: on any error nothing is
 *   launched and nothing is written.  DPG_ERR_HIP reports a failed launch.
 */
#ifndef DPG_H_
#define DPG_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DPG_OK = 0,
  DPG_ERR_INVALID_ARG = 1, /* negative size, ld < cols, NULL pointer for non-empty data, bad enum */
  DPG_ERR_UNSUPPORTED = 2, /* split_k outside 0..64, or a launch beyond the grid limit */
  DPG_ERR_ALIGNMENT = 3,   /* pointer / ld / contiguous extent not 16-byte compatible */
  DPG_ERR_WORKSPACE = 4,   /* workspace smaller than dpg_workspace_size() */
  DPG_ERR_HIP = 5          /* a kernel launch failed */
} dpg_status;

typedef enum { DPG_BF16 = 0, DPG_F32 = 1 } dpg_dtype;

/* Passes; the short names (DPG_FWD ...) are aliases of the long ones. */
typedef enum {
  DPG_PASS_FORWARD = 0,
  DPG_PASS_DGRAD = 1,
  DPG_PASS_WGRAD = 2,
  DPG_PASS_ROUTER_FORWARD = 3,
  DPG_PASS_ROUTER_DGRAD = 4,
  DPG_PASS_ROUTER_WGRAD = 5,
  DPG_FWD = DPG_PASS_FORWARD,
  DPG_DGRAD = DPG_PASS_DGRAD,
  DPG_WGRAD = DPG_PASS_WGRAD,
  DPG_ROUTER_FWD = DPG_PASS_ROUTER_FORWARD,
  DPG_ROUTER_DGRAD = DPG_PASS_ROUTER_DGRAD,
  DPG_ROUTER_WGRAD = DPG_PASS_ROUTER_WGRAD
} dpg_pass;

/*
 * Forward pass, Y[T,N] = X[T,K] . W[N,K]^T: both operands K-major (the
 * row-half-release page, description, names this the K-major-B form).
 *   x  : BF16 [T, K], row stride ldx     w : BF16 [N, K], row stride ldw
 *   y  : y_dtype (BF16 or FP32) [T, N], row stride ldy
 * FP32 accumulation; BF16 output is rounded to nearest even.
 */
dpg_status dpg_forward(const void* x, int64_t ldx, const void* w, int64_t ldw,
                       void* y, int64_t ldy, dpg_dtype y_dtype,
                       int64_t T, int64_t N, int64_t K, int deterministic, int split_k,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Input gradient, dX[T,K] = dY[T,N] . W[N,K]: the reduction runs over N, so W
 * is read with its contiguous dimension along the output (the MN-major B form
 * that the row-half-release page adds, description and commit message).
 *   dy : BF16 [T, N], row stride lddy    w : BF16 [N, K], row stride ldw
 *   dx : dx_dtype [T, K], row stride lddx
 */
dpg_status dpg_dgrad(const void* dy, int64_t lddy, const void* w, int64_t ldw,
                     void* dx, int64_t lddx, dpg_dtype dx_dtype,
                     int64_t T, int64_t N, int64_t K, int deterministic, int split_k,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Weight gradient, dW[N,K] = dY[T,N]^T . X[T,K], reducing over the token count
 * T in 64-token blocks (the K1 weight-gradient page, description; an odd number
 * of 64-token blocks is allowed).  With two K splits, split 0 takes blocks
 * [0, ceil(B/2)) and split 1 the rest, B = ceil(T/64); partials are added in
 * ascending split order.
 *   dy : BF16 [T, N], row stride lddy    x : BF16 [T, K], row stride ldx
 *   dw : dw_dtype [N, K], row stride lddw
 */
dpg_status dpg_wgrad(const void* dy, int64_t lddy, const void* x, int64_t ldx,
                     void* dw, int64_t lddw, dpg_dtype dw_dtype,
                     int64_t T, int64_t N, int64_t K, int deterministic, int split_k,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Arithmetic of the router passes, a process-wide setting read when a router
 * call is planned (it is part of the plan key).  The router page's ratio table
 * shows plain FP32 library calls beating the BF16x3 emulation at small token
 * counts, and the wgrad page's timeline keeps a router FFMA window; this
 * library has both:
 *   DPG_ROUTER_AUTO   : the planner picks, per shape, BF16x3 on the matrix
 *                       cores or FP32 fused multiply-adds on the vector ALUs
 *                       (the latter only where it measured faster);
 *   DPG_ROUTER_BF16X3 : always BF16x3 (hi*hi + hi*lo + lo*hi per product);
 *   DPG_ROUTER_FP32   : always one FP32 fused multiply-add per product, in
 *                       ascending order of the reduction index within a split.
 * Both kinds meet the FP32 budget; they differ from each other in the last
 * bits.  Each is deterministic in the sense of the conventions above.
 * DPG_ERR_INVALID_ARG for another value.  Thread-safe; calls already planned
 * under the previous setting keep their plans only in the cache entries keyed
 * by that setting.
 */
typedef enum { DPG_ROUTER_AUTO = 0, DPG_ROUTER_BF16X3 = 1, DPG_ROUTER_FP32 = 2 } dpg_router_arith;
dpg_status dpg_set_router_arithmetic(dpg_router_arith arith);
dpg_router_arith dpg_get_router_arithmetic(void);

/*
 * Weight gradient that allocates nothing, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving or training
 * loops, harnesses that forbid hipMalloc).  Same arguments, plan and output
 * bits as dpg_wgrad, minus the workspace: the FP32 split partials go to a
 * static device array of the library, DPG_NOALLOC_SCRATCH_BYTES (64 MiB) per
 * GPU, held from the library's first use on that GPU until the process ends.
 * The partial planes are overwritten in full before they are read, so nothing
 * is cleared between calls.  Every call on one GPU shares that GPU's array:
 * calls that may overlap on one GPU (different streams, or different host
 * threads without ordering) race and must not be issued.  A plan whose
 * partials need more than DPG_NOALLOC_SCRATCH_BYTES (dpg_workspace_size above
 * it) returns DPG_ERR_WORKSPACE before any launch; DPG_ERR_HIP if the array's
 * device address cannot be obtained.  Calls no hipMalloc, hipFree or other
 * allocating routine.
 */
#define DPG_NOALLOC_SCRATCH_BYTES (64u << 20)
dpg_status dpg_wgrad_noalloc(const void* dy, int64_t lddy, const void* x, int64_t ldx,
                             void* dw, int64_t lddw, dpg_dtype dw_dtype,
                             int64_t T, int64_t N, int64_t K, int deterministic, int split_k,
                             hipStream_t stream);
/* DPG_NOALLOC_SCRATCH_BYTES as the library was built with it. */
size_t dpg_noalloc_scratch_bytes(void);

/*
 * FP32 router GEMM, E experts (256 on the router page), hidden size H, all
 * operands and outputs FP32 (router page, description and the legend under its
 * ratio table: token-by-hidden activations times a 256-by-hidden weight).  Every product a*b is
 * computed by BF16x3 emulation: hi = bf16_rne(a), lo = bf16_rne(a - hi), and
 * lo_a*hi_b + hi_a*lo_b + hi_a*hi_b accumulate (in that order) in FP32 on the
 * BF16 matrix cores -- or, where dpg_set_router_arithmetic allows it and the
 * plan takes it, by FP32 fused multiply-adds (see below).
 *   forward: y[T,E]  = x[T,H] . w[E,H]^T
 *   dgrad  : dx[T,H] = dy[T,E] . w[E,H]
 *   wgrad  : dw[E,H] = dy[T,E]^T . x[T,H]
 */
dpg_status dpg_router_forward(const float* x, int64_t ldx, const float* w, int64_t ldw,
                              float* y, int64_t ldy, int64_t T, int64_t E, int64_t H,
                              int deterministic, int split_k,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);
dpg_status dpg_router_dgrad(const float* dy, int64_t lddy, const float* w, int64_t ldw,
                            float* dx, int64_t lddx, int64_t T, int64_t E, int64_t H,
                            int deterministic, int split_k,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);
dpg_status dpg_router_wgrad(const float* dy, int64_t lddy, const float* x, int64_t ldx,
                            float* dw, int64_t lddw, int64_t T, int64_t E, int64_t H,
                            int deterministic, int split_k,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Batched projection GEMMs: `batch` independent problems of one shape in one
 * launch, as the page "[Cake 9/13] dense_gemm: batched projection and FP32
 * router GEMMs" (description) describes for the per-head projections: one
 * batched BF16 GEMM over strided views, forward and both gradients, with a
 * choice of weight layout.
 *   Problem b reads x + b * stride_x (and likewise for every operand; strides in
 *   elements) and writes its output at y + b * stride_y.  An input stride may be
 *   0 (the same matrix for every problem); when batch > 1 the outputs must not
 *   overlap: stacked (stride >= (rows - 1) * ld + cols) or interleaved within
 *   rows (stride >= cols and (batch - 1) * stride + cols <= ld, e.g. per-head
 *   views of a token-major buffer), else DPG_ERR_INVALID_ARG.  Every non-zero stride times the element size is a
 *   multiple of 16 bytes (DPG_ERR_ALIGNMENT).
 *   w_layout DPG_WEIGHT_NK: the weight is W[N, K] as in the single entry points;
 *   DPG_WEIGHT_KN: the weight is stored W[K, N] (row stride ldw >= N), i.e. the
 *   forward is Y = X . W.  For the weight gradient w_layout is the layout of the
 *   output: dW[N, K] = dY^T X, or dW[K, N] = X^T dY (row stride lddw >= N).
 *   Everything else (dtypes, alignment, deterministic, split_k, workspace from
 *   dpg_workspace_size_batched, errors) is as for the single entry points; each
 *   problem's result equals what the single entry point computes for it under
 *   the plan the batched call uses.  batch = 0 is a no-op.
 */
typedef enum { DPG_WEIGHT_NK = 0, DPG_WEIGHT_KN = 1 } dpg_weight_layout;

dpg_status dpg_forward_batched(const void* x, int64_t ldx, int64_t stride_x,
                               const void* w, int64_t ldw, int64_t stride_w, dpg_weight_layout w_layout,
                               void* y, int64_t ldy, int64_t stride_y, dpg_dtype y_dtype,
                               int64_t batch, int64_t T, int64_t N, int64_t K, int deterministic, int split_k,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

dpg_status dpg_dgrad_batched(const void* dy, int64_t lddy, int64_t stride_dy,
                             const void* w, int64_t ldw, int64_t stride_w, dpg_weight_layout w_layout,
                             void* dx, int64_t lddx, int64_t stride_dx, dpg_dtype dx_dtype,
                             int64_t batch, int64_t T, int64_t N, int64_t K, int deterministic, int split_k,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

dpg_status dpg_wgrad_batched(const void* dy, int64_t lddy, int64_t stride_dy,
                             const void* x, int64_t ldx, int64_t stride_x,
                             void* dw, int64_t lddw, int64_t stride_dw, dpg_weight_layout w_layout,
                             dpg_dtype dw_dtype, int64_t batch, int64_t T, int64_t N, int64_t K,
                             int deterministic, int split_k,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes of a batched call (projection passes 0..2 only; (size_t)-1
 * for arguments the call would reject). */
size_t dpg_workspace_size_batched(dpg_pass pass, dpg_weight_layout w_layout, int64_t batch, int64_t T,
                                  int64_t N, int64_t K, dpg_dtype out_dtype, int deterministic, int split_k);

/* Host-only plan description of a batched call (as dpg_plan_describe). */
dpg_status dpg_plan_describe_batched(dpg_pass pass, dpg_weight_layout w_layout, int64_t batch, int64_t T,
                                     int64_t N, int64_t K, dpg_dtype out_dtype, int deterministic, int split_k,
                                     char* buf, size_t buflen);

/*
 * Bytes of workspace the call with these arguments needs (0 when the plan has a
 * single K split): the FP32 partial products of the splits, S planes of the
 * output's rows x columns, which a second kernel adds in ascending split order
 * (the router page's commit message sums the split partials positionally over
 * the split dimension; the K1 weight-gradient page's description names one and
 * two K splits).  For router passes N = E, K = H and out_dtype must be DPG_F32.
 * Returns (size_t)-1 for arguments the matching call would reject.  The size
 * does not depend on the row strides.
 */
size_t dpg_workspace_size(dpg_pass pass, int64_t T, int64_t N, int64_t K, dpg_dtype out_dtype,
                          int deterministic, int split_k);

/*
 * Host-only description of the plan the library would use (kernel variant,
 * tile, raster group, K splits and their K-block partition, workspace) as one
 * line of text in `buf` (truncated to buflen - 1 characters, NUL-terminated):
 * the plan a key maps to, as the row-half-release page's description keys its
 * programs by exact token count and the router page's commit message keys
 * entries by shape, split count and alignment.  Split-K mode is described for
 * 256 CUs.  Row strides of 2^22 elements or more run the same K partition on
 * the generic kernel, which this text does not show.  Makes no HIP call;
 * usable without a GPU.  DPG_ERR_INVALID_ARG for a NULL or empty buffer or
 * arguments no plan covers.
 */
dpg_status dpg_plan_describe(dpg_pass pass, int64_t T, int64_t N, int64_t K, dpg_dtype out_dtype,
                             int deterministic, int split_k, char* buf, size_t buflen);

/*
 * The plan cache (router page, commit message and review: calls are cached by
 * their own arguments, never by data pointers, and the cache is refreshed when
 * the route changes).  It is process-global and mutex-protected, holds at most
 * dpg_plan_cache_capacity() plans (least recently used out first), and its
 * keys carry a generation number.  dpg_clear_plan_cache drops every plan and
 * bumps the generation; it never fails.  dpg_plan_cache_stats writes the
 * number of cached plans and the generation through the non-NULL pointers.
 */
void dpg_clear_plan_cache(void);
void dpg_plan_cache_stats(int64_t* entries, int64_t* generation);
int64_t dpg_plan_cache_capacity(void);

/* Static text for a status code ("unknown status" for other values); the
 * error classes follow the validation rules above. */
const char* dpg_status_string(dpg_status status);

/* Library version string (static text naming the target, gfx950). */
const char* dpg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DPG_H_ */
