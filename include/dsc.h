/*
 * dsc.h -- C ABI of the MI355X (gfx950) dynamic short causal convolution.
 *
 * The operation ([gist] = gist.science technical summary "Dynamische Korte
 * Convoluties Verbeteren Transformers", section Methodologie > Dynamische
 * Korte Convoluties):
 *
 *   s[b,t,c] = sum_{k=0}^{W-1} w[b,t,g(c),k] * x[b,t-k,c]     (bullet Mechanisme)
 *   y[b,t,c] = act(s[b,t,c]) + rho * x[b,t,c]                 (bullet Plaatsing:
 *                                                              X + conv(X))
 *
 * with g(c) = floor(c / H): one filter shared by H consecutive channels
 * (bullet Parametrisatie, 2. head-wise tying), G = D / H groups.  In the
 * low-rank form (Parametrisatie, 1.; section Efficiente
 * Trainingsimplementatie, bullet Fused Low-Rank Kernel) the filters are the
 * product w[b,t,g,k] = sum_r z[b,t,r] * U[r, g*W + k], generated on chip and
 * never written to device memory.  Taps before the start of a sequence read
 * zero; sequences b are independent.  rho is 1 with DSC_RESIDUAL, else 0;
 * act is SiLU, s * sigmoid(s), with DSC_ACT_SILU, else the identity.
 *
 * Layouts: every tensor is dense, row-major, in device memory:
 *   x, y, dy, dx : (B, T, D)         w, dw : (B, T, G, W)   (tap k = 0 is x_t)
 *   z, dz        : (B, T, R)         U, dU : (R, G*W)       (column g*W + k)
 * All tensors of one call share its dtype (DSC_F32 or DSC_BF16).  Arithmetic
 * is fp32; bf16 results are rounded to nearest even once, at the store.  In
 * the low-rank path the products z*U are formed from the bf16 (or fp32)
 * inputs and summed in fp32.
 *
 * Ownership and execution: the caller owns every buffer (workspace
 * included).  The library never allocates, frees or synchronises, keeps no
 * pointer after a call returns and holds no state between calls, apart from
 * the one library-owned buffer of dsc_lowrank_bwd_noalloc (below).  Work is
 * queued on `stream` (a hipStream_t; NULL is the legacy default stream) and
 * runs asynchronously; faults during execution surface at the caller's next
 * synchronisation, as usual in HIP.  Outputs are overwritten, never
 * accumulated into.  Results are bitwise reproducible for a given shape,
 * dtype and flags: no atomics, and every cross-tile sum runs in a fixed order.
 *
 * Argument checks run on the host before anything is queued.  A failing call
 * returns an error, queues nothing and changes nothing; dsc_last_error()
 * then names the failing check.  Errors:
 *   DSC_ERR_INVALID_ARG  a size < 0 or D < 1, D % H != 0, D not a multiple of
 *                        the vector width (8 for bf16, 4 for fp32), a NULL
 *                        pointer for a non-empty tensor, a pointer not 16-byte
 *                        aligned, an output overlapping another tensor of the
 *                        call, or more than 2^38 elements in x (far beyond
 *                        one GPU's memory; the bound keeps launch grids
 *                        below 2^31 workgroups);
 *   DSC_ERR_UNSUPPORTED  W outside 1..8, R outside 1..64, an unknown flag or
 *                        dtype, or a tying factor H the kernels do not tile
 *                        (head-wise: H divides the vector width, or H is the
 *                        vector width times 1 .. 64; low-rank:
 *                        H divides the vector width or is a multiple of it),
 *                        or, for the low-rank
 *                        backward, 16 * D * (bytes per element) >= 2^31;
 *   DSC_ERR_WORKSPACE    workspace smaller than dsc_lowrank_bwd_workspace_bytes
 *                        (dsc_static_bwd_workspace_bytes for dsc_static_bwd),
 *                        or NULL while that is non-zero;
 *   DSC_ERR_HIP          a HIP launch error (the message holds HIP's text).
 * B == 0 or T == 0 is legal and empty; the low-rank backward then still
 * writes dU = 0.
 */
#ifndef DSC_H_
#define DSC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dsc_status {
  DSC_OK = 0,
  DSC_ERR_INVALID_ARG = 1,
  DSC_ERR_UNSUPPORTED = 2,
  DSC_ERR_WORKSPACE = 3,
  DSC_ERR_HIP = 4
} dsc_status;

typedef enum dsc_dtype { DSC_F32 = 0, DSC_BF16 = 1 } dsc_dtype;

#define DSC_RESIDUAL 1u /* y = act(s) + x ; dx gains + dy */
#define DSC_ACT_SILU 2u /* act = SiLU on the convolution output */

/* Library version, major * 10000 + minor * 100 + patch. */
int dsc_version(void);

/* Static text of a status code. */
const char *dsc_status_string(dsc_status status);

/* Detail of the last failing call made on this thread ("" if none). */
const char *dsc_last_error(void);

/*
 * Head-wise forward: y from x (B,T,D) and per-token filters w (B,T,G,W).
 * Reads x and w once each and writes y once; the whole window sum happens on
 * chip ([gist] Efficiente Trainingsimplementatie, bullet On-chip Computatie).
 */
dsc_status dsc_headwise_fwd(const void *x, const void *w, void *y, int64_t B,
                            int64_t T, int64_t D, int W, int H, dsc_dtype dtype,
                            unsigned flags, void *stream);

/*
 * Head-wise backward: given dy = dL/dy, writes
 *   dx[b,tau,c] = sum_{k<W, tau+k<T} w[b,tau+k,g(c),k] * ds[b,tau+k,c] + rho*dy[b,tau,c]
 *   dw[b,t,g,k] = sum_{c : g(c)=g} ds[b,t,c] * x[b,t-k,c]     (0 when t-k < 0)
 * with ds = dy * act'(s) (s recomputed on chip when act is SiLU, else ds = dy).
 * The derivative of the forward above; the pages give the forward only.
 */
dsc_status dsc_headwise_bwd(const void *x, const void *w, const void *dy,
                            void *dx, void *dw, int64_t B, int64_t T, int64_t D,
                            int W, int H, dsc_dtype dtype, unsigned flags,
                            void *stream);

/*
 * Low-rank forward: y from x (B,T,D), z (B,T,R) and U (R, G*W).  Filters
 * w = zU are formed on chip per token tile and consumed at once; they never
 * reach device memory ([gist] bullet Fused Low-Rank Kernel).
 */
dsc_status dsc_lowrank_fwd(const void *x, const void *z, const void *U, void *y,
                           int64_t B, int64_t T, int64_t D, int W, int H, int R,
                           dsc_dtype dtype, unsigned flags, void *stream);

/* Bytes of device workspace dsc_lowrank_bwd needs for this shape (fp32 partial
 * sums of dz over channel blocks and of dU over token chunks).  Returns 0 for
 * arguments dsc_lowrank_bwd would reject. */
size_t dsc_lowrank_bwd_workspace_bytes(int64_t B, int64_t T, int64_t D, int W,
                                       int H, int R, dsc_dtype dtype);

/*
 * Low-rank backward: with w = zU and dw as in dsc_headwise_bwd (formed on chip
 * only), writes dx (B,T,D) and
 *   dz[b,t,r]    = sum_{g,k} dw[b,t,g,k] * U[r, g*W+k]
 *   dU[r, g*W+k] = sum_{b,t} z[b,t,r] * dw[b,t,g,k]
 * Partial sums go to `workspace` (at least dsc_lowrank_bwd_workspace_bytes);
 * a second kernel on the same stream adds them in a fixed order.  The
 * workspace content on entry is ignored and on exit is unspecified.
 */
dsc_status dsc_lowrank_bwd(const void *x, const void *z, const void *U,
                           const void *dy, void *dx, void *dz, void *dU,
                           void *workspace, size_t workspace_bytes, int64_t B,
                           int64_t T, int64_t D, int W, int H, int R,
                           dsc_dtype dtype, unsigned flags, void *stream);

/*
 * Low-rank backward for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Arguments, results, checks and errors are those of dsc_lowrank_bwd (plain
 * rows, no pos), with no workspace argument: the partial sums go to a
 * buffer the library owns, DSC_NOALLOC_SCRATCH_BYTES (128 MiB) of device
 * memory per GPU, held from the first use on that GPU until the process ends.
 * The call allocates nothing (no hipMalloc or allocating library routine).
 * A shape whose partial sums need more than that buffer
 * (dsc_lowrank_bwd_workspace_bytes above DSC_NOALLOC_SCRATCH_BYTES) returns
 * DSC_ERR_WORKSPACE and queues nothing.  The buffer's content on entry is
 * never read before it is written.  Every call on one GPU shares that GPU's
 * buffer: calls that overlap in time on one GPU (on different streams, or
 * from different host threads) race on it and give undefined results;
 * serialise them.  The device is the current one (hipGetDevice), which must
 * be the device of `stream`.
 */
#define DSC_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
dsc_status dsc_lowrank_bwd_noalloc(const void *x, const void *z, const void *U,
                                   const void *dy, void *dx, void *dz, void *dU, int64_t B,
                                   int64_t T, int64_t D, int W, int H, int R, dsc_dtype dtype,
                                   unsigned flags, void *stream);

/*
 * One-token (decode) steps.  The pages define the convolution over a whole
 * sequence only; in streaming use, y at the newest token t depends on x_t and
 * the W-1 inputs before it, which a caller keeps in a state buffer
 *   state : (B, W-1, D), row j = x_{t-(W-1)+j} (oldest first, zero before the
 *           start of the sequence; an empty buffer when W == 1).
 * Each call takes x_t : (B, D) and the filter of token t, writes
 *   y[b,c] = act(w[b,g(c),0] x_t[b,c] + sum_{k=1}^{W-1} w[b,g(c),k] state[b,W-1-k,c])
 *            + rho x_t[b,c]
 * -- row t of the forward above, in the same fp32 arithmetic up to the order
 * of the sums -- and then advances the state in place by one token
 * (rows move up by one, x_t becomes the last row; values are copied, not
 * rounded).  `state` is read and written by the call and must not overlap any
 * other tensor of it.  B == 0 is legal and empty.  Errors as above.
 */

/* Head-wise decode step; w : (B, G, W). */
dsc_status dsc_headwise_decode(const void *x, const void *w, void *state, void *y,
                               int64_t B, int64_t D, int W, int H, dsc_dtype dtype,
                               unsigned flags, void *stream);

/* Low-rank decode step; z : (B, R), U : (R, G*W); the filter w = zU is formed
 * in registers ([gist] bullet Fused Low-Rank Kernel). */
dsc_status dsc_lowrank_decode(const void *x, const void *z, const void *U, void *state,
                              void *y, int64_t B, int64_t D, int W, int H, int R,
                              dsc_dtype dtype, unsigned flags, void *stream);

/* State after a prompt x : (B, T, D): state[b,j] = x[b, T-(W-1)+j], zero where
 * that index is below 0.  Writes the (B, W-1, D) state only. */
dsc_status dsc_decode_state(const void *x, void *state, int64_t B, int64_t T, int64_t D,
                            int W, dsc_dtype dtype, void *stream);

/*
 * Static short convolution: the same causal sum with one filter per group
 * for every sequence and position,
 *   y[b,t,c] = act(sum_{k<W} w[g(c),k] * x[b,t-k,c]) + rho * x[b,t,c],
 * w : (G, W).  It is the fixed-filter form the pages contrast with the dynamic
 * one ([wisp] Methodology, 1. Mathematical Intuition) and the kind of kernel
 * they measure the dynamic kernels against ([gist] Efficiente
 * Trainingsimplementatie, bullet Prestaties).  Tying factors, flags, layouts
 * of x, y, dy, dx and errors are those of the head-wise calls.
 */
dsc_status dsc_static_fwd(const void *x, const void *w, void *y, int64_t B, int64_t T,
                          int64_t D, int W, int H, dsc_dtype dtype, unsigned flags,
                          void *stream);

/* Bytes of workspace dsc_static_bwd needs: fp32 partial sums of dw, one row
 * of G*W per sequence and 512-token span.  0 for an empty call or for
 * arguments dsc_static_bwd would reject. */
size_t dsc_static_bwd_workspace_bytes(int64_t B, int64_t T, int64_t D, int W, int H,
                                      dsc_dtype dtype);

/*
 * Static backward: dx (B,T,D) as in dsc_headwise_bwd with the fixed filter, and
 *   dw[g,k] = sum_b sum_{t>=k} sum_{c : g(c)=g} ds[b,t,c] * x[b,t-k,c]   (G, W)
 * summed over every sequence and token; partial sums go to `workspace` and a
 * second kernel on the same stream adds them in a fixed order.  An empty call
 * (B == 0 or T == 0) writes dw = 0.
 */
dsc_status dsc_static_bwd(const void *x, const void *w, const void *dy, void *dx, void *dw,
                          void *workspace, size_t workspace_bytes, int64_t B, int64_t T,
                          int64_t D, int W, int H, dsc_dtype dtype, unsigned flags,
                          void *stream);

/*
 * Rows packed with several documents.  pos (B, T), int32 in device memory,
 * 16-byte aligned, holds each token's index inside its document (0 at a
 * document start; entries must be >= 0).  Tap k >= 1 of token t is used only
 * when k <= pos[b,t], so no tap reaches into the previous document; every
 * other argument, layout and error is that of the call without _varlen, and
 * with pos[b,t] = t the results equal it.  The masked taps contribute nothing
 * to y and dx, and their dw (head-wise) or their share of dz and dU
 * (low-rank) is zero.  The pages train on whole rows and do not discuss
 * packing; this is a training-side layout.
 */
dsc_status dsc_headwise_fwd_varlen(const void *x, const void *w, const int32_t *pos, void *y,
                                   int64_t B, int64_t T, int64_t D, int W, int H,
                                   dsc_dtype dtype, unsigned flags, void *stream);

dsc_status dsc_headwise_bwd_varlen(const void *x, const void *w, const int32_t *pos,
                                   const void *dy, void *dx, void *dw, int64_t B, int64_t T,
                                   int64_t D, int W, int H, dsc_dtype dtype, unsigned flags,
                                   void *stream);

dsc_status dsc_lowrank_fwd_varlen(const void *x, const void *z, const void *U,
                                  const int32_t *pos, void *y, int64_t B, int64_t T, int64_t D,
                                  int W, int H, int R, dsc_dtype dtype, unsigned flags,
                                  void *stream);

/* Workspace as for dsc_lowrank_bwd (dsc_lowrank_bwd_workspace_bytes). */
dsc_status dsc_lowrank_bwd_varlen(const void *x, const void *z, const void *U,
                                  const int32_t *pos, const void *dy, void *dx, void *dz,
                                  void *dU, void *workspace, size_t workspace_bytes, int64_t B,
                                  int64_t T, int64_t D, int W, int H, int R, dsc_dtype dtype,
                                  unsigned flags, void *stream);

/*
 * Head-wise forward with the filters generated on chip from a hidden state
 * ([gist] Parametrisatie: the filter is a learned linear map of the hidden
 * state; [wisp] Limitations: merging the convolution into the preceding
 * matrix product):
 *   w[b,t,:] = xh[b,t,:] M,  xh (B, T, Dh), M (Dh, G*W) with column g*W + k,
 * then y exactly as dsc_headwise_fwd with that w, which never reaches device
 * memory.  M is passed transposed, as Mt (G*W, Dh) row-major: row g*W + k
 * holds column g*W + k of M (the weight layout of a linear layer from Dh to
 * G*W features), so that both operands are contiguous along Dh.  w is rounded to bf16 before use, as a stored w would be.  bf16 only;
 * W in {1, 2, 4, 8}; H a multiple of 8; Dh a multiple of 64; G*W a multiple
 * of 8 (else DSC_ERR_UNSUPPORTED).  Other checks and errors as for the
 * head-wise calls.  Forward only (inference).
 */
dsc_status dsc_headwise_gen_fwd(const void *x, const void *xh, const void *Mt, void *y,
                                int64_t B, int64_t T, int64_t D, int64_t Dh, int W, int H,
                                dsc_dtype dtype, unsigned flags, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DSC_H_ */
