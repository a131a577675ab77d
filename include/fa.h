/*
 * fa.h -- C ABI of the tiled BF16 attention library for AMD Instinct MI355X
 * (gfx950): FlashAttention forward and backward, with the repeated-maximum
 * stabilised softmax shift as a runtime switch.
 *
 * What is computed.  For every (b, h) head, with S = scale * Q K^T:
 *
 *   O   = softmax(S) V,   LSE_i = ln sum_j exp(S_ij)            (forward)
 *   dQ, dK, dV = gradients of sum(O * dO) from the saved LSE       (backward)
 *
 * FlashAttention is exact attention computed tile by tile in on-chip memory
 * (page 3, "Flash Attention: from academic breakthrough to industry
 * standard"); rows are processed with an online safe softmax whose running
 * maximum m and running sum l are FP32, whose unnormalised probabilities are
 * cast to BF16 before the product with V, and whose output is normalised by l
 * at the end (page 2, "Mechanism 2: where the bias comes from"; page 3, "What
 * did Meta's study find": every block is rescaled and updated on its own).
 *
 * The stabilised variant (page 2, same section): when the running maximum of
 * a row of S has been attained more than once, the softmax shift is moved so
 * that the exponent at the maximum is strictly below 1.  With R = m*scale*
 * log2(e) (base-2 units) the shift becomes R + delta, delta = max(|R|, 1/16)
 * for |R| <= 64 (that is 2R for R > 0 and 0 for R < 0), and |R| folded down by
 * whole multiples of 32 into (32, 64] above that; the constants are reported
 * by fa_stabilize_params().  Rows whose maximum never repeats are computed
 * bit-identically with the switch on and off.  The backward recomputes the
 * probabilities from LSE, on which the shift has no influence, so
 * `stabilize` is accepted by fa_bwd for symmetry and ignored.
 *
 * Conventions shared by every entry point
 *   - Q, K, V, O, dO, dQ, dK, dV: bf16 (or IEEE binary16 through the _ex
 *     entry points), shape (B, H, N, d), contiguous row-major (d fastest),
 *     device pointers, 16-byte aligned.
 *   - LSE (and the workspace's D vector): fp32, shape (B, H, N), natural log
 *     of the scaled scores.
 *   - d must be 64 or 128; N >= 1; B, H >= 1; B*H*N*d < 2^40.
 *   - causal != 0: query i attends to keys 0..i (top-left aligned).
 *   - scale: finite and > 0 (callers pass 1/sqrt(d)).
 *   - stream: a hipStream_t, or NULL for the null stream.  All work is
 *     enqueued asynchronously on it; the call returns after the launches.
 *   - Memory is owned by the caller.  The library allocates nothing and keeps
 *     no state between calls; calls are thread-safe.
 *   - Arguments are validated before any launch; on an error return nothing
 *     has been enqueued and no output has been written.  Non-finite input
 *     values are not checked; they propagate to the rows they touch.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1,   /* NULL pointer, bad size, misalignment, bad scale */
  FA_ERR_UNSUPPORTED = -2,   /* head dimension other than 64 / 128 */
  FA_ERR_WORKSPACE = -3,     /* workspace NULL or smaller than fa_bwd_workspace_bytes() */
  FA_ERR_LAUNCH = -4,        /* the HIP runtime rejected a kernel launch */
  FA_ERR_DEVICE = -5         /* no gfx950 device current, or a device query failed */
} fa_status;

/* Forward pass.
 *   in : Q, K, V      bf16 (B,H,N,d)
 *   out: O            bf16 (B,H,N,d)
 *        LSE          fp32 (B,H,N), required (the backward needs it)
 *   stabilize != 0 turns on the repeated-maximum shift.
 * One kernel launch. */
int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
           int B, int H, int N, int d, int causal, float scale, int stabilize,
           void* stream);

/* Forward pass that also reports, per row, whether the stabilised shift was
 * applied at any key block: row_shifted is uint8 (B,H,N), 1 if the running
 * maximum was attained at least twice at some block (only possible with
 * stabilize != 0), else 0.  Otherwise identical to fa_fwd (same kernels, same
 * results).  Used to check that rows the shift never touched are bitwise
 * unchanged by it. */
int fa_fwd_diag(const void* Q, const void* K, const void* V, void* O, float* LSE,
                unsigned char* row_shifted,
                int B, int H, int N, int d, int causal, float scale, int stabilize,
                void* stream);

/* Bytes of device workspace fa_bwd needs: the fp32 vector D = rowsum(dO*O)
 * of shape (B,H,N), rounded up to 256 bytes.  Returns 0 for invalid sizes. */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int d, int causal);

/* Backward pass (dQ, dK, dV of L = sum(O * dO)), recomputing the
 * probabilities from LSE.
 *   in : Q, K, V, O, dO   bf16 (B,H,N,d); O is the forward's bf16 output
 *        LSE              fp32 (B,H,N) from fa_fwd
 *        workspace        device memory of at least fa_bwd_workspace_bytes()
 *   out: dQ, dK, dV       bf16 (B,H,N,d)
 * Runs fa_bwd_dot, then fa_bwd_grads, on `stream` (two launches).
 * Deterministic: no atomics. */
int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
           const float* LSE, void* dQ, void* dK, void* dV,
           void* workspace, size_t workspace_bytes,
           int B, int H, int N, int d, int causal, float scale, int stabilize,
           void* stream);

/* The steps of fa_bwd, exposed so that each can be timed on its own.
 *   fa_bwd_dot  : Dvec[b,h,i] = sum_t dO[b,h,i,t] * O[b,h,i,t]   (fp32 out)
 *   fa_bwd_dkdv : dK, dV for every key, from Q, K, V, dO, LSE, Dvec
 *   fa_bwd_dq   : dQ for every query, from Q, K, V, dO, LSE, Dvec
 *   fa_bwd_grads: dQ, dK and dV in one launch: the workgroups of the two
 *                 kernels above, interleaved per head (what fa_bwd runs)
 * Dvec is fp32 (B,H,N) device memory owned by the caller.  The results of
 * fa_bwd_grads are bitwise those of fa_bwd_dkdv and fa_bwd_dq. */
int fa_bwd_dot(const void* O, const void* dO, float* Dvec,
               int B, int H, int N, int d, void* stream);
int fa_bwd_dkdv(const void* Q, const void* K, const void* V, const void* dO,
                const float* LSE, const float* Dvec, void* dK, void* dV,
                int B, int H, int N, int d, int causal, float scale, void* stream);
int fa_bwd_dq(const void* Q, const void* K, const void* V, const void* dO,
              const float* LSE, const float* Dvec, void* dQ,
              int B, int H, int N, int d, int causal, float scale, void* stream);
int fa_bwd_grads(const void* Q, const void* K, const void* V, const void* dO,
                 const float* LSE, const float* Dvec, void* dQ, void* dK, void* dV,
                 int B, int H, int N, int d, int causal, float scale, void* stream);

/* Element type of the 16-bit tensors. */
typedef enum {
  FA_BF16 = 0,  /* bfloat16: what fa_fwd / fa_bwd take */
  FA_F16 = 1    /* IEEE binary16 */
} fa_dtype;

/* Forward pass with the element type chosen by `dtype` (page 1, sections
 * 1.2 and 6.3: the bias and the fix are described for FP16 and BF16 alike).  With FA_F16, Q, K, V and O
 * are binary16, the products run on the f16 MFMA with FP32 accumulation, and
 * the unnormalised probabilities are rounded to binary16 (to nearest even)
 * before the product with V; everything else (FP32 scores, running maximum,
 * row sum and shift rule) is as in fa_fwd.  row_shifted may be NULL; when
 * given it is filled as by fa_fwd_diag.  FA_BF16 is fa_fwd / fa_fwd_diag.
 * An unknown dtype returns FA_ERR_UNSUPPORTED. */
int fa_fwd_ex(int dtype, const void* Q, const void* K, const void* V, void* O, float* LSE,
              unsigned char* row_shifted,
              int B, int H, int N, int d, int causal, float scale, int stabilize,
              void* stream);

/* Backward pass with the element type chosen by `dtype`: all eight 16-bit
 * tensors are of that type, and P and dS are rounded to it (to nearest even)
 * before their products.  Arguments, workspace and launches as in fa_bwd.
 * FA_BF16 is fa_bwd.  An unknown dtype returns FA_ERR_UNSUPPORTED. */
int fa_bwd_ex(int dtype, const void* Q, const void* K, const void* V, const void* O, const void* dO,
              const float* LSE, void* dQ, void* dK, void* dV,
              void* workspace, size_t workspace_bytes,
              int B, int H, int N, int d, int causal, float scale, int stabilize,
              void* stream);

/* Human-readable text for a status code (static storage, never NULL). */
const char* fa_status_string(int status);

/* Constants of the stabilised shift rule, in base-2 exponent units
 * (reporting only; any pointer may be NULL). */
void fa_stabilize_params(float* delta_min, float* delta_max, float* fold);

/* The same constants for element type `dtype`.  For FA_F16 the largest
 * probability 2^-delta must stay far inside binary16's exponent range (whose
 * normal numbers end at 2^-14), so |R| is folded by whole units into (0, 1]:
 * delta_max = fold = 1.  The folding moves the exponent by whole units only,
 * so the rounding of the largest probability stays that of 2^-|R|.
 * Returns FA_OK, or FA_ERR_UNSUPPORTED for an unknown dtype (nothing written). */
int fa_stabilize_params_ex(int dtype, float* delta_min, float* delta_max, float* fold);

/* Tile shape of the forward kernel for head dimension d (reporting only):
 * query rows and key columns per tile; 0 for unsupported d. */
void fa_fwd_tile(int d, int* block_q, int* block_k);

/* Library version, major*10000 + minor*100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
