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
 *     values are not checked; they propagate to the rows they touch: a
 *     non-finite Q row to that output row, a non-finite K row to the rows that
 *     see that key, and a non-finite V row to every row that processes the
 *     forward's key block holding it (fa_fwd_tile; the masked keys of a block
 *     still enter its product with V, with probability 0).
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
  FA_ERR_UNSUPPORTED = -2,   /* head dimension other than 64 / 128; baseline N > 16384 */
  FA_ERR_WORKSPACE = -3,     /* workspace NULL or smaller than fa_bwd_workspace_bytes() */
  FA_ERR_LAUNCH = -4,        /* the HIP runtime rejected a kernel launch */
  FA_ERR_DEVICE = -5,        /* no gfx950 device current, or a device query failed */
  FA_ERR_TOO_LARGE = -6      /* B*H*N above fa_bwd_noalloc's fixed scratch (FA_BWD_NOALLOC_MAX_ROWS) */
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

/* Forward pass split over keys, for launches too small to fill the GPU (a
 * single head, short sequences).  Each (head, 128-row query block) is cut
 * into `splits` contiguous ranges of its 128-key blocks (fa_fwd_tile), one
 * workgroup each.
 * A workgroup first replays the key blocks before its range through the
 * running row maximum and repeated-maximum bookkeeping alone (scores only,
 * no exponentials or products), so its own blocks are shifted, and their
 * unnormalised probabilities rounded to BF16, exactly as in one pass over
 * the row (page 2, "Mechanism 2": the fix acts on the running maximum of a
 * row).  It writes its unnormalised output, row sum and final shift M_s to
 * the workspace; a second launch merges the ranges with weights
 * 2^(M_s - M), M the last range's shift (the row's):
 *   O = bf16(sum_s 2^(M_s - M) O_bar_s / sum_s 2^(M_s - M) l_s).
 * Against fa_fwd only the FP32 rounding of those rescalings differs (one
 * product per range instead of one per block); with splits = 1 the result
 * is bitwise fa_fwd's.  bf16 tensors as in fa_fwd; 1 <= splits <= 64; the
 * workspace (256-byte aligned) holds at least
 * fa_fwd_split_workspace_bytes() bytes.  Two launches.  On return the
 * workspace holds each range's partial results, fp32, each part starting at
 * the next multiple of 256 bytes: O_bar (splits, B, H, N, d), then
 * l (splits, B, H, N), then the shift M (splits, B, H, N) in base-2 units
 * (range splits-1 holds the row's final shift). */
size_t fa_fwd_split_workspace_bytes(int B, int H, int N, int d, int splits);
int fa_fwd_split(const void* Q, const void* K, const void* V, void* O, float* LSE,
                 int splits, void* workspace, size_t workspace_bytes,
                 int B, int H, int N, int d, int causal, float scale, int stabilize,
                 void* stream);

/* Bytes of device workspace fa_bwd needs: the fp32 vector D = rowsum(dO*O)
 * of shape (B,H,N), rounded up to 256 bytes.  Returns 0 for invalid sizes. */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int d, int causal);

/* Backward pass (dQ, dK, dV of L = sum(O * dO)), recomputing the
 * probabilities from LSE.  Page 1, section 4.3: once the forward's softmax
 * output is off, the gradients with respect to Q and K that back-propagation
 * relies on are off the true derivatives too; here that happens through
 * D = rowsum(dO * O), taken from the bf16 forward output, and through
 * dS = P (dP - D).  The recipe is the usual tiled one for exact attention
 * (page 3, "Flash Attention: from academic breakthrough to industry
 * standard": the N x N matrices are never stored, so they are recomputed
 * block by block):
 *   P = exp(S - LSE) (FP32),  dP = dO V^T,  dS = P (dP - D),
 *   dV = bf16(P)^T dO,  dK = scale bf16(dS)^T Q,  dQ = scale bf16(dS) K,
 * with FP32 accumulation and bf16 results.
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

/* Backward pass that allocates nothing, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid hipMalloc.  It computes exactly what fa_bwd computes,
 * with the same kernels and bitwise the same dQ, dK and dV, but keeps the
 * fp32 vector D = rowsum(dO*O) in a scratch array of the library instead of
 * a caller workspace.  That array is a fixed device array of
 * FA_BWD_NOALLOC_MAX_ROWS floats (16 MiB) on every GPU the library runs on,
 * held until the process ends; its address on a device is looked up on the
 * first call made with that device current.  B*H*N above
 * FA_BWD_NOALLOC_MAX_ROWS returns FA_ERR_TOO_LARGE before anything is
 * enqueued.  Every call on one GPU uses that GPU's one array: two calls that
 * may overlap on the same GPU (different streams, or threads that do not
 * order their calls) race on it, and the caller must serialise them.
 * Arguments, layouts and launches otherwise as in fa_bwd (bf16 tensors). */
#define FA_BWD_NOALLOC_MAX_ROWS 4194304
int fa_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                   const float* LSE, void* dQ, void* dK, void* dV,
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

/* ------------------------------------------------------------------------
 * Baseline attention with FP32 accumulation (page 3, "What did Meta's study
 * find": FlashAttention's numeric deviation is measured there against a
 * baseline attention that accumulates in FP32, in an isolated BF16 forward
 * pass).  This is the plain unfused computation, for comparison with
 * fa_fwd on the same device and inputs; it is bound by HBM traffic on the
 * N x N matrices it materialises:
 *
 *   S   = fl32(fl32(Q K^T) * scale)        FP32, (B,H,N,ld); for causal
 *                                           attention keys j > i are not read
 *   r_i = max_j S_ij,  e_ij = fl32(2^(fl32(S_ij - r_i) * log2 e)),
 *   l_i = sum_j e_ij (FP32),  P_ij = bf16(e_ij * fl32(1 / l_i))
 *   O   = bf16(P V) (FP32 accumulation),  LSE_i = r_i + ln l_i
 *
 * The probabilities are normalised before their BF16 cast (in fa_fwd the
 * unnormalised ones are cast and O is divided by l at the end).  Q, K, V, O
 * are bf16 (B,H,N,d) with d 64 or 128, LSE fp32 (B,H,N).  N is limited to
 * 16384 (FA_ERR_UNSUPPORTED above) and B*H*N to below 2^31.  The S and P
 * matrices have a row stride of ld = fa_base_ld(N) elements (N rounded up
 * to 64); for causal attention only the 64-key blocks up to the diagonal
 * are written and read.  Other conventions as above.
 * ------------------------------------------------------------------------ */

/* Row stride (in elements) of the baseline's S and P: N rounded up to 64
 * (0 for N < 1). */
int fa_base_ld(int N);

/* Bytes of device workspace fa_base_fwd needs: S (fp32) at offset 0, then P
 * (bf16) at the next multiple of 256 bytes, each (B,H,N,fa_base_ld(N)).
 * Returns 0 for invalid or unsupported sizes. */
size_t fa_base_workspace_bytes(int B, int H, int N, int d, int causal);

/* The baseline forward: fa_base_scores, fa_base_softmax and fa_base_pv on
 * `stream` (three launches), with S and P in the caller's workspace
 * (256-byte aligned, at least fa_base_workspace_bytes()).
 *   in : Q, K, V bf16 (B,H,N,d)     out: O bf16 (B,H,N,d), LSE fp32 (B,H,N)
 * Returns FA_ERR_WORKSPACE for a missing or short workspace. */
int fa_base_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
                void* workspace, size_t workspace_bytes,
                int B, int H, int N, int d, int causal, float scale, void* stream);

/* The three steps of fa_base_fwd, exposed so that each can be timed:
 *   fa_base_scores : S = fl32(fl32(Q K^T) * scale) into S (fp32, 16-byte
 *                    aligned, (B,H,N,ld)); entries past the diagonal block
 *                    (causal) and past column N are not written
 *   fa_base_softmax: P (bf16, (B,H,N,ld), 16-byte aligned) and LSE from S;
 *                    P is written for every key the PV step reads, zeros past
 *                    the row's last visible key
 *   fa_base_pv     : O = bf16(P V) */
int fa_base_scores(const void* Q, const void* K, float* S,
                   int B, int H, int N, int d, int causal, float scale, void* stream);
int fa_base_softmax(const float* S, void* P, float* LSE,
                    int B, int H, int N, int causal, void* stream);
int fa_base_pv(const void* P, const void* V, void* O,
               int B, int H, int N, int d, int causal, void* stream);

/* Measured MFMA ceiling (reporting only): launches `blocks` workgroups of
 * four waves that each run `iters` rounds of eight independent
 * v_mfma_f32_32x32x16_bf16 chains on register operands (the product
 * instruction of every attention kernel here), and writes one float per
 * thread to `out` (blocks*256 floats, device memory) so that the work is
 * kept.  Returns the FLOP that launch performs (> 0), or a negative status
 * (FA_ERR_INVALID_ARG for a NULL `out` or non-positive sizes, FA_ERR_DEVICE,
 * FA_ERR_LAUNCH).  Timing it with events on `stream` gives the dense bf16
 * rate the chip sustains, against which the attention kernels' achieved
 * rates are also quoted. */
long long fa_mfma_probe(float* out, int blocks, int iters, void* stream);

/* Measured HBM ceiling (reporting only): reads `bytes` (a multiple of 16) of
 * `src` (device memory, 16-byte aligned) with 16-byte loads and writes one
 * folded value per thread to `sink` (device memory, 4096*256 unsigned ints),
 * so that the loads are kept.  Timed with events on `stream`, bytes over the
 * time is the streaming read bandwidth the memory-bound kernels (whose
 * traffic is almost all reads) are compared with.
 * Returns FA_OK, FA_ERR_INVALID_ARG, FA_ERR_DEVICE or FA_ERR_LAUNCH. */
int fa_hbm_probe(const void* src, size_t bytes, unsigned int* sink, void* stream);

/* Instruction-issue probe (reporting only): what the softmax's instructions
 * cost on a SIMD beside MFMA work, and what LDS operand reads add; run
 * long, it also shows the board power each kind of work draws.  Launches `blocks`
 * workgroups of 512 threads, one per CU (their LDS allocation allows no
 * second), in which `waves_per_simd` (1 or 2) waves per SIMD loop `iters`
 * times; per iteration an active wave issues
 *   kind 0: 8 bf16 MFMAs;  kind 1..5: 64 of v_fma_f32, v_max3_f32,
 *   v_med3_f32, v_exp_f32 or v_cvt_pk_bf16_f32;  kind 6: 8 MFMAs each
 *   followed by 8 v_fma_f32;  kind 7 (two waves per SIMD only): 16 MFMAs in
 *   one wave, 128 v_fma_f32 in the other;  kind 8: 8 LDS reads of 16 bytes
 *   per lane (ds_read_b128);  kind 9: 8 MFMAs, each with its A operand read
 *   from LDS (16 bytes per lane);  kind 10: 16 transposing LDS reads of 8
 *   bytes per lane (ds_read_b64_tr_b16);  kind 11: 8 MFMAs, each with its A
 *   operand from two transposing LDS reads;  kind 12: 8 MFMAs each followed
 *   by 8 v_exp_f32;  kind 13: 8 MFMAs each followed by 8 instructions of the
 *   softmax's mix (2 exponentials, 2 FMAs, 2 adds, a max3 and a med3);
 *   kinds 14, 15, 16: 8 MFMAs each followed by 8 v_max3_f32, 8
 *   v_cvt_pk_bf16_f32 or 8 two-operand v_max_f32.
 * Writes one float per thread to `out` (blocks*512 floats, device memory).
 * Timed with events on `stream`, time / (blocks / CUs) / iters is the time of
 * one iteration of a SIMD's waves.  Returns FA_OK, FA_ERR_INVALID_ARG (kind
 * outside 0..16, waves_per_simd not 1 or 2, kind 7 with one wave, NULL or
 * misaligned out, non-positive sizes), FA_ERR_DEVICE or FA_ERR_LAUNCH. */
int fa_issue_probe(int kind, int waves_per_simd, float* out, int blocks, int iters, void* stream);

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
 * query rows per workgroup and keys per block (128 and 128 for both d = 64
 * and d = 128); 0 for unsupported d.  The key block is also the unit of the
 * running maximum and repeated-maximum bookkeeping. */
void fa_fwd_tile(int d, int* block_q, int* block_k);

/* Library version, major*10000 + minor*100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
