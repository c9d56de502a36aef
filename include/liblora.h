/*
 * liblora -- LoRA-adapted linear layer and LoRA-SwiGLU MLP, forward and
 * hand-derived backward, for AMD Instinct MI355X (gfx950).
 *
 * Definitions the entry points implement (sources are web pages; sections
 * as printed on them):
 *   [DD]  "Unsloth deep-dive: Triton kernels + hand-written backprop"
 *         (chenxutan.com/d/6058) -- 1.2 low-rank update dW = B.A,
 *         1.3 LoRALayer/LinearWithLoRA: y = x W^T + (x A^T B^T) * alpha/r,
 *         W frozen; 1.4 QLoRA 4-bit NormalFloat codes; 2.4 hand-written
 *         backward without an autograd graph.
 *   [WHY] "Why Unsloth trains 5-8x faster" (mokono.cn/news/868259) --
 *         3.1/3.2 the rank-r product x A^T stays on chip inside one fused
 *         kernel; 5.2 4-bit dequantisation fused into the matmul.
 *   [TB] "Unsloth speed secrets: Triton kernels accelerate backprop"
 *         (mokono.cn/news/201055) -- 3.2 RMSNorm kernel: per-row mean of
 *         squares, reciprocal root saved for the backward, times weight.
 *   [CR]  "Unsloth code-reading guide" (ai-reference-codex.pages.dev/
 *         frontier/unsloth) -- 2.1 4-bit weights decoded to bf16 every
 *         step; 2.3 mlp.forward := LoRA SwiGLU MLP with a manual backward;
 *         4 the MLP saves only X, e (gate output) and g (up output);
 *         5 the fast path exists only for dropout 0, no bias, no DoRA;
 *         highlights: RMSNorm statistics in fp32, cast back at the end.
 *
 * Notation: T tokens, k in_features, n out_features, r rank, s = alpha/r
 * computed in fp32.  Row-major, contiguous tensors:
 *   X [T x k], W [n x k] (frozen), A [r x k], B [n x r], Y/dY [T x n].
 *   MLP: d hidden, f ffn; gate/up W [f x d], A [r x d], B [f x r];
 *        down W [d x f], A [r x f], B [d x r]; e, g [T x f].
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library never allocates, frees or retains them.  Pointers must be
 *     16-byte aligned (LORA_ERR_MISALIGNED otherwise).
 *   - bf16 (LORA_BF16): tensors hold bfloat16; products accumulate in fp32
 *     and results are rounded once to bf16 (round to nearest even).  Rows
 *     must be 16-byte multiples: k % 8 == 0 and n % 8 == 0 (d, f for the
 *     MLP); r may be anything in 1..LORA_MAX_RANK.
 *   - fp32 (LORA_F32): every tensor fp32, fp32 arithmetic throughout, any
 *     shape.  4-bit weights are bf16-only.
 *   - Outputs are overwritten (except where a flag says accumulate).
 *     dA and dB are reduced over all T tokens in a fixed order, so results
 *     are bitwise reproducible run to run.
 *   - T == 0 is valid: forwards write nothing, backwards write dA = dB = 0;
 *     the token-sized pointers (X, Y, dY, dX, e, g) may then be NULL.
 *   - `ws`/`ws_bytes`: caller-provided device workspace of at least
 *     lora_workspace_bytes(op | LORA_WS_MINIMAL, ...) bytes (may be NULL
 *     when that is 0).  The size picks the strategy (bf16 path):
 *       >= lora_workspace_bytes(op, ...): a 4-bit base weight is first
 *         decoded to bf16 into the workspace (transposed for the backward
 *         dX products) and the GEMMs read the copy; the fused q/k/v
 *         backward also copies dense weights (stacked, transposed);
 *       otherwise (minimal): no weight copy; 4-bit codes are decoded
 *         inside the GEMM while its LDS tiles fill.
 *     Dense weights are read in place by both strategies (the backward
 *     GEMMs take W row-major [n x k] as the B operand of dY W), so for
 *     them the two sizes are equal except for the fused q/k/v backward.
 *     Both give results within the same tolerance of the exact product
 *     (fp32 accumulation in a different summation order).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *     asynchronous on it; kernel faults surface at the caller's next
 *     synchronisation.  The library keeps no mutable state between calls
 *     (beyond a once-per-device kernel-attribute setup), so calls from
 *     several host threads are safe; calls that run concurrently on the
 *     device must not share a workspace or outputs.
 *   - HIP graphs: a call launches kernels only (no allocation, memset,
 *     copy or synchronisation), so it can be captured into a graph and
 *     replayed; replays reproduce eager results bit for bit.  The first
 *     call of an op on a device sets kernel attributes (dynamic LDS size):
 *     make it once outside capture.
 *   - Every argument is validated BEFORE any HIP call; on error nothing is
 *     launched and a status code below is returned.  No exception crosses
 *     the ABI and nothing aborts.
 *   - Sizes: T <= 2^30; feature sizes (k, n, d, f) <= 2^20 (so the 256 rows
 *     of a GEMM tile of any operand span less than 2^31 bytes, one buffer
 *     descriptor's range), LORA_ERR_BAD_SHAPE otherwise.
 *   - Dropout, bias and DoRA are not representable ([CR] 5).
 */
#ifndef LIBLORA_H
#define LIBLORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LORA_ABI_VERSION 4
#define LORA_MAX_RANK 128

/* status codes */
#define LORA_OK               0
#define LORA_ERR_NULL_POINTER 1
#define LORA_ERR_BAD_SHAPE    2
#define LORA_ERR_UNSUPPORTED  3
#define LORA_ERR_WORKSPACE    4
#define LORA_ERR_MISALIGNED   5
#define LORA_ERR_HIP          6

typedef enum { LORA_F32 = 0, LORA_BF16 = 1 } lora_dtype;
typedef enum { LORA_W_DENSE = 0, LORA_W_Q4 = 1, LORA_W_Q4_DQ = 2 } lora_wfmt;

/* flags */
#define LORA_FLAG_ACCUMULATE_DX 1u   /* lora_linear_bwd: dX += result */

/*
 * Frozen base weight, logical shape [n x k] (out x in).
 *   DENSE: `w` holds n*k elements of the call's dtype.
 *   Q4 ([DD] 1.4, [CR] 2.1): 4-bit codes of a 16-level codebook with one
 *     fp32 scale per block of `blocksize` (= 64) consecutive k of one row.
 *     codes:    n*k/2 bytes; flat row-major element 2j is the LOW nibble of
 *               byte j, element 2j+1 the high nibble.
 *     absmax:   n*k/64 fp32, block b covers flat elements [64b, 64b+64).
 *     codebook: 16 fp32 levels (device memory).
 *   Decoded value of element i: bf16_rne(codebook[c_i] * absmax[i/64]) with
 *   the product taken as one fp32 multiply (round to nearest even).
 *   Requires k % 64 == 0 and the bf16 dtype.
 *   Q4_DQ ([DD] 1.4, double quantisation: the per-block constants are
 *     themselves quantised): as Q4, but `absmax` is unused and the scale of
 *     64-block b is decoded from 8 bits,
 *       absmax[b] = absmax_codebook[absmax_codes[b]] * absmax_scale[b / 256]
 *                   + absmax_offset,
 *     the product and the sum each one fp32 operation rounded to nearest
 *     even (no fused multiply-add).  The pages name the technique only;
 *     the 8-bit codes through a 256-level table, one fp32 scale per 256
 *     first-level blocks and one fp32 offset are this library's reading.
 *     absmax_codes:    n*k/64 bytes;  absmax_codebook: 256 fp32 (device);
 *     absmax_scale:    ceil(n*k/64 / 256) fp32;  absmax_blocksize: 256.
 *   Fields `absmax_codes` .. `absmax_blocksize` are read only for Q4_DQ.
 *   DENSE, optional `wt`: the same weight transposed, W^T [k x n] row-major
 *     (bf16 only; NULL: none).  A frozen weight may keep this copy next to W
 *     (made once, e.g. at load time); the backward dX products dY W then run
 *     the K-contiguous (NT) GEMM form on it, measured faster than reading W
 *     as stored.  The MLP's gate/up backward uses the gate and up copies as
 *     the two K halves of one product and needs f % 64 == 0 for that (other
 *     shapes read W as stored).  Its contents must equal W^T.
 *   All device pointers 16-byte aligned.  The library never writes through
 *   any of them.
 */
typedef struct {
  int32_t fmt;              /* lora_wfmt */
  int32_t blocksize;        /* Q4, Q4_DQ; must be 64 */
  const void *w;            /* DENSE */
  const uint8_t *codes;     /* Q4, Q4_DQ */
  const float *absmax;      /* Q4 */
  const float *codebook;    /* Q4, Q4_DQ */
  const uint8_t *absmax_codes;     /* Q4_DQ */
  const float *absmax_codebook;    /* Q4_DQ */
  const float *absmax_scale;       /* Q4_DQ */
  float absmax_offset;             /* Q4_DQ */
  int32_t absmax_blocksize;        /* Q4_DQ; must be 256 */
  const void *wt;                  /* DENSE, optional: W^T [k x n] */
} lora_weight;

/* ops for lora_workspace_bytes */
#define LORA_OP_LINEAR_FWD 0
#define LORA_OP_LINEAR_BWD 1
#define LORA_OP_MLP_FWD    2
#define LORA_OP_MLP_BWD    3
#define LORA_OP_QKV_FWD    4   /* lora_qkv_workspace_bytes only */
#define LORA_OP_QKV_BWD    5
#define LORA_OP_RMSNORM_MLP_FWD 6   /* lora_rmsnorm_swiglu_mlp_fwd */
#define LORA_OP_RMSNORM_MLP_BWD 7   /* lora_rmsnorm_swiglu_mlp_bwd */
#define LORA_OP_RMSNORM_QKV_FWD 8   /* lora_rmsnorm_qkv_fwd (lora_qkv_workspace_bytes) */
#define LORA_OP_RMSNORM_QKV_BWD 9   /* lora_rmsnorm_qkv_bwd (lora_qkv_workspace_bytes) */
/* or-ed into `op`: size of the minimal-memory strategy */
#define LORA_WS_MINIMAL    0x100

/*
 * Y = X W^T + s (X A^T) B^T                                  ([DD] 1.3)
 * The rank-r product s (X A^T) is formed once per call by a skinny MFMA
 * kernel and written to the workspace as bf16 [T x r] (rounded up to 16
 * columns); the GEMM adds it in its epilogue as a second MFMA pass with
 * K = r against B.  ([WHY] 3.2 keeps x A^T on chip inside the fused kernel;
 * measured on MI355X, computing it inside the GEMM's K loop pushed the
 * register file over its 512 entries and made the layer slower than this
 * one extra [T x r] round trip, under 0.1 % of the GEMM's traffic.)
 * In: X [T x k], W (lora_weight [n x k]), A [r x k], B [n x r].
 * Out: Y [T x n].
 */
int lora_linear_fwd(int dtype, int64_t T, int64_t k, int64_t n, int64_t r,
                    float alpha, const void *X, const lora_weight *W,
                    const void *A, const void *B, void *Y,
                    void *ws, size_t ws_bytes, void *stream);

/*
 * Hand-derived backward of lora_linear_fwd for upstream gradient dY
 * ([DD] 2.4; W frozen, so there is no dW):
 *   G = dY B,  dX = dY W + s G A,  dA = s G^T X,  dB = s dY^T (X A^T).
 * In: X, W, A, B as in the forward, dY [T x n].
 * Out: dX [T x k] (NULL skips it; with LORA_FLAG_ACCUMULATE_DX the result
 *      is added to dX, which lets projections that share one input, such as
 *      q/k/v, sum their input gradients), dA [r x k], dB [n x r].
 */
int lora_linear_bwd(int dtype, int64_t T, int64_t k, int64_t n, int64_t r,
                    float alpha, const void *X, const lora_weight *W,
                    const void *A, const void *B, const void *dY, void *dX,
                    void *dA, void *dB, uint32_t flags,
                    void *ws, size_t ws_bytes, void *stream);

/*
 * lora_linear_bwd without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments (minus ws/ws_bytes), results and errors as lora_linear_bwd run
 * with the minimal workspace (4-bit weights are decoded inside the GEMM).
 * Its scratch memory is a static device array of LORA_NOALLOC_SCRATCH_BYTES
 * (128 MiB) per GPU, held from the library's first use on that GPU until the
 * process ends; a call whose minimal workspace would exceed it returns
 * LORA_ERR_WORKSPACE before any HIP call.  The need is
 * lora_workspace_bytes(LORA_OP_LINEAR_BWD | LORA_WS_MINIMAL, ...): with
 * k = n = 4096, 23 MiB at T = 16384, r = 16 and 92 MiB at T = 16384, r = 64
 * (the 8B model's projections fit); r = 128 with T = 4096 needs 152 MiB
 * and is refused.  Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (concurrent streams, or host
 * threads) race and must be serialised by the caller.  No part of the array
 * needs to start at zero: every kernel writes its scratch before reading it.
 * The first call on a device looks up the array's device address (a HIP
 * call); make it once outside graph capture.
 */
#define LORA_NOALLOC_SCRATCH_BYTES (128u << 20)
int lora_linear_bwd_noalloc(int dtype, int64_t T, int64_t k, int64_t n, int64_t r,
                            float alpha, const void *X, const lora_weight *W,
                            const void *A, const void *B, const void *dY, void *dX,
                            void *dA, void *dB, uint32_t flags, void *stream);

/*
 * LoRA-SwiGLU MLP forward ([CR] 2.3, 4; SwiGLU per [HF]-blog section 1):
 *   e = lin(X; gate), g = lin(X; up), h = silu(e) * g, Y = lin(h; down),
 * each lin a LoRA linear with the same r and alpha.  silu(z) = z/(1+e^-z).
 * Out: Y [T x d]; e_saved, g_saved [T x f] (the activations the backward
 * needs; X is the caller's).  h lives in the workspace.  The down
 * projection's rank-r product s (h Ad^T) comes, for r <= 16 with dense or
 * decoded weights, from the gate/up GEMM's epilogue (per-tile sums over its
 * features, added in a fixed order) instead of a second pass over h.
 */
int lora_swiglu_mlp_fwd(int dtype, int64_t T, int64_t d, int64_t f, int64_t r,
                        float alpha, const void *X,
                        const lora_weight *Wg, const void *Ag, const void *Bg,
                        const lora_weight *Wu, const void *Au, const void *Bu,
                        const lora_weight *Wd, const void *Ad, const void *Bd,
                        void *Y, void *e_saved, void *g_saved,
                        void *ws, size_t ws_bytes, void *stream);

/*
 * LoRA-SwiGLU MLP backward from the saved X, e, g and upstream dY:
 *   h = silu(e) g;  (dh, dAd, dBd) = linear_bwd(h, dY; down)
 *   de = dh g sig(e) (1 + e (1 - sig(e))),  dg = dh silu(e)
 *   (dXg, dAg, dBg) = linear_bwd(X, de; gate), same for up; dX = dXg + dXu.
 * Out: dX [T x d] (NULL skips it), dAg, dAu [r x d], dBg, dBu [f x r],
 *      dAd [r x f], dBd [d x r].
 */
int lora_swiglu_mlp_bwd(int dtype, int64_t T, int64_t d, int64_t f, int64_t r,
                        float alpha, const void *X,
                        const lora_weight *Wg, const void *Ag, const void *Bg,
                        const lora_weight *Wu, const void *Au, const void *Bu,
                        const lora_weight *Wd, const void *Ad, const void *Bd,
                        const void *e_saved, const void *g_saved, const void *dY,
                        void *dX, void *dAg, void *dBg, void *dAu, void *dBu,
                        void *dAd, void *dBd,
                        void *ws, size_t ws_bytes, void *stream);

/*
 * RMSNorm fused into the gate/up projections of the LoRA-SwiGLU MLP
 * ([HF]-blog section 1: RMSNorm fused with the linear projections; [TB] 3.2
 * the RMSNorm kernel), forward:
 *   rstd[t] = 1 / sqrt(sum_j X[t,j]^2 / d + eps),  Xn = X rstd diag(w),
 *   (Y, e, g) = lora_swiglu_mlp_fwd(Xn, ...)
 * without forming Xn: the norm weight w is frozen like the base weights, so
 * the caller passes the gate and up base weights ALREADY FOLDED,
 * Wg' = Wg diag(w) and Wu' = Wu diag(w) (lora_fold_norm_weight, once), and
 * the GEMMs read the raw rows X and scale each output row by rstd (an exact
 * row factor of every term); the adapters A stay the trainable parameters
 * and A diag(w) is formed per call.  X is the raw [T x d] input (the residual
 * stream), norm_w [d], rstd [T] fp32 is written for the backward.  bf16 and
 * dense weights only (LORA_ERR_UNSUPPORTED otherwise: a 4-bit weight cannot
 * hold W diag(w); use lora_rmsnorm_fwd in front of lora_swiglu_mlp_fwd).
 * eps finite and >= 0.  Workspace: LORA_OP_RMSNORM_MLP_FWD.
 */
int lora_rmsnorm_swiglu_mlp_fwd(int dtype, int64_t T, int64_t d, int64_t f, int64_t r,
                                float alpha, float eps, const void *X, const void *norm_w,
                                const lora_weight *Wg, const void *Ag, const void *Bg,
                                const lora_weight *Wu, const void *Au, const void *Bu,
                                const lora_weight *Wd, const void *Ad, const void *Bd,
                                void *Y, void *e_saved, void *g_saved, float *rstd,
                                void *ws, size_t ws_bytes, void *stream);

/*
 * Backward of lora_rmsnorm_swiglu_mlp_fwd from X, rstd, e, g and dY (same
 * folded gate/up weights): the adapter gradients of lora_swiglu_mlp_bwd
 * taken at Xn, and dX the gradient with respect to the RAW input X,
 *   dX = rstd gn - rstd^3 X (sum_j gn_j X_j) / d,   gn = dXn diag(w),
 * where dXn is the MLP's input gradient (the folded projections return gn
 * directly).  The row sum comes from the down backward's epilogue
 * (sum_j gn_j X_j = sum_k (de e + dg g) / rstd over the ffn features) and
 * dX is written by the dX GEMM's epilogue, so neither Xn nor gn is ever
 * stored.  LORA_FLAG_ACCUMULATE_DX adds dX to the caller's dX (the residual
 * branch's gradient).  dX NULL skips it.  Workspace: LORA_OP_RMSNORM_MLP_BWD.
 */
int lora_rmsnorm_swiglu_mlp_bwd(int dtype, int64_t T, int64_t d, int64_t f, int64_t r,
                                float alpha, const void *X, const void *norm_w,
                                const float *rstd,
                                const lora_weight *Wg, const void *Ag, const void *Bg,
                                const lora_weight *Wu, const void *Au, const void *Bu,
                                const lora_weight *Wd, const void *Ad, const void *Bd,
                                const void *e_saved, const void *g_saved, const void *dY,
                                void *dX, void *dAg, void *dBg, void *dAu, void *dBu,
                                void *dAd, void *dBd, uint32_t flags,
                                void *ws, size_t ws_bytes, void *stream);

/*
 * out[i][j] = bf16_rne(W[i][j] * w[j]) (one fp32 multiply): a frozen RMSNorm
 * weight w [k] folded into a frozen base weight W [n x k] that reads the
 * norm's output, for lora_rmsnorm_swiglu_mlp_fwd/bwd and lora_rmsnorm_qkv_fwd/bwd.  bf16, k % 8 == 0;
 * out may be W itself (in place).  No workspace.
 */
int lora_fold_norm_weight(int dtype, int64_t n, int64_t k, const void *W, const void *norm_w,
                          void *out, void *stream);

/*
 * Standalone 4-bit decode ([CR] 2.1 fast_dequantize; [DD] 1.4):
 * out[i] = bf16_rne(codebook[c_i] * absmax[i/64]) for i in [0, n*k),
 * same layout rules as lora_weight Q4.  out_dtype must be LORA_BF16.
 * out: n*k bf16, device.
 */
int lora_dequant4(int64_t n, int64_t k, const uint8_t *codes, const float *absmax,
                  const float *codebook, int blocksize, int out_dtype, void *out,
                  void *stream);

/*
 * Decode a quantised base weight of either 4-bit format (Q4 or Q4_DQ,
 * [DD] 1.4) to bf16 with exactly the values every other entry point uses:
 * out[i] = bf16_rne(codebook[c_i] * absmax[i / 64]), absmax decoded from
 * its 8-bit codes first for Q4_DQ (see lora_weight).  out: n*k bf16,
 * device, 16-byte aligned; out_dtype must be LORA_BF16.  DENSE weights are
 * rejected with LORA_ERR_UNSUPPORTED.  No workspace.
 */
int lora_decode_weight(int64_t n, int64_t k, const lora_weight *W, int out_dtype, void *out,
                       void *stream);

/*
 * RMSNorm over the rows of X [T x d], the step in front of the gate/up and
 * q/k/v projections ([TB] 3.2; statistics in fp32 and one cast at the end
 * per [CR] highlights):
 *   rstd[t] = 1 / sqrt(sum_j X[t,j]^2 / d + eps)       (fp32, [T])
 *   Y[t,j]  = X[t,j] * rstd[t] * w[j]                  (fp32, rounded once)
 * X, Y [T x d] and w [d] in `dtype`; Y may not alias X.  rstd is saved for
 * lora_rmsnorm_bwd.  eps must be finite and >= 0 (LORA_ERR_UNSUPPORTED).
 * Sums run in a fixed order: bitwise reproducible.  No workspace.
 */
int lora_rmsnorm_fwd(int dtype, int64_t T, int64_t d, float eps, const void *X, const void *w,
                     void *Y, float *rstd, void *stream);

/*
 * Input gradient of lora_rmsnorm_fwd for upstream dY [T x d] (w frozen, so
 * there is no dw):  g = dY * w,
 *   dX[t,i] = rstd g_i - rstd^3 X[t,i] (sum_j g_j X[t,j]) / d   (fp32).
 * With LORA_FLAG_ACCUMULATE_DX the result is added to dX (the residual
 * branch's gradient), rounded once.  X, w, rstd as in the forward.
 */
int lora_rmsnorm_bwd(int dtype, int64_t T, int64_t d, const void *X, const void *w,
                     const float *rstd, const void *dY, void *dX, uint32_t flags,
                     void *stream);

/*
 * Fused q/k/v LoRA projections of one input (the LoRA_QKV pattern of
 * [CR] 4: three LoRA linears that share X, computed as one):
 *   Q = lin(X; Wq, Aq, Bq) [T x nq], K = lin(X; Wk, Ak, Bk) [T x nkv],
 *   V = lin(X; Wv, Av, Bv) [T x nkv], each exactly as lora_linear_fwd.
 * bf16 with nq, nkv multiples of 256 and 3r <= 256: one GEMM over the
 * stacked weights [Wq; Wk; Wv] with one rank-3r LoRA pass; other shapes,
 * ranks and fp32 run the three projections one by one (same results within
 * the same tolerance).  Weights share one format.  Workspace:
 * lora_qkv_workspace_bytes(LORA_OP_QKV_FWD, ...).
 */
int lora_qkv_fwd(int dtype, int64_t T, int64_t k, int64_t nq, int64_t nkv, int64_t r,
                 float alpha, const void *X,
                 const lora_weight *Wq, const void *Aq, const void *Bq,
                 const lora_weight *Wk, const void *Ak, const void *Bk,
                 const lora_weight *Wv, const void *Av, const void *Bv,
                 void *Q, void *K, void *V, void *ws, size_t ws_bytes, void *stream);

/*
 * Backward of lora_qkv_fwd from dQ, dK, dV:
 *   dX (+)= sum over p in {q, k, v} of dY_p W_p + s (dY_p B_p) A_p
 *   dA_p = s (dY_p B_p)^T X,  dB_p = s dY_p^T (X A_p^T)
 * dX NULL skips it; LORA_FLAG_ACCUMULATE_DX adds to dX.  bf16 with the
 * fast workspace and 3r <= 256: [dQ | dK | dV] is packed into the workspace
 * and dX is one GEMM with K = nq + 2 nkv against the transposed stacked
 * weights; otherwise the three projections run one by one.
 */
int lora_qkv_bwd(int dtype, int64_t T, int64_t k, int64_t nq, int64_t nkv, int64_t r,
                 float alpha, const void *X,
                 const lora_weight *Wq, const void *Aq, const void *Bq,
                 const lora_weight *Wk, const void *Ak, const void *Bk,
                 const lora_weight *Wv, const void *Av, const void *Bv,
                 const void *dQ, const void *dK, const void *dV, void *dX,
                 void *dAq, void *dBq, void *dAk, void *dBk, void *dAv, void *dBv,
                 uint32_t flags, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes of lora_qkv_fwd / lora_qkv_bwd (op LORA_OP_QKV_FWD or
 * LORA_OP_QKV_BWD, optionally | LORA_WS_MINIMAL) and of lora_rmsnorm_qkv_fwd
 * / _bwd (LORA_OP_RMSNORM_QKV_FWD / _BWD, one strategy); 0 for invalid
 * arguments or shapes the op does not take. */
size_t lora_qkv_workspace_bytes(int op, int dtype, int wfmt, int64_t T, int64_t k, int64_t nq,
                                int64_t nkv, int64_t r);

/*
 * RMSNorm fused into the q/k/v projections ([HF]-blog section 1: RMSNorm
 * fused with the linear projections; [TB] 3.2 the RMSNorm kernel), forward:
 *   rstd[t] = 1 / sqrt(sum_j X[t,j]^2 / k + eps),  Xn = X rstd diag(w),
 *   (Q, K, V) = lora_qkv_fwd(Xn, ...)
 * without forming Xn, as lora_rmsnorm_swiglu_mlp_fwd does for the MLP: the
 * caller passes the three base weights folded with the frozen norm weight,
 * Wp' = Wp diag(w) (lora_fold_norm_weight), the stacked GEMM reads the raw
 * rows X and its store epilogue scales each output row by rstd; A diag(w)
 * is formed per call.  X [T x k] raw rows, norm_w [k], rstd [T] fp32
 * written for the backward.  bf16, dense weights, nq and nkv multiples of
 * 256 and 3r <= 256 (LORA_ERR_UNSUPPORTED otherwise; lora_rmsnorm_fwd in
 * front of lora_qkv_fwd takes every shape).  eps finite and >= 0.
 * Workspace: lora_qkv_workspace_bytes(LORA_OP_RMSNORM_QKV_FWD, ...).
 */
int lora_rmsnorm_qkv_fwd(int dtype, int64_t T, int64_t k, int64_t nq, int64_t nkv, int64_t r,
                         float alpha, float eps, const void *X, const void *norm_w,
                         const lora_weight *Wq, const void *Aq, const void *Bq,
                         const lora_weight *Wk, const void *Ak, const void *Bk,
                         const lora_weight *Wv, const void *Av, const void *Bv,
                         void *Q, void *K, void *V, float *rstd,
                         void *ws, size_t ws_bytes, void *stream);

/*
 * Backward of lora_rmsnorm_qkv_fwd from X, rstd and dQ, dK, dV (same folded
 * weights): the adapter gradients of lora_qkv_bwd taken at Xn (formed from
 * X with the rstd row and w column factors, Xn never stored), and dX the
 * gradient with respect to the RAW input X,
 *   dX = rstd gn - rstd^3 X (sum_j gn_j X_j) / k,   gn = dXn diag(w),
 * where the folded projections' dX GEMM returns gn directly.  Unlike the
 * MLP, no earlier step of this backward holds partial sums that give
 * sum_j gn_j X_j, so gn goes through the workspace once and one row pass
 * applies the norm's gradient.  LORA_FLAG_ACCUMULATE_DX adds dX to the
 * caller's dX (the residual branch's gradient); dX NULL skips it.
 * Workspace: lora_qkv_workspace_bytes(LORA_OP_RMSNORM_QKV_BWD, ...).
 */
int lora_rmsnorm_qkv_bwd(int dtype, int64_t T, int64_t k, int64_t nq, int64_t nkv, int64_t r,
                         float alpha, const void *X, const void *norm_w, const float *rstd,
                         const lora_weight *Wq, const void *Aq, const void *Bq,
                         const lora_weight *Wk, const void *Ak, const void *Bk,
                         const lora_weight *Wv, const void *Av, const void *Bv,
                         const void *dQ, const void *dK, const void *dV, void *dX,
                         void *dAq, void *dBq, void *dAk, void *dBk, void *dAv, void *dBv,
                         uint32_t flags, void *ws, size_t ws_bytes, void *stream);

/*
 * Merged weight out = W + sign * s * B A, s = alpha / r ([DD] 1.2: the
 * low-rank update dW = B.A; added to the frozen weight it gives one plain
 * linear layer with the same output, the merged export of [DD] 5.1).
 * sign = +1 merges, -1 unmerges.  W: dense [n x k] in `dtype`, or 4-bit
 * (dtype must be LORA_BF16; decoded to bf16 first).  A [r x k], B [n x r]
 * in `dtype`.  out: [n x k] in `dtype`, device, may not alias W.  B A is
 * accumulated in fp32; the sum is rounded once to `dtype`.  No workspace.
 */
int lora_merge(int dtype, int64_t n, int64_t k, int64_t r, float alpha, int sign,
               const lora_weight *W, const void *A, const void *B, void *out,
               void *stream);

/* Workspace bytes of an op (k_or_d / n_or_f as in the op's signature;
 * `wfmt` is the base-weight format): the fast strategy's size, or with
 * LORA_WS_MINIMAL or-ed into `op` the smallest size the op accepts.
 * Returns 0 for invalid arguments. */
size_t lora_workspace_bytes(int op, int dtype, int wfmt, int64_t T,
                            int64_t k_or_d, int64_t n_or_f, int64_t r);

const char *lora_strerror(int status);
int lora_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* LIBLORA_H */
