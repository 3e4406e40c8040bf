/*
 * qlora_nf4.h -- C ABI of the MI355X (gfx950) QLoRA linear-layer library.
 *
 * The library computes the hot path of QLoRA fine-tuning on one GPU:
 *   1. blockwise NF4 quantization of a frozen fp32 weight (64-weight blocks,
 *      absmax scale, 16 levels at N(0,1) quantiles),
 *   2. double quantization of the per-block constants to 8-bit codes in
 *      groups of 256 with one fp32 scale per group,
 *   3. dequantization to bf16,
 *   4. the fused forward Y = X W'^T + (alpha/r) (X A^T) B^T and its backward
 *      (dX through the dequantized frozen base W', dA and dB for the bf16
 *      adapters; the base gets no gradient), optionally with LoRA dropout
 *      on the adapter input;
 * and around it: dequantize-and-merge of an adapter into a dense bf16
 * weight, codec variants (FP4 / INT4 tables, fp32 or centered 8-bit block
 * constants) for quantization-error comparisons, and an 8-bit AdamW step on
 * the adapters with its state in device memory or paged through host memory.
 *
 * Sources for what each call computes are the pages "Qlora Expert" (Core
 * Concept), "QLoRA: The 4-bit Revolution" (sections 1 and 2), "QLoRA Guide"
 * (How QLoRA Works: Forward pass; NF4 vs uniform INT4), "QLoRA Implementation
 * Details (2025 Edition)" (Step 1 NF4 Math; Step 4 LoRA adapters) and
 * "QLORA: Efficient Finetuning of Quantized LLMs" (paper summary: Methods,
 * Notes).  The fused calls follow the pages' BitsAndBytesConfig: quant type
 * NF4, double quantization on, bf16 compute; and their LoraConfig: rank r,
 * lora_alpha, bias "none", lora_dropout (the *_dropout entry points).  Each
 * further call cites its own passages.
 *
 * Conventions for every call
 *   - Shapes follow the Linear convention: W is [N, K] (out, in), X [M, K],
 *     Y [M, N], A [r, K], B [N, r].  All matrices are dense row-major.
 *   - bf16 tensors are passed as raw uint16_t bit patterns.
 *   - Pointers marked "device" are device (HBM) addresses; the caller owns
 *     every buffer, including workspaces.  The library never allocates or
 *     frees memory, keeps no pointer after a call returns, and holds no
 *     global device state, so calls are reentrant (the paged optimizer step
 *     creates HIP events for its copies and destroys them before returning).
 *   - All device work is enqueued asynchronously on `stream` (a hipStream_t
 *     passed as void*; NULL is the default stream).  Outputs are valid once
 *     the stream reaches them; inputs must stay unchanged until then.
 *   - Return value: 0 on success or a negative QN_E* code.  Argument errors
 *     are detected on the host before anything is launched.
 */
#ifndef QLORA_NF4_H
#define QLORA_NF4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QN_OK 0
#define QN_EINVAL (-1)      /* null pointer, bad size, r out of range,
                               K % 64 != 0 in a fused call, unknown dtype,
                               misaligned pointer */
#define QN_EWORKSPACE (-2)  /* workspace smaller than qlora_workspace_bytes */
#define QN_EHIP (-3)        /* the HIP runtime reported a launch error */
#define QN_ENONFINITE (-4)  /* written to *status_dev by nf4_quantize */
#define QN_ESYNC (-5)       /* written to a fused call's workspace status
                               word when one piece of a split output tile
                               never published its partial sum (see
                               qlora_linear_fwd); never observed in normal
                               operation, the wait is bounded against hangs */

#define QN_F32 0            /* output element type: fp32 */
#define QN_BF16 1           /* output element type: bf16 (RNE) */

#define QN_FWD 0
#define QN_BWD 1
#define QN_FWD_DROPOUT 2    /* forward with LoRA dropout (general path) */

#define QN_BLOCK 64         /* weights per absmax block */
#define QN_GROUP 256        /* block constants per double-quant group */
#define QN_MAX_RANK 256

/*
 * An NF4 + double-quantized weight of rows x cols elements (numel =
 * rows*cols), flattened row-major:
 *   packed : device, ceil(numel/2) bytes.  Element 2i sits in bits 0-3 of
 *            byte i, element 2i+1 in bits 4-7; an odd tail nibble is 7.
 *   qabs   : device, nb = ceil(numel/64) bytes, the 8-bit code of each
 *            block's absmax.
 *   gscale : device, ng = ceil(nb/256) floats, the fp32 scale d of each
 *            group of 256 block codes.
 * The dequantized value of element e in block b = e/64, group g = b/256 is
 *   bf16_rne( L[code_e] * (float(qabs[b]) * gscale[g]) )
 * with both products in fp32 and L the 16 levels of nf4_codebook().
 * packed must be 16-byte aligned.
 */
typedef struct {
  uint8_t* packed;
  uint8_t* qabs;
  float* gscale;
  int64_t rows;
  int64_t cols;
} nf4_tensor;

/*
 * nf4_codebook -- the 16 NF4 levels and the 15 decision thresholds (host).
 *
 * "Qlora Expert", Core Concept: the 16 levels sit at quantiles of N(0,1).
 * Construction: 8 positive levels at the normal quantiles of the
 * probabilities delta - i*(delta-1/2)/8 (i = 0..7), 7 negative levels at the
 * negated quantiles of delta - i*(delta-1/2)/7 (i = 0..6), and 0, divided by
 * the largest, with delta = 1 - (1/32 + 1/30)/2; computed in double, rounded
 * once to float.  thresholds[j] = float((double(L[j]) + double(L[j+1])) / 2).
 * levels: 16 floats, ascending (L[0] = -1, L[7] = 0, L[15] = 1).
 * Either pointer may be NULL.  Returns 0.
 */
int nf4_codebook(float levels[16], float thresholds[15]);

/*
 * nf4_quantize -- NF4 block quantization + double quantization (device).
 *
 * "Qlora Expert", Core Concept (NF4; DQ of the per-block fp32 constants to
 * 8 bit); "QLoRA Implementation Details", NF4 Math (blocks of 64 values);
 * "QLoRA: The 4-bit Revolution", section 2 (scaling factors 32 -> 8 bit).
 * For each block of 64 consecutive elements of the flattened weight
 * (the last block may be shorter):
 *   c = max |w|;  n = w / c (IEEE fp32 division; n = 0 if c = 0);
 *   code = number of thresholds t_j with n > t_j (nearest level, ties low).
 * For each group of 256 consecutive blocks (the last may be shorter):
 *   s = max c;  d = s / 255 (fp32; d = 0 if s = 0);
 *   qabs = min(255, rint_half_even(c / d)) (0 if s = 0).
 * w       : device, rows*cols floats, 16-byte aligned.
 * out     : host struct; its device buffers receive packed, qabs, gscale
 *           (rows and cols give the element count).
 * status_dev : device int32 or NULL.  If any weight is non-finite the
 *           kernel stores QN_ENONFINITE there and the outputs are undefined;
 *           otherwise it is left untouched (clear it before the call).
 * Errors: QN_EINVAL (null pointer, rows or cols <= 0, misalignment),
 *         QN_EHIP.
 */
int nf4_quantize(const float* w, const nf4_tensor* out, int32_t* status_dev,
                 void* stream);

/*
 * nf4_dequantize -- NF4 + DQ weight to bf16 (device).
 *
 * "QLORA ... paper summary", Notes: load the 4-bit weights and dequantize
 * to BF16; "QLoRA Guide", Forward pass: dequantize to BF16 on the fly.
 * w_bf16 : device, rows*cols uint16 (bf16 bits), 16-byte aligned, the
 *          row-major dequantized weight (formula at nf4_tensor).
 * Errors: QN_EINVAL, QN_EHIP.
 */
int nf4_dequantize(const nf4_tensor* w, uint16_t* w_bf16, void* stream);

/*
 * nf4_dequantize_batch -- the same for several weights in one launch.
 *
 * Same operation as nf4_dequantize (pages and formula above), for all the
 * projections of a layer at once: their whole 2048-weight spans form one
 * work list, so the pass runs as one kernel instead of count kernels.
 * w      : host array of count tensors (device buffers, as nf4_dequantize).
 * w_bf16 : host array of count device pointers, each rows*cols uint16,
 *          16-byte aligned.  The outputs must not overlap.
 * count  : 1 .. QN_DEQUANT_BATCH_MAX.
 * Errors: QN_EINVAL (count out of range, or any tensor / output invalid as
 *         for nf4_dequantize; nothing is launched then), QN_EHIP.
 */
#define QN_DEQUANT_BATCH_MAX 16
int nf4_dequantize_batch(const nf4_tensor* w, uint16_t* const* w_bf16,
                         int32_t count, void* stream);

/*
 * nf4_merge -- dequantize-and-merge: the dense bf16 weight with the adapter
 * folded in (device).
 *
 * "Qlora Expert", When to Use and Common Pitfalls: an adapter is merged into
 * a dense model by dequantizing the base, which materialises the full bf16
 * weight; "QLoRA Implementation Details (2025 Edition)", Step 7 (Merge &
 * Save); s = alpha / r as in the linear layer (Step 4).
 *   w_merged[n][k] = bf16_rne(W'[n][k] + s * sum_j B[n][j] A[j][k])
 * with W' the dequantized base (formula at nf4_tensor); the sum and the
 * addition are formed in fp32 (fused multiply-add), then rounded once.
 * w        : NF4 weight [N = rows, K = cols], K % 64 == 0.
 * A        : device, bf16 [r][K] row-major, 16-byte aligned.
 * B        : device, bf16 [N][r] row-major.
 * r, alpha : 1 <= r <= QN_MAX_RANK.
 * w_merged : device, bf16 [N][K] row-major, 16-byte aligned, written whole.
 * Errors: QN_EINVAL (null or misaligned pointer, r out of range,
 *         K % 64 != 0, operands of 2 GiB or more), QN_EHIP.
 */
int nf4_merge(const nf4_tensor* w, const uint16_t* A, const uint16_t* B,
              int32_t r, float alpha, uint16_t* w_merged, void* stream);

/*
 * Codec variants -- other 4-bit tables and other storage of the block
 * constants, for quantization-error comparisons.
 *
 * "Qlora Expert", Hyperparameter Guidance: quant type "fp4" exists beside
 * "nf4", and double quantization can be switched off; Memory Math prices the
 * constants at 0.5 bit per weight without it.  "QLoRA Guide", NF4 vs uniform
 * INT4; "QLoRA Implementation Details", Step 1 NF4 Math (the signed 4-bit
 * range [-8, 7]).  The pages define none of these, so each keeps NF4's
 * block scheme (absmax per 64 weights, one IEEE division, the number of
 * fp32 midpoint thresholds strictly below w/absmax, ties to the lower code,
 * two codes per byte) and swaps only the sorted 16-level table:
 *   QN_CODE_NF4  : the NF4 levels of nf4_codebook();
 *   QN_CODE_FP4  : the 16 values of the 4-bit float E2M1 (+-{0, 0.5, 1, 1.5,
 *                  2, 3, 4, 6}) divided by 6, both zeros as +0 (codes 7, 8);
 *   QN_CODE_INT4 : the integers -8..7 divided by 7 (code 0 is never chosen).
 * The stored code is the index into the sorted table.  Block constants:
 *   QN_CONST_DQ8      : as nf4_tensor (unsigned 8-bit code, fp32 scale per
 *                       group of 256): c' = fp32(q) * d;
 *   QN_CONST_FP32     : the fp32 absmax itself, c' = c (4.5 bits/weight);
 *   QN_CONST_CENTERED : per group of 256, mu = fp32 pairwise sum of the
 *                       constants (adjacent pairs, level by level, padded
 *                       with zeros to 256) / count; d = max|c - mu| / 127;
 *                       q = clamp(rint_even((c - mu) / d), -127, 127) as
 *                       int8 (d = q = 0 when every c equals mu);
 *                       c' = fp32(fp32(q * d) + mu), no fused multiply-add.
 * Dequantized value: bf16_rne(fp32(L[code] * c')).  QN_CODE_NF4 with
 * QN_CONST_DQ8 is exactly nf4_quantize / nf4_dequantize.
 */
#define QN_CODE_NF4 0
#define QN_CODE_FP4 1
#define QN_CODE_INT4 2
#define QN_CONST_DQ8 0
#define QN_CONST_FP32 1
#define QN_CONST_CENTERED 2

/*
 * A weight of rows x cols elements in one of the variant formats:
 *   packed : device, ceil(numel/2) bytes, 16-byte aligned; layout as in
 *            nf4_tensor; an odd tail nibble is the code of a zero weight.
 *   consts : device, nb = ceil(numel/64) entries: uint8 (QN_CONST_DQ8),
 *            float (QN_CONST_FP32, 4-byte aligned) or int8
 *            (QN_CONST_CENTERED).
 *   gscale : device, ng = ceil(nb/256) floats (DQ8, CENTERED; else unused).
 *   gmean  : device, ng floats (CENTERED; else unused).
 *   code   : QN_CODE_*;  consts_mode: QN_CONST_*.
 */
typedef struct {
  uint8_t* packed;
  void* consts;
  float* gscale;
  float* gmean;
  int64_t rows, cols;
  int32_t code;
  int32_t consts_mode;
} qn_qtensor;

/* qn_codebook -- the 16 sorted levels and 15 fp32 midpoint thresholds of a
 * QN_CODE_* table (host).  Errors: QN_EINVAL for an unknown table. */
int qn_codebook(int32_t code, float levels[16], float thresholds[15]);

/* qn_quantize -- quantize an fp32 weight w (device, numel floats, 16-byte
 * aligned) into `out` (device).  Non-finite weights set *status_dev to
 * QN_ENONFINITE as nf4_quantize does.  Errors: QN_EINVAL, QN_EHIP. */
int qn_quantize(const float* w, const qn_qtensor* out, int32_t* status_dev,
                void* stream);

/* qn_dequantize -- bf16 copy of a variant-format weight (device, numel
 * bf16, 16-byte aligned).  Errors: QN_EINVAL, QN_EHIP. */
int qn_dequantize(const qn_qtensor* w, uint16_t* w_bf16, void* stream);

/*
 * 8-bit AdamW on the adapters -- "Qlora Expert", Core Concept item 3 (paged
 * optimizers keep the Adam moments in memory paged between GPU and CPU)
 * and Hyperparameter Guidance (paged_adamw_8bit); "QLoRA Implementation
 * Details (2025 Edition)", Step 5 (states in CPU RAM, paged in and out);
 * "QLORA ... paper summary", Notes (adapters stored and trained in BF16).
 * The pages give no state format; the one used:
 *   - blocks of QN_ADAMW_BLOCK consecutive elements; per block m is stored
 *     as OCP FP8 E4M3 codes of m / s_m and the second moment as E4M3 codes
 *     of sqrt(v) / s_r, s = fp32(block absmax / 448) (0 and codes 0 for a
 *     zero block); a fresh state is all zero bytes;
 *   - E4M3 encoding clamps the magnitude to 448 and rounds to nearest
 *     even; a value that rounds to zero is code 0.
 * Step t (1-based), per element, in fp32 in this order with no fused
 * multiply-add, host constants rounded once from double (c1 = 1-beta1,
 * c2 = 1-beta2, bc1 = 1/(1-beta1^t), bc2 = 1/(1-beta2^t),
 * decay = 1 - lr*weight_decay):
 *   g = g*grad_scale;  m = beta1*m' + c1*g;  v = beta2*v' + c2*(g*g)
 *   p = bf16_rne(p*decay - lr*((m*bc1) / (sqrt(v*bc2) + eps)))
 * (AdamW with decoupled weight decay), with m', v' = r'^2 decoded from the
 * stored state; then m and sqrt(v) are re-encoded.  grad_scale carries
 * gradient clipping (the caller's min(1, max_norm/||g||)).  Gradients must
 * be finite.
 */
#define QN_ADAMW_BLOCK 256

typedef struct {
  double lr, beta1, beta2, eps, weight_decay, grad_scale;
} qn_adamw_hparams;

/* State of n parameters: m_codes, r_codes: n bytes each (4-byte aligned);
 * m_scale, r_scale: ceil(n/256) floats each. */
typedef struct {
  uint8_t* m_codes;
  float* m_scale;
  uint8_t* r_codes;
  float* r_scale;
} qn_adamw8_state;

/* qn_adamw8_step -- one step with the state in device memory.
 * p : device bf16 [n], updated in place, 8-byte aligned;
 * g : device fp32 [n], 16-byte aligned;  st: device state;
 * hp: host; step >= 1; 0 <= beta < 1, eps > 0.
 * Errors: QN_EINVAL, QN_EHIP. */
int qn_adamw8_step(uint16_t* p, const float* g, int64_t n,
                   const qn_adamw8_state* st, const qn_adamw_hparams* hp,
                   int64_t step, void* stream);

/* qn_adamw8_staging_bytes -- device staging the paged step needs for pages
 * of `chunk` elements (a positive multiple of QN_ADAMW_BLOCK); 0 if chunk
 * is invalid. */
size_t qn_adamw8_staging_bytes(int64_t chunk);

/* qn_adamw8_paged_step -- the same step with the state in host memory
 * (pinned, from hipHostMalloc, for the copies to be asynchronous).  The
 * state is paged through the caller's device `staging` buffer in pages of
 * `chunk` elements, two pages in flight: page i is copied in on
 * `h2d_stream`, stepped on `stream`, and copied back on `d2h_stream`, so the
 * copies of one page overlap the step of the next.  Null copy streams mean
 * `stream`.  All work is ordered after what `stream` held at the call, and
 * `stream` reaches the end of the call only after the last page is back in
 * host memory.  The copy streams must have the default priority.
 * Errors: QN_EINVAL, QN_EWORKSPACE (staging smaller than
 * qn_adamw8_staging_bytes(chunk)), both before anything is queued; QN_EHIP,
 * possibly after some pages were queued: then `stream` still waits for
 * every copy already queued (or, if that cannot be arranged, the copy
 * streams are drained before the call returns), so the host state and the
 * staging buffer are free once `stream` gets past the call, but the state
 * may hold a mix of stepped and unstepped pages. */
int qn_adamw8_paged_step(uint16_t* p, const float* g, int64_t n,
                         const qn_adamw8_state* host_st, void* staging,
                         size_t staging_bytes, int64_t chunk,
                         const qn_adamw_hparams* hp, int64_t step,
                         void* stream, void* h2d_stream, void* d2h_stream);

/*
 * qlora_workspace_bytes -- device workspace a fused call needs (host).
 * which: QN_FWD, QN_BWD or QN_FWD_DROPOUT.  Returns 0 for invalid
 * arguments.
 */
size_t qlora_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t r,
                             int32_t which);

/*
 * qlora_linear_fwd -- fused QLoRA linear forward (device).
 *
 * "QLoRA Guide", How QLoRA Works / Forward pass: the dequantized frozen W
 * times x is summed with the adapter branch B(A(x)); "QLoRA Implementation
 * Details", Step 4: the branch is scaled by alpha/r.  With s = alpha / r:
 *   T = X A^T            (fp32, written to t_save)
 *   Y = X W'^T + s T B^T (fp32 accumulation)
 * W' is dequantized inside the kernel and never written to memory.
 * x      : device bf16 [M, K];  w: NF4 tensor with rows = N, cols = K;
 * A      : device bf16 [r, K];  B: device bf16 [N, r];  1 <= r <= 256;
 * y      : device [M, N] of y_dtype (QN_F32 or QN_BF16);
 * t_save : device fp32 [M, r], T for the backward;
 * ws     : device workspace of ws_bytes >= qlora_workspace_bytes(M, N, K,
 *          r, QN_FWD), 16-byte aligned (holds the bf16 hi/lo parts of s T,
 *          B padded to a multiple of 16 columns and, when the GEMM's last
 *          wave of 256 x 256 output tiles is ragged, one fp32 partial tile
 *          per tile of that wave); calls that run at the same time need
 *          workspaces of their own.  Status word: when M > 16 (the general
 *          path), the first int32 of ws is zeroed by the call and set to
 *          QN_ESYNC if a tile of the ragged last wave was split in two and
 *          its second piece waited in vain for the first piece's partial
 *          sum; that tile of y is then NaN.  Read it after the stream has
 *          reached the call's end.
 * Requires K % 64 == 0 (blocks never straddle rows), N % 8 == 0 (16-byte
 * aligned rows), M, N >= 1, every operand smaller than 2 GiB, and all
 * matrix pointers 16-byte aligned.
 * Errors: QN_EINVAL, QN_EWORKSPACE, QN_EHIP.
 */
int qlora_linear_fwd(const uint16_t* x, int64_t M, const nf4_tensor* w,
                     const uint16_t* A, const uint16_t* B, int32_t r,
                     float alpha, void* y, int32_t y_dtype, float* t_save,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * qlora_linear_bwd -- fused QLoRA linear backward (device).
 *
 * "QLoRA Guide", Forward pass: only A and B receive gradients, the
 * dequantized W is treated as a constant; "QLORA ... paper summary", Notes:
 * gradients only for the LoRA adapters.  With s = alpha / r and G = dY B:
 *   dX = dY W' + s G A   (output dtype dx_dtype)
 *   dA = s G^T X         (fp32 [r, K])
 *   dB = s dY^T T        (fp32 [N, r])
 * No gradient is formed for the frozen base.
 * dy     : device bf16 [M, N];  x: device bf16 [M, K];
 * t_saved: device fp32 [M, r] from qlora_linear_fwd;
 * dx     : device [M, K] of dx_dtype;  dA, dB: device fp32 outputs;
 * ws     : device workspace, ws_bytes >= qlora_workspace_bytes(M, N, K, r,
 *          QN_BWD) (the transposed and padded adapter operands, the rank-r
 *          partial sums and, when the dX GEMM's last wave of 256 x 256 tiles
 *          is ragged, one fp32 partial tile per tile of that wave).  The
 *          first int32 of ws is a status word as in qlora_linear_fwd (for
 *          every M), about the dX tiles.
 * Same shape and alignment rules as qlora_linear_fwd.
 * Errors: QN_EINVAL, QN_EWORKSPACE, QN_EHIP.
 */
int qlora_linear_bwd(const uint16_t* dy, const uint16_t* x, int64_t M,
                     const nf4_tensor* w, const uint16_t* A,
                     const uint16_t* B, int32_t r, float alpha,
                     const float* t_saved, void* dx, int32_t dx_dtype,
                     float* dA, float* dB, void* ws, size_t ws_bytes,
                     void* stream);

/*
 * LoRA dropout -- qlora_linear_fwd / qlora_linear_bwd with dropout on the
 * adapter branch input.  The pages carry lora_dropout (0.05 in "Qlora
 * Expert", Core Concept code and "QLoRA Guide", Example; 0.1 in "QLoRA
 * Implementation Details (2025 Edition)", Step 4) next to r and
 * lora_alpha.  Inverted dropout on X before A, the same mask in the
 * backward:
 *   X_d = X * mask / (1 - p)  (kept: bf16_rne(fp32(x) * fp32(1/(1-p))))
 *   T = X_d A^T;  Y = X W'^T + s T B^T
 *   dX = dY W' + s (G A) * mask / (1 - p);  dA = s G^T X_d;  dB = s dY^T T
 * The mask is counter-based, so the backward regenerates it: element
 * (m, k) of X is kept when word m % 4 of Philox4x32-10 (Salmon et al.,
 * "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011) at counter
 * (k, m / 4, 0, 0) under key (seed mod 2^32, seed / 2^32) is at least
 * floor(p * 2^32).  Use one seed per layer and step; the forward and
 * backward of one step must get the same p and seed.  p == 0 is the layer
 * without dropout.  The forward's workspace is qlora_workspace_bytes(...,
 * QN_FWD_DROPOUT) (the general path for every M); the backward's is
 * QN_BWD.  Arguments otherwise as qlora_linear_fwd / qlora_linear_bwd.
 * Errors: as those, and QN_EINVAL for a null drop or p outside [0, 1).
 */
typedef struct {
  double p;
  uint64_t seed;
} qn_dropout;

int qlora_linear_fwd_dropout(const uint16_t* x, int64_t M,
                             const nf4_tensor* w, const uint16_t* A,
                             const uint16_t* B, int32_t r, float alpha,
                             void* y, int32_t y_dtype, float* t_save,
                             const qn_dropout* drop, void* ws,
                             size_t ws_bytes, void* stream);

int qlora_linear_bwd_dropout(const uint16_t* dy, const uint16_t* x,
                             int64_t M, const nf4_tensor* w,
                             const uint16_t* A, const uint16_t* B, int32_t r,
                             float alpha, const float* t_saved, void* dx,
                             int32_t dx_dtype, float* dA, float* dB,
                             const qn_dropout* drop, void* ws,
                             size_t ws_bytes, void* stream);

/*
 * qlora_linear_fwd_batch -- qlora_linear_fwd for up to QN_FWD_BATCH_MAX
 * projections with few tokens (M <= 16 each), as one pair of launches
 * (device).
 *
 * "QLoRA Guide", How QLoRA Works / Forward pass, for each job: T = X A^T
 * (fp32, to t_save) and Y = X W'^T + (alpha / r) T B^T; decoding through a
 * QLoRA model runs every projection of a layer at a handful of tokens,
 * where the pass is bound by streaming the 4-bit weights.  The kernels are
 * those of qlora_linear_fwd at M <= 16; the split of each reduction into K
 * slices (and with it the order of the fp32 sums) is chosen for the whole
 * batch, so a job agrees with its single call up to fp32 rounding, and a
 * batch of one gives qlora_linear_fwd's bits.  Jobs are independent: each has its
 * own x, weight, adapters and outputs, and no output may overlap another
 * job's inputs or outputs.  The work of all jobs is dealt to the CUs as one
 * list, so small projections (the k / v of grouped-query attention) do
 * not leave the GPU idle and a layer costs two launches, not two per
 * projection.
 * jobs : host array of `count` descriptors (1 <= count <= QN_FWD_BATCH_MAX),
 *        fields as the qlora_linear_fwd arguments of the same names;
 *        1 <= M <= 16 for every job.
 * ws   : device workspace, ws_bytes >= qlora_fwd_batch_workspace_bytes(jobs,
 *        count) (fp32 K-slice partial sums of every job), 16-byte aligned.
 * Errors: QN_EINVAL (a job qlora_linear_fwd would reject, M > 16, count out
 * of range), QN_EWORKSPACE, QN_EHIP.
 */
#define QN_FWD_BATCH_MAX 8

typedef struct {
  const uint16_t* x;      /* device bf16 [M, K] */
  int64_t M;              /* 1 .. 16 */
  const nf4_tensor* w;    /* host descriptor: rows = N, cols = K */
  const uint16_t* A;      /* device bf16 [r, K] */
  const uint16_t* B;      /* device bf16 [N, r] */
  int32_t r;
  float alpha;
  void* y;                /* device [M, N] of y_dtype */
  int32_t y_dtype;        /* QN_F32 or QN_BF16 */
  float* t_save;          /* device fp32 [M, r] */
} qlora_fwd_job;

/* Workspace for qlora_linear_fwd_batch (host); 0 for an invalid batch. */
size_t qlora_fwd_batch_workspace_bytes(const qlora_fwd_job* jobs,
                                       int32_t count);

int qlora_linear_fwd_batch(const qlora_fwd_job* jobs, int32_t count,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * qlora_linear_fwd_noalloc -- qlora_linear_fwd without a workspace argument
 * (device), for callers that cannot allocate device memory: code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * allocation.  It computes exactly what qlora_linear_fwd computes, with the
 * same kernels, and calls no allocating routine.
 *
 * Its workspace is a file-scope device array of QN_NOALLOC_SCRATCH_BYTES
 * (32 MiB) inside the library, one copy per GPU, held until the process
 * ends; its device address is looked up once per GPU on the first call
 * made with that GPU current (`stream` must belong to the current device).
 * Every call on a GPU uses the same array, so calls that overlap on one
 * GPU (different streams, or different host threads) race: serialize them.
 * The GEMM does not split a ragged last wave here (no room is kept for
 * partial tiles), so results can differ from qlora_linear_fwd's in the fp32
 * summation order of such tiles; with no split planned they are identical.
 * The first int32 of the array is the status word described under
 * qlora_linear_fwd.
 * Arguments as qlora_linear_fwd without ws / ws_bytes.
 * Errors: QN_EINVAL, QN_EWORKSPACE (the shape's workspace exceeds
 * QN_NOALLOC_SCRATCH_BYTES), QN_EHIP.
 */
#define QN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

int qlora_linear_fwd_noalloc(const uint16_t* x, int64_t M,
                             const nf4_tensor* w, const uint16_t* A,
                             const uint16_t* B, int32_t r, float alpha,
                             void* y, int32_t y_dtype, float* t_save,
                             void* stream);

/* qn_strerror -- static text for a QN_* code (host). */
const char* qn_strerror(int code);

/*
 * qn_profile_kernel -- measurement hook (host), for benchmarks; active only
 * in the profiling build of the library (compiled with QN_PROFILE_HOOK:
 * libqlora_nf4_prof.so).  The default build keeps no state for it and
 * returns QN_EINVAL.
 *
 * Arms per-launch timing of one internal kernel: each later launch of the
 * kernel called `name` (e.g. "k_fwd_gemm", "k_bwd_dx_gemm", "k_dequant")
 * records ev_start[i] on its stream right before the launch and ev_stop[i]
 * right after, for i = 0, 1, ... up to `capacity` launches.  ev_start and
 * ev_stop are host arrays of hipEvent_t (as void*) created by the caller and
 * must stay valid while armed.  name == NULL disarms.  Returns the number of
 * launches recorded since the last arming (>= 0), or QN_EINVAL.  In the
 * profiling build the armed state is process-global and not thread-safe:
 * arm it from one thread while no other thread calls the library.
 */
int qn_profile_kernel(const char* name, void** ev_start, void** ev_stop,
                      int32_t capacity);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_NF4_H */
