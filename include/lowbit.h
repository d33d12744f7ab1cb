/*
 * lowbit.h - C ABI of the MI355X low-bit linear layer
 *
 *     y = s_w * s_x * (Q(W) . Q8(x))
 *
 * following the operator statement of "M8.8 - Native Binary and Ternary
 * Transformers" (sections 0x02C-0x02D, 0x05A-0x05D and the reference decoder
 * of 0x09C): latent weights become packed 1-, 2- or 4-bit codes with fp32
 * scales, activations become int8 codes with one fp32 scale per token, the
 * product is accumulated exactly in int32, and an fp32 epilogue rescales it.
 *
 * Conventions
 *  - W is [n, k] (k contiguous) before packing; x and q are [t, k], y is
 *    [t, n], all row-major.
 *  - Host pointers are plain CPU memory.  Device pointers are HIP device
 *    memory on the current device (e.g. torch tensor data pointers).
 *  - The caller owns every buffer; the library allocates nothing.  Its only
 *    state is a per-device cache of the compute-unit count, filled on first
 *    use; all entry points are reentrant and thread-safe.
 *  - Device calls are asynchronous on `hip_stream` (a hipStream_t, NULL = the
 *    null stream); their outputs are valid once the stream has synchronised.
 *  - No entry point reads device memory on the host.  Argument checks are
 *    synchronous and happen before any launch; a rejected call launches
 *    nothing.  No exception crosses this interface.
 *
 * Packed weight layout.  The code alphabets and their widths follow the pages;
 * the arrangement of the fields is this library's own (M8.8 section 0x07D
 * leaves the physical representation of a ternary matrix open), chosen so
 * that one 16-row tile of one k-step is a single contiguous block that a
 * wavefront reads with one 16-byte load per lane.
 *  - Fields.  LOWBIT_BINARY1: one bit per code, bit = (1 - s) / 2 (the binary
 *    export reference of M8.8 section 0x06E).  LOWBIT_TERNARY2: 2-bit two's
 *    complement, +1 = 01, 0 = 00, -1 = 11, 10 reserved (two physical bits per
 *    ternary code, M8.8 section 0x01A; four codes per byte).  LOWBIT_INT4:
 *    4-bit two's complement for the symmetric levels -7..+7 of the T4NT model
 *    card, 1000 reserved.
 *  - Words.  A little-endian 32-bit word holds CPW codes (ternary 16, int4 8,
 *    binary 32).  Ternary code j sits in byte j % 4 at bit 2 * (j / 4); int4
 *    code j in byte j % 4, low nibble for j < 4; binary code j in byte j / 8
 *    at bit j % 8 (little-bit-first, as numpy.packbits(bitorder="little")).
 *  - Blocks.  KB consecutive k (ternary and int4 64, binary 128) split into
 *    four quarters; quarter g is "lane group" g's, held as WB words (ternary
 *    1, int4 2, binary 1) of consecutive codes.
 *  - Steps.  wpl words per (lane group, row) = wpl / WB consecutive blocks =
 *    step_k = 4 * wpl * CPW consecutive k.  wpl is the widest of 4, 2, 1
 *    (int4: 4, 2) whose step pads k no further than the narrowest step does.
 *  - Tiles.  16 consecutive rows.
 *  - Order.  Word w of (tile t, step s, lane group g, row r of the tile) is at
 *    byte ((((t * n_steps + s) * 4 + g) * 16 + r) * wpl + w) * 4; it covers
 *    block w / WB of the step, codes (w % WB) * CPW onwards of quarter g.
 *  - Padding.  Rows n.. of the last tile and codes k.. are zero fields.
 *    packed_bytes = ceil(n / 16) * n_steps * 256 * wpl.
 * Scales are fp32 arrays: [1] (tensor), [n] (row), or, for groups of `group`
 * consecutive columns (the last one possibly shorter), tiled like the codes:
 * scale (row r, group j) at ((r / 16) * n_groups + j) * 16 + r % 16, padding
 * rows zero, n_scales = ceil(n / 16) * 16 * n_groups.
 */
#ifndef LOWBIT_H
#define LOWBIT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lowbit_status {
    LOWBIT_OK = 0,
    LOWBIT_E_ARG = 1,        /* null pointer, bad size, unknown enum, inconsistent descriptor */
    LOWBIT_E_RANGE = 2,      /* the int32 accumulator could overflow for this k */
    LOWBIT_E_NONFINITE = 3,  /* lowbit_pack: a latent weight is NaN or infinite */
    LOWBIT_E_FORMAT = 4,     /* reserved for packed-data format errors */
    LOWBIT_E_HIP = 5         /* a HIP launch failed (hipGetLastError) */
} lowbit_status;

typedef enum lowbit_format {
    LOWBIT_TERNARY2 = 0,     /* {-1, 0, +1} */
    LOWBIT_BINARY1 = 1,      /* {-1, +1} */
    LOWBIT_INT4 = 2          /* -7..+7 */
} lowbit_format;

typedef enum lowbit_scale {
    LOWBIT_SCALE_TENSOR = 0, /* one scale for all of W */
    LOWBIT_SCALE_ROW = 1,    /* one scale per output row */
    LOWBIT_SCALE_GROUP = 2   /* one scale per (row, group of `group` columns) */
} lowbit_scale;

/* lowbit_desc.flags */
#define LOWBIT_FLAG_TANH3 1     /* lowbit_pack maps w -> 3 tanh(w / 3) first (T4NT soft clipping) */
#define LOWBIT_FLAG_CENTERED 2  /* binary only: code = +1 where w > mean of the scale domain, else -1
                                   (the original BitNet's centered sign, M8.8 0x02B) */

/* lowbit_act_quant *status bits */
#define LOWBIT_ACT_NONFINITE 1   /* some row held NaN or Inf */
#define LOWBIT_ACT_OVERFLOW 2    /* some row's 127 / max|x| overflowed fp32 */

/* Shape and size of one packed weight matrix.  Fill it with lowbit_describe;
 * every other call re-derives the size fields and rejects a mismatch. */
typedef struct lowbit_desc {
    int32_t format;          /* lowbit_format */
    int32_t scale;           /* lowbit_scale */
    int32_t n;               /* output rows, >= 1 */
    int32_t k;               /* input columns, >= 1 */
    int32_t group;           /* group mode: columns per group; else 0 */
    int32_t flags;           /* LOWBIT_FLAG_* */
    int32_t wpl;             /* packed words per (lane group, row) per k-step: 1, 2 or 4 */
    int32_t step_k;          /* codes per k-step: 4 * wpl * codes per word */
    int64_t n_steps;         /* ceil(k / step_k) */
    int64_t packed_bytes;    /* ceil(n / 16) * n_steps * 256 * wpl */
    int64_t n_groups;        /* ceil(k / group) in group mode, else 1 */
    int64_t n_scales;        /* 1, n, or ceil(n / 16) * 16 * n_groups */
} lowbit_desc;

/*
 * lowbit_describe - validate a weight shape and fill *out with its sizes.
 *   group: group mode needs a positive multiple of 64 (ternary, int4) or of
 *          128 (binary) - the k-extent of one matrix-core step of the kernels;
 *          it must be 0 otherwise.
 *   flags: LOWBIT_FLAG_TANH3, LOWBIT_FLAG_CENTERED (binary only), both or 0.
 * Errors: LOWBIT_E_ARG for any invalid field or a null `out`;
 *         LOWBIT_E_RANGE when k exceeds lowbit_max_k(format).
 */
lowbit_status lowbit_describe(int32_t format, int32_t scale, int32_t n, int32_t k,
                              int32_t group, int32_t flags, lowbit_desc* out);

/*
 * lowbit_pack - quantise latent fp32 weights and pack them (host, offline).
 *   w      host float [n, k]           latent weights
 *   packed host uint8  [packed_bytes]  out: codes in the tiled layout above
 *   scales host float  [n_scales]      out: fp32 scales (group scales tiled)
 * Per scale domain (M8.8 0x05A, 0x06E; T4NT model card):
 *   ternary: s = mean |w| (binary64 sum in ascending index order / count,
 *            rounded once to fp32); code = clip(rint(w / s), -1, 1) in fp32
 *            with ties to even; a zero domain gets s = 0 and codes 0.
 *   binary : s = mean |w| as above; code = +1 if w >= 0 (either zero) else -1;
 *            with LOWBIT_FLAG_CENTERED, code = +1 if w > a else -1 (a tie
 *            goes to -1), a = the domain's mean (binary64 sum in ascending
 *            index order / count, rounded once to fp32), compared in fp32.
 *   int4   : s = max |w| / 7 in fp32; code = clip(rint(w / s), -7, 7).
 *   LOWBIT_FLAG_TANH3 first maps w -> fp32(3 tanh(w / 3)) (binary64 tanh).
 * Runs on host threads; reads and writes host memory only.
 * Errors: LOWBIT_E_ARG (null pointer, bad descriptor), LOWBIT_E_NONFINITE
 * (a NaN or infinite weight; the outputs are then unspecified).
 */
lowbit_status lowbit_pack(const lowbit_desc* d, const float* w, uint8_t* packed, float* scales);

/*
 * lowbit_act_quant - per-token absmax int8 quantisation (M8.8 0x02C, 0x05C).
 *   x      device float [t, k]
 *   q      device int8  [t, k]   out: clip(rint(x * (127 / m)), -127, 127), fp32,
 *                                ties to even, m = max_k |x[row]|
 *   sx     device float [t]      out: m / 127 (fp32); 0 for an all-zero row
 *   status device int32 [1] or NULL: the kernel ORs LOWBIT_ACT_* bits into it
 *          (the caller clears it beforehand).  A row holding NaN/Inf, or whose
 *          127 / m overflows, gets zero codes and sx = NaN, so any output
 *          computed from it is visibly NaN.
 *   t, k   >= 1
 * Errors: LOWBIT_E_ARG, LOWBIT_E_HIP.
 */
lowbit_status lowbit_act_quant(const float* x, int32_t t, int32_t k, int8_t* q, float* sx,
                               int32_t* status, void* hip_stream);

/*
 * lowbit_act_quant_h4 - H-BitLinear's activation quantiser (M8.8 "Native
 * Binary and Ternary Transformers", 0x07C, BitNet v2): each token row is
 * rotated by the orthonormal Walsh-Hadamard transform (Sylvester order) over
 * consecutive blocks of B channels, B the largest power of two dividing k
 * (at most 2048), and the rotated row x' gets per-token absmax INT4 codes.
 *   x      device float [t, k], 16-byte aligned
 *   q      device int8  [t, k], 4-byte aligned   out: clip(rint(x' * (7 / m)),
 *                              -7, 7), fp32, ties to even, m = max_k |x'[row]|
 *   sx     device float [t]    out: m / 7 (fp32); 0 for an all-zero row
 *   status device int32 [1] or NULL: LOWBIT_ACT_* bits ORed in, as
 *          lowbit_act_quant; a row whose x' holds NaN/Inf, or whose 7 / m
 *          overflows, gets zero codes and sx = NaN.
 *   t >= 1; k a multiple of 64, at most 65536.
 * x' is computed as fp32 butterflies in increasing half-width (each pair
 * (a, c) -> (a + c, a - c)), then one multiply by fp32(1 / sqrt(B)), so the
 * codes are a deterministic function of x.  q and sx are the operands of
 * lowbit_linear / lowbit_linear_batched: y = s_w * sx * (Q(W) . q) is the
 * layer's output when W was trained (or rotated) in the transformed basis.
 * Errors: LOWBIT_E_ARG (null or misaligned pointer, t < 1, k not a multiple
 *         of 64), LOWBIT_E_RANGE (k > 65536), LOWBIT_E_HIP.
 */
lowbit_status lowbit_act_quant_h4(const float* x, int32_t t, int32_t k, int8_t* q, float* sx,
                                  int32_t* status, void* hip_stream);

/*
 * lowbit_act_quant_a4 - BitNet a4.8's 4-bit codes for the inputs of the
 * attention and FFN projections (M8.8 "Native Binary and Ternary
 * Transformers", 0x07B), the per-token absmax INT4 rule without a rotation:
 *   x      device float [t, k]
 *   q      device int8  [t, k]   out: clip(rint(x * (7 / m)), -7, 7), fp32,
 *                                ties to even, m = max_k |x[row]|
 *   sx     device float [t]      out: m / 7 (fp32); 0 for an all-zero row
 *   status device int32 [1] or NULL: LOWBIT_ACT_* bits ORed in; a row holding
 *          NaN / Inf, or whose 7 / m overflows, gets zero codes and sx = NaN.
 *   t >= 1, k >= 1.  q and sx are the operands of lowbit_linear /
 *   lowbit_linear_batched.
 * Errors: LOWBIT_E_ARG (null pointer, t < 1, k < 1), LOWBIT_E_HIP.
 */
lowbit_status lowbit_act_quant_a4(const float* x, int32_t t, int32_t k, int8_t* q, float* sx,
                                  int32_t* status, void* hip_stream);

/*
 * lowbit_act_quant_sparse8 - BitNet a4.8's sparse 8-bit codes for the
 * intermediate states in front of the attention output and FFN down
 * projections (M8.8 "Native Binary and Ternary Transformers", 0x07B): each
 * token row keeps its `keep` entries of largest |x| - at the threshold
 * magnitude the lower channels first - and the kept entries get the
 * per-token INT8 codes of lowbit_act_quant; the others get code 0.
 *   x      device float [t, k], 16-byte aligned
 *   keep   1 <= keep <= k: entries kept per row (keep = k is lowbit_act_quant)
 *   q      device int8  [t, k], 4-byte aligned   out: clip(rint(x * (127 / m)),
 *          -127, 127) where kept, else 0; m = max_k |x[row]|, always kept
 *   sx     device float [t]    out: m / 127 (fp32); 0 for an all-zero row
 *   status device int32 [1] or NULL: LOWBIT_ACT_* bits ORed in; a row holding
 *          NaN / Inf anywhere, or whose 127 / m overflows, gets zero codes and
 *          sx = NaN.
 *   t >= 1; k a multiple of 4, at most 32768.
 * The product of (q, sx) with packed weights is then the dense product over
 * the kept entries (lowbit_linear / lowbit_linear_batched).
 * Errors: LOWBIT_E_ARG (null or misaligned pointer, t < 1, k not a positive
 *         multiple of 4, keep outside [1, k]), LOWBIT_E_RANGE (k > 32768),
 *         LOWBIT_E_HIP.
 */
lowbit_status lowbit_act_quant_sparse8(const float* x, int32_t t, int32_t k, int32_t keep, int8_t* q, float* sx,
                                       int32_t* status, void* hip_stream);

/*
 * lowbit_act_quant_v1 - the original BitNet forward's activation codes (M8.8
 * "Native Binary and Ternary Transformers", 0x02C and the forward of 0x02E),
 * Q_b = 128, for the normalised input x (lowbit_layernorm):
 *   gamma  = max |x| over the token row (per_tensor = 0, the inference rule)
 *            or over all of x (per_tensor = 1, the training rule)
 *   q      = clip(rint((128 x) / (gamma + eps)), -128, 127): an exact
 *            multiply, then one IEEE fp32 division by fp32(gamma + eps),
 *            ties to even; a row with gamma = 0 gets zero codes
 *   sx     = gamma / 128 (fp32), so that lowbit_linear / lowbit_linear_batched
 *            on (q, sx) yield y = acc * s_w * gamma / 128, the forward's rescale
 *   x      device float [t, k]
 *   q      device int8  [t, k]  out        sx device float [t]  out
 *   eps    >= 0, finite (the forward's default is 1e-5)
 *   status device int32 [1] or NULL: LOWBIT_ACT_* bits ORed in.  A row holding
 *          NaN / Inf, or whose 128 gamma overflows fp32, gets zero codes and
 *          sx = NaN; with per_tensor = 1 such a value anywhere rejects every row.
 *   work   device uint32 [2], 4-byte aligned, required when per_tensor = 1
 *          (the tensor-wide max is reduced into it; its contents on entry do
 *          not matter), ignored otherwise.  Concurrent calls need their own.
 *   t >= 1; 1 <= k <= 262143: the codes reach -128, and the products' int32
 *   sums stay exact for k * 128 * 64 < 2^31 with binary or ternary weights
 *   (k <= 149796 with int4 weights).
 * Errors: LOWBIT_E_ARG (null or misaligned pointer, bad t / eps / per_tensor,
 *         per_tensor without work), LOWBIT_E_RANGE (k > 262143), LOWBIT_E_HIP.
 */
lowbit_status lowbit_act_quant_v1(const float* x, int32_t t, int32_t k, float eps, int32_t per_tensor, int8_t* q,
                                  float* sx, int32_t* status, uint32_t* work, void* hip_stream);

/*
 * lowbit_onebit_linear - OneBit's W1A16 projection (M8.8 "Native Binary and
 * Ternary Transformers", 0x06A): a sign matrix S, an FP16 input vector g and
 * an FP16 output vector h,
 *     y[t, n] = h[n] * sum_k S[n, k] * fp16(x[t, k] * g[k])
 * with fp16 products and fp32 sums on the matrix cores (the sum's order is
 * the kernel's: y differs from an exact evaluation by fp32 rounding only).
 * The layer's LayerNorm over n is lowbit_layernorm(y, t, n, ...) after it.
 *   d       a binary descriptor (LOWBIT_BINARY1, any scale mode; its scales
 *           are not used); packed from lowbit_pack: S = +1 where w >= 0
 *           (either zero), else -1
 *   packed  device uint8 [d->packed_bytes], 16-byte aligned
 *   g       device fp16 bits [k]      h  device fp16 bits [n]
 *   x       device fp16 bits [t, k]   (2-byte aligned)
 *   y       device float [t, n]       out
 *   t >= 1
 * Errors: LOWBIT_E_ARG (null or misaligned pointer, t < 1, a descriptor that
 *         is not binary or does not check out), LOWBIT_E_HIP.
 */
lowbit_status lowbit_onebit_linear(const lowbit_desc* d, const uint8_t* packed, const uint16_t* g, const uint16_t* h,
                                   const uint16_t* x, int32_t t, float* y, void* hip_stream);

/*
 * lowbit_layernorm - the sub-layer LayerNorm ahead of the original BitNet's
 * quantiser (M8.8 0x02E, 0x03A): per row of t, out = (x - mean) /
 * sqrt(var + eps) [* g] [+ b], population variance, fp32 sums.
 *   x, out device float [t, d] (may be the same buffer); g, b device float [d]
 *   or NULL; 1 <= d, eps >= 0 finite.
 * Errors: LOWBIT_E_ARG, LOWBIT_E_HIP.
 */
lowbit_status lowbit_layernorm(const float* x, int32_t t, int32_t d, float eps, const float* g, const float* b,
                               float* out, void* hip_stream);

/*
 * lowbit_linear - decode-shaped product (GEMV), tuned for t <= 16 and correct
 * for any t (tokens are processed 16 at a time).
 *   d       descriptor of the packed matrix (from lowbit_describe)
 *   packed  device uint8 [packed_bytes]    from lowbit_pack
 *   scales  device float [n_scales]
 *   q, sx   device int8 [t, k], device float [t]   from lowbit_act_quant
 *   y       device float [t, n]  out:
 *             tensor/row: y = fp32(acc) * (sx[t] * s_w[n])
 *             group     : y = sx[t] * sum_g s_w[n, g] * fp32(acc[t, n, g])
 *   acc     device int32 [t, n, n_groups] or NULL: when given, the exact
 *           integer products sum_k q[t, k] * code[n, k] (per group in group
 *           mode) are written too.
 * Accumulation is exact in int32; y may differ from a sequential fp32
 * evaluation by rounding order only.
 * Errors: LOWBIT_E_ARG (null pointer, t < 1, descriptor mismatch),
 *         LOWBIT_E_RANGE (k > lowbit_max_k(format)), LOWBIT_E_HIP.
 */
lowbit_status lowbit_linear(const lowbit_desc* d, const uint8_t* packed, const float* scales,
                            const int8_t* q, const float* sx, int32_t t,
                            float* y, int32_t* acc, void* hip_stream);

/*
 * lowbit_linear_batched - prefill-shaped product (GEMM on the matrix cores),
 * tuned for large t and correct for any t.  Same arguments, outputs and
 * errors as lowbit_linear; the two produce identical acc.
 */
lowbit_status lowbit_linear_batched(const lowbit_desc* d, const uint8_t* packed, const float* scales,
                                    const int8_t* q, const float* sx, int32_t t,
                                    float* y, int32_t* acc, void* hip_stream);

/*
 * lowbit_linear_grouped - `count` independent decode products in as few
 * launches as possible (up to 256 matrices per launch), e.g. the projections
 * that read one input (q/k/v, gate/up) or any set of same-width layers whose
 * inputs are ready.  Each matrix i computes exactly what lowbit_linear
 * computes for (descs[i], packed[i], scales[i], q[i], sx[i], t, y[i], acc[i]).
 *   count   >= 1
 *   descs   host array [count]; all must share format, scale mode, group, flags
 *           and k (n may differ)
 *   packed, scales, q, sx, y: host arrays [count] of device pointers
 *   acc     host array [count] of device pointers (entries may be NULL), or NULL
 *   t       tokens per matrix, the same for all (>= 1; 16 per launch)
 * One persistent kernel streams every matrix's tiles back to back, so small
 * matrices share one launch's ramp-up instead of paying one each.
 * Errors: as lowbit_linear, plus LOWBIT_E_ARG when the descriptors disagree.
 */
lowbit_status lowbit_linear_grouped(int32_t count, const lowbit_desc* descs, const uint8_t* const* packed,
                                    const float* const* scales, const int8_t* const* q,
                                    const float* const* sx, int32_t t, float* const* y,
                                    int32_t* const* acc, void* hip_stream);

/*
 * lowbit_linear_batched_grouped - several independent prefill products
 * (lowbit_linear_batched each) of equal format, scale mode, group, flags and
 * k, and one token count t, in as few launches as the argument space allows
 * (at most 64 products per launch, the launches of near-equal size): product i reads q[i] [t, k], sx[i] [t] and writes y[i]
 * [t, n_i] (and acc[i] when acc and acc[i] are not NULL).  One launch fills
 * the chip with the output tiles of all its products, which small products
 * (n of a few hundred) cannot do alone.  Results equal those of the single
 * calls bit for bit.
 * Errors: as lowbit_linear_batched; LOWBIT_E_ARG when the descriptors differ
 *         in format, scale mode, group, flags or k.
 */
lowbit_status lowbit_linear_batched_grouped(int32_t count, const lowbit_desc* descs, const uint8_t* const* packed,
                                            const float* const* scales, const int8_t* const* q,
                                            const float* const* sx, int32_t t, float* const* y,
                                            int32_t* const* acc, void* hip_stream);

/*
 * lowbit_linear_fused - the decode product with the activation quantiser fused
 * into it (M8.8 "Native Binary and Ternary Transformers" 0x02C / 0x05C
 * quantiser, 0x02D product): what lowbit_act_quant(x, t, k, q, sx, status)
 * followed by lowbit_linear(d, packed, scales, q, sx, t, y, NULL) computes,
 * bit for bit, from fp32 x, in one call.  For one token (t = 1) with
 * k % 4 == 0, x 16-byte aligned and the row within the product's LDS stage,
 * every workgroup of the product quantises the row into its own stage (one
 * launch, the codes never read back; one workgroup per matrix still writes
 * q and sx).  Otherwise the quantiser kernel runs first and the product reads
 * its codes: redoing a row per workgroup costs more than that launch once
 * there are several token rows.
 *   x       device float [t, k]
 *   q, sx   device int8 [t, k], device float [t]   out (as lowbit_act_quant)
 *   status  device int32 [1] or NULL: LOWBIT_ACT_* bits ORed in, as lowbit_act_quant
 *   other arguments and y as lowbit_linear (no integer output)
 * Errors: as lowbit_linear.
 */
lowbit_status lowbit_linear_fused(const lowbit_desc* d, const uint8_t* packed, const float* scales,
                                  const float* x, int32_t t, int8_t* q, float* sx, float* y,
                                  int32_t* status, void* hip_stream);

/*
 * lowbit_linear_grouped_fused - lowbit_linear_grouped with the quantiser fused
 * as in lowbit_linear_fused: matrix i quantises x[i] (device float [t, k])
 * into q[i], sx[i] and computes y[i].  One status word for all matrices.
 * Where the quantiser does not run in the product's prologue, one quantiser
 * launch covers the inputs of up to 40 matrices before the products.
 * Errors: as lowbit_linear_grouped.
 */
lowbit_status lowbit_linear_grouped_fused(int32_t count, const lowbit_desc* descs, const uint8_t* const* packed,
                                          const float* const* scales, const float* const* x, int8_t* const* q,
                                          float* const* sx, int32_t t, float* const* y, int32_t* status,
                                          void* hip_stream);

/* ---------------------------------------------------------------------------
 * One decode step of a BitLinear decoder.
 *
 * The block is the LLaMA-like recipe of the b1.58 models (M8.8 "Native Binary
 * and Ternary Transformers", the b1.58 section): pre-norm RMSNorm, attention
 * with rotary position embeddings over a key/value cache, a SwiGLU FFN,
 * residual adds, a final RMSNorm and a head; every projection a BitLinear
 * (lowbit_linear_fused: per-token int8 codes of its input, exact integer
 * product, fp32 rescale).  Its shape follows the add/sub-only engine's
 * quick-start model (Atomic-1Bit README: 256-d, 6 layers, 4 heads, 4096
 * vocabulary, 128-token context, fp32 token embedding).
 *   RMSNorm(x; g) = x / sqrt(mean(x^2) + norm_eps) * g
 *   rotary: head dimension i < 32 paired with i + 32, angle pos * base^(-i/32)
 *   attention: per head, softmax over cached positions 0 .. pos of
 *              q . k_j / sqrt(64), output sum_j p_j v_j
 *   SwiGLU: a = SiLU(x W_gate) * (x W_up), SiLU(z) = z / (1 + e^-z)
 *   next token: argmax of the logits (lowest index among equal maxima)
 * ------------------------------------------------------------------------- */

#define LOWBIT_STEP_POSITION 1   /* position outside [0, context): nothing computed */
#define LOWBIT_STEP_TOKEN 2      /* token outside [0, vocab): clamped into it */

/* Projection slots of lowbit_model.proj and of the per-layer weight arrays. */
enum { LOWBIT_PROJ_QKV = 0, LOWBIT_PROJ_O = 1, LOWBIT_PROJ_GATE = 2, LOWBIT_PROJ_UP = 3, LOWBIT_PROJ_DOWN = 4,
       LOWBIT_PROJ_HEAD = 5 };

typedef struct lowbit_model {
    int32_t d_model;         /* n_heads * 64 (head dimension 64), <= 4096 */
    int32_t n_layers;        /* >= 1 */
    int32_t n_heads;         /* >= 1 */
    int32_t d_ff;            /* FFN width, >= 1 */
    int32_t vocab;           /* >= 1 */
    int32_t context;         /* positions the caches hold, 1 .. 8192 */
    float norm_eps;          /* RMSNorm epsilon, >= 0 */
    float rope_base;         /* rotary base, > 0 */
    /* shapes of every layer's projections and of the head: qkv [3 d_model,
     * d_model] (rows: q, k, v), o [d_model, d_model], gate and up [d_ff,
     * d_model], down [d_model, d_ff], head [vocab, d_model]; any format and
     * scale mode (lowbit_describe) */
    lowbit_desc proj[6];
    const float* embed;               /* device [vocab, d_model] fp32 */
    const float* norms;               /* device [2 n_layers + 1, d_model]: attention, FFN gain per layer, then final */
    const uint8_t* const* packed;     /* host array [5 n_layers + 1] of device pointers: per layer qkv, o, gate,
                                         up, down; then the head (lowbit_pack output, 16-byte aligned) */
    const float* const* scales;       /* host array, same indexing */
    float* k_cache;                   /* device [n_layers, context, d_model] fp32 (rotated keys), 16-byte aligned */
    float* v_cache;                   /* device [n_layers, context, d_model] fp32 */
    void* work;                       /* device workspace, lowbit_model_work_bytes() bytes, 16-byte aligned */
} lowbit_model;

/* The step's building blocks on their own (the same kernels).
 *
 * lowbit_rmsnorm - per row of t: v = x + r (r NULL: v = x), x_out = v (when
 *   not NULL; may equal x), h = v / sqrt(mean(v^2) + eps) * g.  fp32 sums.
 *   x, r, x_out, h device float [t, d]; g device float [d]; 1 <= d <= 4096.
 * lowbit_rope_attention - one layer's attention for one token at position
 *   pos (0 <= pos < context <= 8192): the query and key of qkv (device
 *   float [3 * 64 * n_heads]: q, k, v blocks) rotated by pos, key and value
 *   stored at row pos of k_cache / v_cache (device float [context, 64 *
 *   n_heads]; k_cache 16-byte aligned), attn (device float [64 * n_heads]) =
 *   per-head softmax attention over rows 0 .. pos.  Rows above pos are not
 *   read.
 * lowbit_swiglu - a = SiLU(gate) * up elementwise, n >= 1 elements.
 * Errors: LOWBIT_E_ARG for null / misaligned pointers or sizes out of range;
 *         LOWBIT_E_HIP. */
lowbit_status lowbit_rmsnorm(const float* x, const float* r, float* x_out, const float* g, int32_t t, int32_t d,
                             float eps, float* h, void* hip_stream);
lowbit_status lowbit_rope_attention(const float* qkv, int32_t n_heads, int32_t pos, int32_t context, float rope_base,
                                    float* k_cache, float* v_cache, float* attn, void* hip_stream);
lowbit_status lowbit_swiglu(const float* gate, const float* up, int64_t n, float* a, void* hip_stream);

/* Bytes of lowbit_model.work for this model (the intermediates of one step),
 * or -1 when the model's sizes are invalid. */
int64_t lowbit_model_work_bytes(const lowbit_model* m);

/* 4-byte words of the optional trace buffer of lowbit_decode_step; -1 when
 * the model's sizes are invalid.  Two parts:
 *  - floats: x0 [d] (the embedding row), then per layer h [d], qkv [3d],
 *    q rotated [d], k rotated [d], attention output [d], o [d], x after
 *    attention [d], h2 [d], gate [ff], up [ff], SwiGLU output [ff], down [d],
 *    x after the FFN [d], and last the final norm's output [d]; padded with
 *    up to 3 unused floats to a multiple of 4;
 *  - code records, one per product in the order per layer qkv, o, gate, up,
 *    down, then the head: 16 bytes whose first float is the product's s_x,
 *    then its input's k int8 codes (k = d, or ff for down), padded with
 *    unused bytes to a multiple of 16.  These are the per-token codes
 *    (M8.8 0x02C) the product consumed, so a test can hold each BitLinear of
 *    the step against the oracle's codes and integer product of its own
 *    traced input. */
int64_t lowbit_model_trace_floats(const lowbit_model* m);

/*
 * lowbit_decode_step - one token through the model, on the device.
 *   state   device int32[4]: [0] the token (in), replaced by the greedy next
 *           token; [1] its position, advanced by one; [2] LOWBIT_ACT_* bits
 *           ORed in by the products (a rejected activation row); [3]
 *           LOWBIT_STEP_* bits ORed in.  Token and position are read on the
 *           device, so a captured graph of this call replays step after step.
 *           A position outside [0, context) leaves caches, state [0..1],
 *           tokens and trace untouched (logits are then unspecified).
 *   logits  device float [vocab], out
 *   tokens  device int32 [context] or NULL: tokens[pos + 1] = next token
 *           when pos + 1 < context
 *   trace   device float [lowbit_model_trace_floats(m)] or NULL (16-byte
 *           aligned): every intermediate of the step, for tests
 * The caches receive this position's rotated key and value per layer.  All
 * launches go to hip_stream in order; nothing is allocated.
 * Errors: LOWBIT_E_ARG (invalid model, descriptor shape mismatch, null or
 *         misaligned pointer), LOWBIT_E_RANGE, LOWBIT_E_HIP.
 */
lowbit_status lowbit_decode_step(const lowbit_model* m, int32_t* state, float* logits, int32_t* tokens,
                                 float* trace, void* hip_stream);

/* Bytes of the library-held workspace of lowbit_decode_step_noalloc, per GPU. */
#define LOWBIT_NOALLOC_WORK_BYTES (1 << 20)

/*
 * lowbit_decode_step_noalloc - lowbit_decode_step for callers that cannot
 *   allocate device memory (code under HIP graph capture, tight serving
 *   loops, harnesses that forbid allocation): the same step, the same
 *   kernels and the same results, but m->work is ignored (it may be NULL).
 *   The step's intermediates live instead in a static device array of
 *   LOWBIT_NOALLOC_WORK_BYTES that the library holds on each GPU it runs on
 *   until the process ends.  Every call on a GPU shares that GPU's array and
 *   it keeps the last call's contents (the step writes every intermediate
 *   before reading it, so nothing needs clearing): calls that overlap on one
 *   GPU (on different streams, or from several threads without ordering)
 *   race and must be serialised by the caller.  Nothing is allocated: the
 *   first call on a device looks up the array's device address there
 *   (hipGetSymbolAddress) and keeps it.
 * Errors: as lowbit_decode_step; LOWBIT_E_RANGE also when the model's
 *         lowbit_model_work_bytes exceeds LOWBIT_NOALLOC_WORK_BYTES (checked
 *         before any HIP call).
 */
lowbit_status lowbit_decode_step_noalloc(const lowbit_model* m, int32_t* state, float* logits, int32_t* tokens,
                                         float* trace, void* hip_stream);

/* Device ceilings for the roofline fractions (measurement utilities, not part
 * of the operator).  The published MI355X figures are 8 TB/s of HBM and 5.0
 * POPS of dense int8 matrix-core work; these calls measure what the device
 * reaches, so a product's rate can be read against both.
 *
 * lowbit_calib_read - every lane streams 16-byte words of src (device, 16-byte
 *   aligned, `bytes` a positive multiple of 16) once, non-temporally, and
 *   folds them into *sink (device uint32, a value of no meaning).  Time it with
 *   events: bytes / time is the read rate (HBM-sourced when the buffer is
 *   several times the 256 MB last-level cache).
 * lowbit_calib_mfma_i8 - two wavefronts per SIMD on every CU issue
 *   v_mfma_i32_32x32x32_i8 back to back (eight independent accumulators, no
 *   memory traffic) `iters` >= 1 times each; lowbit_calib_mfma_i8_ops(iters)
 *   is the number of int8 operations (2 per multiply-add) that launch does
 *   (-1 for iters < 1).  *sink as above.
 * Errors: LOWBIT_E_ARG (null / misaligned pointer, size), LOWBIT_E_HIP. */
lowbit_status lowbit_calib_read(const void* src, int64_t bytes, uint32_t* sink, void* hip_stream);
lowbit_status lowbit_calib_mfma_i8(int32_t iters, uint32_t* sink, void* hip_stream);
int64_t lowbit_calib_mfma_i8_ops(int32_t iters);

/* Largest k the kernels accept for a format.  The operator's own bound
 * (M8.8 0x09C) is k * 127 * qmax < 2^31; the kernels hold each code scaled
 * by 64 (ternary, binary) or 16 (int4) in int8 lanes, and activation codes
 * reach -128 (lowbit_act_quant_v1), so their int32 sums need
 * k * 128 * qmax * scale < 2^31: k <= 262143 (ternary, binary), 149796 (int4). */
int32_t lowbit_max_k(int32_t format);

const char* lowbit_status_string(lowbit_status s);

/* Text of the HIP error behind the calling thread's most recent LOWBIT_E_HIP
 * ("no error" if there was none).  The returned string is static. */
const char* lowbit_last_hip_error(void);

/* ABI version: bump on any incompatible change. */
int32_t lowbit_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LOWBIT_H */
