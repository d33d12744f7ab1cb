/*
 * oracle.c - CPU oracle for the low-bit linear layer.
 *
 * TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the bench's CPU
 * baseline are its only callers.  Plain scalar C, one loop per definition,
 * OpenMP only across independent rows/domains.  Built with
 * -O2 -ffp-contract=off and no fast-math, so every float operation below is a
 * single IEEE-754 binary32 (or binary64 where stated) operation rounded to
 * nearest-even, in the order written.
 *
 * Sources (cited by page title and section):
 *  [NBT]  "M8.8 - Native Binary and Ternary Transformers"
 *  [A1B]  Atomic-1Bit README ("Run language models using only addition and
 *         subtraction")
 *  [T4NT] "T4NT-0.5B" model card (Tanh 4-bit Neural Transformer)
 *
 * Readings taken where the pages leave a step open are marked READING.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads the parallel loops use from now on (n >= 1); a timing knob only. */
void orc_set_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------ layout */

/*
 * Packed layout.  The pages fix the code alphabets and their physical width -
 * [NBT] 0x06E: binary bit = (1 - s) / 2, packed little-bit-first; [NBT] 0x01A:
 * two physical bits per ternary code; [A1B]: four ternary codes per byte;
 * [T4NT]: 15 levels, i.e. 4-bit codes - and leave the arrangement of fields
 * to the implementation ([NBT] 0x07D: "not one universal physical
 * representation").  READING (this library's arrangement):
 *
 *  field  ternary: 2-bit two's complement (+1 = 01, 0 = 00, -1 = 11, 10 reserved)
 *         int4   : 4-bit two's complement (-7..+7, 1000 reserved)
 *         binary : 1 bit, (1 - s) / 2
 *  word   32 bits holding CPW codes (ternary 16, int4 8, binary 32):
 *         ternary code j in byte j%4 at bit 2*(j/4); int4 code j in byte j%4,
 *         low nibble if j < 4 else high; binary code j in byte j/8, bit j%8.
 *  block  KB consecutive k (ternary, int4 64; binary 128) split in four
 *         quarters of KB/4 codes, quarter g held by "lane group" g as WB
 *         words (ternary 1, int4 2, binary 1).
 *  step   wpl words per (lane group, row) = wpl/WB consecutive blocks,
 *         SK = 4 * wpl * CPW consecutive k.
 *  tile   16 consecutive rows.
 *  order  byte offset of word w of (tile t, step s, lane group g, row r of the
 *         tile): ((((t * n_steps + s) * 4 + g) * 16 + r) * wpl + w) * 4, where
 *         word w covers block w / WB, codes (w % WB) * CPW .. of the quarter.
 *  wpl    the largest of 4, 2, 1 (int4: 4, 2) whose step pads k no further
 *         than the smallest step does.
 *  padding rows n >= N of the last tile and codes k >= K are zero fields.
 */
static int fmt_ok(int fmt) { return fmt == ORC_TERNARY || fmt == ORC_BINARY || fmt == ORC_INT4; }
static int cpw_of(int fmt) { return fmt == ORC_TERNARY ? 16 : (fmt == ORC_INT4 ? 8 : 32); }
static int kb_of(int fmt) { return fmt == ORC_BINARY ? 128 : 64; }
static int field_bits(int fmt) { return fmt == ORC_TERNARY ? 2 : (fmt == ORC_INT4 ? 4 : 1); }

int orc_layout(int fmt, int64_t n, int64_t k, int* wpl, int64_t* n_steps, int64_t* step_k,
               int64_t* packed_bytes) {
    if (!fmt_ok(fmt) || n < 1 || k < 1) return ORC_E_ARG;
    const int wmin = fmt == ORC_INT4 ? 2 : 1;
    const int64_t sk_min = 4 * wmin * cpw_of(fmt);
    const int64_t padded_min = (k + sk_min - 1) / sk_min * sk_min;
    int w = 4;
    for (; w > wmin; w /= 2) {
        const int64_t sk = 4 * (int64_t)w * cpw_of(fmt);
        if ((k + sk - 1) / sk * sk == padded_min) break;
    }
    const int64_t sk = 4 * (int64_t)w * cpw_of(fmt);
    const int64_t steps = (k + sk - 1) / sk;
    const int64_t tiles = (n + 15) / 16;
    if (wpl) *wpl = w;
    if (n_steps) *n_steps = steps;
    if (step_k) *step_k = sk;
    if (packed_bytes) *packed_bytes = tiles * steps * 4 * 16 * w * 4;
    return 0;
}

int64_t orc_n_groups(int scale_mode, int64_t k, int64_t group) {
    if (scale_mode != ORC_SCALE_GROUP) return 1;
    if (group < 1) return -1;
    return (k + group - 1) / group;
}

/* group scales are stored [tile][group][16 rows]; tensor [1]; row [n] */
int64_t orc_n_scales(int scale_mode, int64_t n, int64_t k, int64_t group) {
    if (scale_mode == ORC_SCALE_TENSOR) return 1;
    if (scale_mode == ORC_SCALE_ROW) return n;
    return (n + 15) / 16 * orc_n_groups(scale_mode, k, group) * 16;
}

int orc_pack_scales(int scale_mode, int64_t n, int64_t k, int64_t group, const float* natural, float* packed) {
    const int64_t ns = orc_n_scales(scale_mode, n, k, group);
    if (ns < 1 || !natural || !packed) return ORC_E_ARG;
    if (scale_mode != ORC_SCALE_GROUP) {
        memcpy(packed, natural, (size_t)ns * sizeof(float));
        return 0;
    }
    const int64_t G = orc_n_groups(scale_mode, k, group);
    memset(packed, 0, (size_t)ns * sizeof(float));
    for (int64_t r = 0; r < n; ++r)
        for (int64_t gi = 0; gi < G; ++gi)
            packed[((r / 16) * G + gi) * 16 + r % 16] = natural[r * G + gi];
    return 0;
}

int orc_unpack_scales(int scale_mode, int64_t n, int64_t k, int64_t group, const float* packed, float* natural) {
    const int64_t ns = orc_n_scales(scale_mode, n, k, group);
    if (ns < 1 || !natural || !packed) return ORC_E_ARG;
    if (scale_mode != ORC_SCALE_GROUP) {
        memcpy(natural, packed, (size_t)ns * sizeof(float));
        return 0;
    }
    const int64_t G = orc_n_groups(scale_mode, k, group);
    for (int64_t r = 0; r < n; ++r)
        for (int64_t gi = 0; gi < G; ++gi)
            natural[r * G + gi] = packed[((r / 16) * G + gi) * 16 + r % 16];
    return 0;
}

/* byte offset (from the start of the packed matrix) and bit shift of the
 * field of code (row, k) */
static void code_position(int fmt, int wpl, int64_t n_steps, int64_t row, int64_t k, int64_t* byte, int* shift) {
    const int cpw = cpw_of(fmt), kb = kb_of(fmt), wb = kb / 4 / cpw;
    const int64_t sk = 4 * (int64_t)wpl * cpw;
    const int64_t t = row / 16, r = row % 16, s = k / sk, kk = k % sk;
    const int64_t b = kk / kb, q = kk % kb, g = q / (kb / 4), qq = q % (kb / 4);
    const int64_t h = qq / cpw, j = qq % cpw;
    const int64_t w = b * wb + h;
    const int64_t word = (((t * n_steps + s) * 4 + g) * 16 + r) * wpl + w;
    if (fmt == ORC_BINARY) {
        *byte = word * 4 + j / 8;
        *shift = (int)(j % 8);
    } else {
        *byte = word * 4 + j % 4;
        *shift = (int)(field_bits(fmt) * (j / 4));
    }
}

/* code -> field value.  binary: bit = (1 - s) / 2 ([NBT] 0x06E).
 * ternary/int4: the code's two's-complement low bits. */
static int encode_field(int fmt, int code) {
    if (fmt == ORC_BINARY) return (1 - code) / 2;
    return code & ((1 << field_bits(fmt)) - 1);
}

/* field value -> code, or 99 for a reserved pattern (ternary 10, int4 1000) */
static int decode_field(int fmt, int f) {
    if (fmt == ORC_BINARY) return 1 - 2 * f;
    if (fmt == ORC_TERNARY) {
        if (f == 2) return 99;
        return f == 3 ? -1 : f;
    }
    if (f == 8) return 99;
    return f >= 8 ? f - 16 : f;
}

int orc_pack(int fmt, int64_t n, int64_t k, const int8_t* codes, uint8_t* packed) {
    if (!fmt_ok(fmt) || n < 1 || k < 1 || !codes || !packed) return ORC_E_ARG;
    int wpl; int64_t steps, sk, nbytes;
    orc_layout(fmt, n, k, &wpl, &steps, &sk, &nbytes);
    const int lo = fmt == ORC_INT4 ? -7 : -1, hi = fmt == ORC_INT4 ? 7 : 1;
    for (int64_t i = 0; i < n * k; ++i) {
        int c = codes[i];
        if (c < lo || c > hi || (fmt == ORC_BINARY && c == 0)) return ORC_E_FORMAT;
    }
    memset(packed, 0, (size_t)nbytes);       /* padding fields stay zero */
    for (int64_t r = 0; r < n; ++r)
        for (int64_t c = 0; c < k; ++c) {
            int64_t byte; int shift;
            code_position(fmt, wpl, steps, r, c, &byte, &shift);
            packed[byte] |= (uint8_t)(encode_field(fmt, codes[r * k + c]) << shift);
        }
    return 0;
}

/* [NBT] 0x06E binary unpack reference and 0x0BB "reserved patterns reject":
 * every field slot of every padded row is visited; reserved fields and any
 * nonzero field outside the logical extent are rejected. */
int orc_unpack(int fmt, int64_t n, int64_t k, const uint8_t* packed, int8_t* codes) {
    if (!fmt_ok(fmt) || n < 1 || k < 1 || !codes || !packed) return ORC_E_ARG;
    int wpl; int64_t steps, sk, nbytes;
    orc_layout(fmt, n, k, &wpl, &steps, &sk, &nbytes);
    const int bits = field_bits(fmt);
    const int64_t rows = (n + 15) / 16 * 16, cols = steps * sk;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            int64_t byte; int shift;
            code_position(fmt, wpl, steps, r, c, &byte, &shift);
            int f = (packed[byte] >> shift) & ((1 << bits) - 1);
            if (r >= n || c >= k) {
                if (f != 0) return ORC_E_FORMAT;      /* noncanonical padding */
                continue;
            }
            int v = decode_field(fmt, f);
            if (v == 99) return ORC_E_FORMAT;          /* reserved pattern */
            codes[r * k + c] = (int8_t)v;
        }
    return 0;
}

/* ------------------------------------------------------- weight quantiser */

static float clampf(float v, float lo, float hi) { return v < lo ? lo : (v > hi ? hi : v); }

/*
 * Latent weights -> codes and fp32 scales, one scale domain at a time
 * (tensor: all of W; row: one row; group: `group` consecutive columns of one
 * row, the last group possibly shorter).
 *
 * ternary: [NBT] 0x05A (b1.58 absmean): s = mean |W| over the domain,
 *          code = RoundClip(W / s, -1, 1).  READING: no epsilon (the zero
 *          domain is special-cased to s = 0, codes 0), the mean is a
 *          sequential binary64 sum in ascending index order divided by the
 *          count and rounded once to fp32, and W / s is an fp32 division
 *          rounded half-to-even.  Exact ties |W / s| = 0.5 go to 0 ([NBT]
 *          0x05B thresholds +-s/2, ties left to the rounding policy).
 * binary : [NBT] 0x06E total sign rule, +1 if w >= 0 (either signed zero)
 *          else -1; scale = mean |W| over the domain ([NBT] 0x02B).
 * int4   : [T4NT] "What is T4NT?": symmetric levels -7..+7; READING: scale =
 *          max |W| / 7 over the domain in fp32, code = clip(rint(W / s)).
 * premap : [T4NT] tanh soft clipping w -> tanh(w / 3) * 3, evaluated in
 *          binary64 and rounded once to fp32, before any of the above.
 */
int orc_weight_codes(int fmt, int scale_mode, int64_t group, int premap,
                     int64_t n, int64_t k, const float* w, int8_t* codes, float* scales) {
    if (!fmt_ok(fmt) || n < 1 || k < 1 || !w || !codes || !scales) return ORC_E_ARG;
    if (scale_mode < ORC_SCALE_TENSOR || scale_mode > ORC_SCALE_GROUP) return ORC_E_ARG;
    if (scale_mode == ORC_SCALE_GROUP && group < 1) return ORC_E_ARG;
    for (int64_t i = 0; i < n * k; ++i)
        if (!isfinite(w[i])) return ORC_E_NONFINITE;

    float* wp = (float*)malloc((size_t)(n * k) * sizeof(float));
    if (!wp) return ORC_E_ARG;
    for (int64_t i = 0; i < n * k; ++i)
        wp[i] = premap ? (float)(3.0 * tanh((double)w[i] / 3.0)) : w[i];

    const int64_t G = orc_n_groups(scale_mode, k, group);
    /* domain list: (row0, row1, col0, col1) */
    int64_t n_dom = scale_mode == ORC_SCALE_TENSOR ? 1 : (scale_mode == ORC_SCALE_ROW ? n : n * G);

    #pragma omp parallel for schedule(static)
    for (int64_t d = 0; d < n_dom; ++d) {
        int64_t r0, r1, c0, c1;
        if (scale_mode == ORC_SCALE_TENSOR) { r0 = 0; r1 = n; c0 = 0; c1 = k; }
        else if (scale_mode == ORC_SCALE_ROW) { r0 = d; r1 = d + 1; c0 = 0; c1 = k; }
        else {
            r0 = d / G; r1 = r0 + 1;
            c0 = (d % G) * group; c1 = c0 + group < k ? c0 + group : k;
        }
        float s;
        if (fmt == ORC_INT4) {
            float m = 0.0f;
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t c = c0; c < c1; ++c) {
                    float a = fabsf(wp[r * k + c]);
                    if (a > m) m = a;
                }
            s = m / 7.0f;
        } else {
            double sum = 0.0;
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t c = c0; c < c1; ++c)
                    sum += fabs((double)wp[r * k + c]);
            s = (float)(sum / (double)((r1 - r0) * (c1 - c0)));
        }
        scales[d] = s;
        for (int64_t r = r0; r < r1; ++r)
            for (int64_t c = c0; c < c1; ++c) {
                float v = wp[r * k + c];
                int8_t code;
                if (fmt == ORC_BINARY) {
                    code = v >= 0.0f ? 1 : -1;
                } else if (s == 0.0f) {
                    code = 0;
                } else {
                    float lim = fmt == ORC_INT4 ? 7.0f : 1.0f;
                    float qv = v / s;
                    code = (int8_t)clampf(rintf(qv), -lim, lim);
                }
                codes[r * k + c] = code;
            }
    }
    free(wp);
    return 0;
}

/* --------------------------------------------------- activation quantiser */

/*
 * Per-token absmax int8 quantisation, [NBT] 0x02C and 0x05C (the 127-based
 * per-token realisation):  m = max_k |x|;  q = clip(rint(x * 127 / m));
 * s_x = m / 127;  an all-zero row gives zero codes and s_x = 0.
 * READING: no epsilon; r = 127 / m is one fp32 division, q = rint(x * r) one
 * fp32 multiply rounded half-to-even, clip to [-127, 127]; s_x = m / 127 in
 * fp32.  A row with a non-finite entry, or whose 127 / m overflows, is
 * rejected ([NBT] 0x05C: the reference rejects non-finite rows and
 * unrepresentable scales).
 */
int64_t orc_act_quant(int64_t t, int64_t k, const float* x, int8_t* q, float* sx,
                      int32_t* row_status) {
    if (t < 1 || k < 1 || !x || !q || !sx || !row_status) return ORC_E_ARG;
    int64_t rejected = 0;
    #pragma omp parallel for schedule(static) reduction(+ : rejected)
    for (int64_t i = 0; i < t; ++i) {
        const float* xr = x + i * k;
        int8_t* qr = q + i * k;
        int finite = 1;
        float m = 0.0f;
        for (int64_t c = 0; c < k; ++c) {
            if (!isfinite(xr[c])) { finite = 0; break; }
            float a = fabsf(xr[c]);
            if (a > m) m = a;
        }
        if (!finite) {
            memset(qr, 0, (size_t)k); sx[i] = NAN; row_status[i] = ORC_ROW_NONFINITE; ++rejected;
            continue;
        }
        if (m == 0.0f) {
            memset(qr, 0, (size_t)k); sx[i] = 0.0f; row_status[i] = ORC_ROW_OK;
            continue;
        }
        float r = 127.0f / m;
        if (!isfinite(r)) {
            memset(qr, 0, (size_t)k); sx[i] = NAN; row_status[i] = ORC_ROW_OVERFLOW; ++rejected;
            continue;
        }
        for (int64_t c = 0; c < k; ++c) {
            float v = xr[c] * r;
            qr[c] = (int8_t)clampf(rintf(v), -127.0f, 127.0f);
        }
        sx[i] = m / 127.0f;
        row_status[i] = ORC_ROW_OK;
    }
    return rejected;
}

/* ------------------------------------------------------- integer product */

/*
 * acc = Q8(x) . Q(W)^T in 64-bit integers, the plain definition of
 * [NBT] 0x02D and 0x09C (the reference decoder's int64 matmul), kept per
 * scale group: acc[t, n, g] sums columns [g * group_cols, (g+1) * group_cols).
 * group_cols <= 0 means one group spanning all of k.
 */
int orc_int_matmul(int64_t t, int64_t n, int64_t k, int64_t group_cols,
                   const int8_t* q, const int8_t* codes, int64_t* acc) {
    if (t < 1 || n < 1 || k < 1 || !q || !codes || !acc) return ORC_E_ARG;
    const int64_t gc = group_cols > 0 ? group_cols : k;
    const int64_t G = (k + gc - 1) / gc;
    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < t; ++i)
        for (int64_t r = 0; r < n; ++r) {
            const int8_t* qi = q + i * k;
            const int8_t* cr = codes + r * k;
            for (int64_t g = 0; g < G; ++g) {
                int64_t c0 = g * gc, c1 = c0 + gc < k ? c0 + gc : k;
                int64_t s = 0;
                for (int64_t c = c0; c < c1; ++c) s += (int64_t)qi[c] * (int64_t)cr[c];
                acc[(i * n + r) * G + g] = s;
            }
        }
    return 0;
}

/*
 * Rescale, [NBT] 0x02D / 0x09C: y = acc * s_x * s_w.
 * READING (fp32, left to right, no fused multiply-add):
 *   tensor / row scales: y = (float)acc * (s_x[t] * s_w[n])
 *   group scales       : y = s_x[t] * sum_{g ascending} (s_w[n, g] * (float)acc[t, n, g])
 * y64 is the same expression evaluated in binary64 from the same inputs.
 */
int orc_epilogue(int scale_mode, int64_t t, int64_t n, int64_t n_groups,
                 const int64_t* acc, const float* sx, const float* scales,
                 float* y32, double* y64) {
    if (t < 1 || n < 1 || n_groups < 1 || !acc || !sx || !scales || !y32 || !y64) return ORC_E_ARG;
    #pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < t; ++i)
        for (int64_t r = 0; r < n; ++r) {
            const int64_t* a = acc + (i * n + r) * n_groups;
            if (scale_mode == ORC_SCALE_GROUP) {
                float s32 = 0.0f;
                double s64 = 0.0;
                for (int64_t g = 0; g < n_groups; ++g) {
                    float term = scales[r * n_groups + g] * (float)a[g];
                    s32 = s32 + term;
                    s64 = s64 + (double)scales[r * n_groups + g] * (double)a[g];
                }
                y32[i * n + r] = sx[i] * s32;
                y64[i * n + r] = (double)sx[i] * s64;
            } else {
                float sw = scale_mode == ORC_SCALE_TENSOR ? scales[0] : scales[r];
                float prod = sx[i] * sw;
                y32[i * n + r] = (float)a[0] * prod;
                y64[i * n + r] = (double)a[0] * (double)sx[i] * (double)sw;
            }
        }
    return 0;
}

/* worst case of [NBT] 0x09C: |acc| <= k * 127 * qmax must fit a signed 32-bit
 * accumulator (127 is the largest activation code this quantiser emits). */
int orc_acc_bound_ok(int fmt, int64_t k) {
    int64_t qmax = fmt == ORC_INT4 ? 7 : 1;
    if (k < 1) return 0;
    return k <= (int64_t)2147483647 / (127 * qmax);
}

int orc_linear(int fmt, int scale_mode, int64_t group, int64_t n, int64_t k,
               const uint8_t* packed, const float* scales,
               int64_t t, const int8_t* q, const float* sx,
               float* y32, double* y64, int64_t* acc) {
    if (!fmt_ok(fmt) || n < 1 || k < 1 || t < 1) return ORC_E_ARG;
    if (!orc_acc_bound_ok(fmt, k)) return ORC_E_RANGE;
    const int64_t G = orc_n_groups(scale_mode, k, group);
    if (G < 1) return ORC_E_ARG;
    int8_t* codes = (int8_t*)malloc((size_t)(n * k));
    float* nat = (float*)malloc((size_t)(scale_mode == ORC_SCALE_GROUP ? n * G : (scale_mode == ORC_SCALE_ROW ? n : 1)) * sizeof(float));
    int rc = (!codes || !nat) ? ORC_E_ARG : 0;
    if (rc == 0) rc = orc_unpack(fmt, n, k, packed, codes);
    if (rc == 0) rc = orc_unpack_scales(scale_mode, n, k, group, scales, nat);
    if (rc == 0)
        rc = orc_int_matmul(t, n, k, scale_mode == ORC_SCALE_GROUP ? group : 0, q, codes, acc);
    if (rc == 0)
        rc = orc_epilogue(scale_mode, t, n, G, acc, sx, nat, y32, y64);
    free(codes);
    free(nat);
    return rc;
}
