/*
 * oracle.h - CPU oracle for the low-bit linear layer  y = s_w * s_x * (Q(W) . Q8(x)).
 *
 * TEST INFRASTRUCTURE ONLY.  This is a plain, slow, obviously-correct scalar C
 * implementation used to check the GPU library.  Only the tests, the smoke
 * check and the bench's CPU-baseline leg may load it; the product path never
 * does.  It shares no source, header or constant table with the GPU library.
 *
 * Conventions (all arrays row-major, caller-owned):
 *   W latent  float [n, k]         codes int8 [n, k]
 *   x         float [t, k]         q     int8 [t, k]      sx float [t]
 *   scales    float [1] | [n] | [n, G] with G = ceil(k / group)  ("natural" order;
 *             the packed artifact stores group scales tiled, orc_pack_scales)
 *   acc       int64 [t, n, G]  (G = 1 unless group scales)
 *   y         float [t, n] and double [t, n]
 *
 * Every function returns 0 on success or a negative ORC_E_* code.
 */
#ifndef LOWBIT_ORACLE_H
#define LOWBIT_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* formats */
#define ORC_TERNARY 0   /* {-1, 0, +1}, 2-bit fields                      */
#define ORC_BINARY  1   /* {-1, +1}, 1 bit per code                         */
#define ORC_INT4    2   /* -7..+7, 4-bit two's-complement fields            */
/* scale domains */
#define ORC_SCALE_TENSOR 0
#define ORC_SCALE_ROW    1
#define ORC_SCALE_GROUP  2
/* errors */
#define ORC_E_ARG        (-1)
#define ORC_E_RANGE      (-2)
#define ORC_E_NONFINITE  (-3)
#define ORC_E_FORMAT     (-4)
/* act-quant per-row status */
#define ORC_ROW_OK        0
#define ORC_ROW_NONFINITE 1
#define ORC_ROW_OVERFLOW  2

/* Tiled packed layout: rows in tiles of 16, k in steps of `wpl` 32-bit words
 * per (lane group, row); see oracle.c.  Returns 0 and fills the sizes. */
int orc_layout(int fmt, int64_t n, int64_t k, int* wpl, int64_t* n_steps, int64_t* step_k,
               int64_t* packed_bytes);
int64_t orc_n_groups(int scale_mode, int64_t k, int64_t group);
/* scale array sizes and the tiled order of group scales */
int64_t orc_n_scales(int scale_mode, int64_t n, int64_t k, int64_t group);
int orc_pack_scales(int scale_mode, int64_t n, int64_t k, int64_t group, const float* natural, float* packed);
int orc_unpack_scales(int scale_mode, int64_t n, int64_t k, int64_t group, const float* packed, float* natural);

/* latent weights -> codes + fp32 scales (premap: 1 = w -> 3 tanh(w/3) first) */
int orc_weight_codes(int fmt, int scale_mode, int64_t group, int premap,
                     int64_t n, int64_t k, const float* w, int8_t* codes, float* scales);

/* codes <-> packed bytes (tiled layout) */
int orc_pack(int fmt, int64_t n, int64_t k, const int8_t* codes, uint8_t* packed);
int orc_unpack(int fmt, int64_t n, int64_t k, const uint8_t* packed, int8_t* codes);

/* per-token absmax int8 activation quantisation; returns the number of
 * rejected rows (row_status != 0), whose q/sx are left as zero / NaN */
int64_t orc_act_quant(int64_t t, int64_t k, const float* x, int8_t* q, float* sx,
                      int32_t* row_status);

/* integer product: acc[t, n, g] = sum_{k in group g} q[t, k] * codes[n, k] */
int orc_int_matmul(int64_t t, int64_t n, int64_t k, int64_t group_cols,
                   const int8_t* q, const int8_t* codes, int64_t* acc);

/* fp32 epilogue (and an fp64 second reference) */
int orc_epilogue(int scale_mode, int64_t t, int64_t n, int64_t n_groups,
                 const int64_t* acc, const float* sx, const float* scales,
                 float* y32, double* y64);

/* whole linear from packed bytes and packed (tiled) scales: unpack, integer
 * product, epilogue */
int orc_linear(int fmt, int scale_mode, int64_t group, int64_t n, int64_t k,
               const uint8_t* packed, const float* scales,
               int64_t t, const int8_t* q, const float* sx,
               float* y32, double* y64, int64_t* acc);

/* worst-case |acc| bound of the operator: k * 127 * qmax must fit int32 */
int orc_acc_bound_ok(int fmt, int64_t k);

int orc_num_threads(void);
void orc_set_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
