// kernels.hpp - internal launcher interface between the C ABI layer and the
// HIP kernels.  Arguments have been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lowbit.h"

namespace lowbit {

struct LinearArgs {
    int fmt;             // FMT_*
    int scale;           // 0 tensor, 1 row, 2 group
    int group;           // group mode: columns per group
    int n_groups;        // group mode: ceil(k / group), else 1
    int n, k, t;
    int wpl;             // packed words per (lane group, row) per k-step
    int step_k;          // codes per k-step
    int n_steps;         // k-steps per row
    const uint8_t* packed;
    const float* scales;
    const int8_t* q;
    const float* sx;
    float* y;
    int32_t* acc;        // nullable
    // fused activation quantisation (decode path only): x fp32 [t, k] is
    // quantised inside the product, and q / sx above are then outputs (the
    // codes and scales lowbit_act_quant would write); nullptr = q / sx given
    const float* x = nullptr;
    int32_t* status = nullptr;   // nullable: LOWBIT_ACT_* bits of rejected rows
    // an input transform in the fused prologue (one token; see gemv_kernel's
    // PRE): pre = 1 norm (x + pre_r, RMSNorm with pre_g / pre_eps; x + pre_r to
    // pre_xo, the norm to pre_ho), 2 SwiGLU (SiLU(x) * pre_r to pre_ho); taken
    // from the first matrix of a launch, whose matrices all share x
    int pre = 0;
    const float* pre_r = nullptr;
    const float* pre_g = nullptr;
    float pre_eps = 0.0f;
    float* pre_xo = nullptr;
    float* pre_ho = nullptr;
};

hipError_t launch_act_quant(const float* x, int t, int k, int8_t* q, float* sx, int32_t* status,
                            hipStream_t stream);
// the inputs of `count` matrices of equal [t, k] in as few launches as possible
constexpr int kActQuantMaxSrc = 40;
hipError_t launch_act_quant_group(const float* const* x, int8_t* const* q, float* const* sx, int count, int t,
                                  int k, int32_t* status, hipStream_t stream);
// H-BitLinear's rotated 4-bit quantiser (hadamard.hip): block size of a row
// width (0 when k has no power-of-two factor of 64 or more), widest row
constexpr int kH4MaxBlock = 2048;
constexpr int kH4MaxK = 65536;
int h4_block(int k);
hipError_t launch_act_quant_h4(const float* x, int t, int k, int8_t* q, float* sx, int32_t* status,
                               hipStream_t stream);
// BitNet a4.8's codes: 4-bit per-token codes of projection inputs
// (act_quant.hip), and the sparse 8-bit codes of intermediate states, each
// row keeping its `keep` largest |x| (sparse8.hip), rows up to kSparse8MaxK
constexpr int kSparse8MaxK = 32768;
hipError_t launch_act_quant_a4(const float* x, int t, int k, int8_t* q, float* sx, int32_t* status,
                               hipStream_t stream);
hipError_t launch_act_quant_sparse8(const float* x, int t, int k, int keep, int8_t* q, float* sx, int32_t* status,
                                    hipStream_t stream);
// the original BitNet forward's pieces: Q_b = 128 codes with the encoder
// epsilon, per token (tensor == nullptr) or with the tensor-wide max a prior
// launch_tensor_absmax left in tensor[0..1]; the sub-layer LayerNorm
hipError_t launch_act_quant_v1(const float* x, int t, int k, float eps, const uint32_t* tensor, int8_t* q,
                               float* sx, int32_t* status, hipStream_t stream);
hipError_t launch_tensor_absmax(const float* x, int64_t n, uint32_t* work, hipStream_t stream);
hipError_t launch_layernorm(const float* x, int t, int d, float eps, const float* g, const float* b, float* out,
                            hipStream_t stream);
// OneBit's W1A16 projection: y = h * (fp16(x * g) . S^T), signs in the binary layout
hipError_t launch_onebit(const uint8_t* packed, const uint16_t* g, const uint16_t* h, const uint16_t* x, float* y,
                         int n, int k, int t, int wpl, int step_k, int n_steps, hipStream_t stream);
hipError_t launch_gemv(const LinearArgs& a, hipStream_t stream);
// several matrices of equal fmt / scale mode / group / k and t <= 16 in one launch
hipError_t launch_gemv_group(const LinearArgs* mats, int count, hipStream_t stream);
hipError_t launch_gemm(const LinearArgs& a, hipStream_t stream);
// several products of equal fmt / scale mode / group / k / t in as few launches as possible
hipError_t launch_gemm_group(const LinearArgs* mats, int count, hipStream_t stream);
hipError_t launch_gemm_mfma_group(const LinearArgs* mats, int count, hipStream_t stream);
// the streaming GEMM (k % 16 == 0, 16-byte aligned q and packed) and the general one
bool gemm_mfma_supported(const LinearArgs& a);
hipError_t launch_gemm_mfma(const LinearArgs& a, hipStream_t stream);
hipError_t launch_gemm_generic(const LinearArgs& a, hipStream_t stream);
// compute units of the current device (cached per device)
int device_cu_count();

// the small kernels of a decode step (decode_model.hip); state = int32[4],
// or nullptr outside a step (then the position is `pos` and nothing is skipped)
hipError_t launch_embed_norm(const float* embed, int vocab, int d, const float* g, float eps, int32_t* state,
                             int context, float* x, float* h, hipStream_t st);
hipError_t launch_add_norm(const float* xs, const float* r, float* xd, int rows, int d, const float* g,
                           float eps, const int32_t* state, int context, float* h, hipStream_t st);
hipError_t launch_rope_attn(const float* qkv, int d, int heads, double base, const int32_t* state, int pos,
                            int context, float* kc, float* vc, float* attn, float* q_trace, float* k_trace,
                            hipStream_t st);
hipError_t launch_swiglu(const float* gate, const float* up, float* a, int64_t n, const int32_t* state,
                         int context, hipStream_t st);
hipError_t launch_argmax_advance(const float* logits, int vocab, int32_t* state, int context, int32_t* tokens,
                                 hipStream_t st);

// device ceilings (calib.hip): a 16-byte read stream over `bytes` (a multiple
// of 16, 16-byte aligned), and an int8 matrix-core loop of `iters` iterations
// whose operations per iteration calib_mfma_i8_ops_per_iter() gives
hipError_t launch_calib_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream);
int64_t calib_mfma_i8_ops_per_iter();
hipError_t launch_calib_mfma_i8(int32_t iters, uint32_t* sink, hipStream_t stream);

}  // namespace lowbit
