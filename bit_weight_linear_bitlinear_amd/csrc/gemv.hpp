// gemv.hpp - launch parameters of the decode GEMV (one launch, one or more
// weight matrices of equal k, format, scale mode and token count).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lowbit {

constexpr int kGemvMaxMats = 256;    // matrices per launch (a 17 KB kernel-argument table)
constexpr int kGemvLdsA = 56 * 1024; // activation bytes a 4-wavefront workgroup may stage in LDS
constexpr int kGemvLdsWide = 20 * 1024;   // above this stage, 16-wavefront workgroups share it (t > 1)
constexpr int kGemvLdsMax = 160 * 1024;   // LDS of a CU
constexpr int kGemvLdsHalf = 80 * 1024;   // a 16-wavefront stage that leaves room for a second workgroup
constexpr int kGemvD = 4;                 // k-steps of weight loads in flight per wavefront

// input transforms of the fused prologue (PRE_* of gemv_kernel)
enum { PRE_NONE = 0, PRE_NORM = 1, PRE_SWIGLU = 2 };

struct GemvMat {
    const uint8_t* packed;
    const float* scales;
    const int8_t* q;     // fused launches: written (the codes of x) by the matrix's first workgroup
    const float* sx;     // fused launches: written likewise
    const float* x;      // fused launches: fp32 activations [T, K]; else unused
    float* y;
    int32_t* acc;        // nullable
    int n;               // rows
    int n_tiles;         // ceil(n / 16)
};

struct GemvParams {
    int n_mats;
    int K;
    int T;               // tokens, 1..16
    int n_steps;         // k-steps per row (packed layout)
    int G;               // scale groups per row (group mode)
    int upg;             // group mode: scale units per group
    int upg_shift;       // log2(upg), or -1 when upg is not a power of two
    int scale_per_row;   // tensor/row mode: 1 = scales[n], 0 = scales[0]
    int ksplit;          // wavefronts sharing one tile's k-range (1, 2, 4)
    int ksplit_log;
    int part_len;        // k-steps per part (the last part may run short)
    int tiles_per_wg;    // waves per workgroup / ksplit
    int stride;          // LDS bytes per staged token row (the phase's k padded, + 16)
    int ph_steps;        // k-steps per LDS phase (n_steps: the whole row is staged at once)
    int q_vec;           // k % 16 == 0 and every q 16-byte aligned
    int lds_a_bytes;     // T * stride when activations are staged in LDS, else 0
    int q_word;          // fused: k % 4 == 0 and every q 4-byte aligned
    int32_t* status;     // fused: LOWBIT_ACT_* bits of rejected rows (nullable)
    // PRE_NORM: residual r (nullable), gain g, eps; out: x + r (pre_xo), h (pre_ho, nullable)
    // PRE_SWIGLU: up (pre_r); out: a (pre_ho, nullable).  Every matrix of the launch shares x.
    const float* pre_r;
    const float* pre_g;
    float pre_eps;
    float* pre_xo;
    float* pre_ho;
    int wg_start[kGemvMaxMats + 1];   // first workgroup of each matrix (ascending; INT_MAX past n_mats)
    GemvMat m[kGemvMaxMats];
};

// Launch configuration chosen on the host.
struct GemvCfg {
    int wpl;             // packed words per lane per k-step
    int nr;              // C registers per lane holding live tokens: 1 (t <= 4) or 4
    int sps;             // group mode: scale units per k-step (1, 2, 4); 0 = tensor/row scales
    bool lds_a;          // activations staged in LDS (else read from global memory)
    bool acc;            // some matrix wants the integer products
    bool fuse;           // activations quantised in the kernel's prologue (needs lds_a, 4 waves)
    int waves;           // wavefronts per workgroup: 4, or 16 with a large LDS stage
    int pre;             // PRE_*: the fused prologue's input transform
    int grid;
    size_t lds_bytes;
};

// Per-format launchers (gemv_ternary.hip, gemv_int4.hip, gemv_binary.hip).
hipError_t gemv_launch_ternary(const GemvParams& p, const GemvCfg& c, hipStream_t stream);
hipError_t gemv_launch_int4(const GemvParams& p, const GemvCfg& c, hipStream_t stream);
hipError_t gemv_launch_binary(const GemvParams& p, const GemvCfg& c, hipStream_t stream);

}  // namespace lowbit
