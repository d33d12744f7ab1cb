// gemv.hpp - launch parameters of the decode GEMV (one launch, one or more
// weight matrices of equal k, format, scale mode and token count).
#pragma once

#include <stdint.h>

namespace lowbit {

constexpr int kGemvMaxMats = 40;   // matrices per launch (kernel-argument space)

struct GemvMat {
    const uint8_t* packed;
    const float* scales;
    const int8_t* q;
    const float* sx;
    float* y;
    int32_t* acc;        // nullable
    int n;               // rows
    int tile0;           // first global 16-row tile of this matrix
};

struct GemvParams {
    int n_mats;
    int K;
    int T;               // tokens, 1..16
    int n_steps;         // k-steps per row
    int spu;             // k-steps per scale group (1 unless group mode)
    int G;               // scale groups per row (group mode)
    int scale_per_row;   // tensor/row mode: 1 = scales[n], 0 = scales[0]
    int q_aligned;       // K % 16 == 0 and every q 16-byte aligned
    int spu_shift;       // log2(spu) when spu is a power of two
    int ksplit;          // wavefronts sharing one tile's k-range (1, 2, 4)
    int tpw;             // tiles per workgroup = 4 / ksplit
    int part_len;        // k-steps per part (the last part may run short)
    int loop_steps;      // part_len rounded up to the prefetch depth
    int total_tiles;
    int n_tile_groups;   // ceil(total_tiles / tpw)
    int64_t row_bytes;
    GemvMat m[kGemvMaxMats];
};

}  // namespace lowbit
