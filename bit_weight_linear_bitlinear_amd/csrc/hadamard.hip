// hadamard.hip - rotated 4-bit activation quantiser of H-BitLinear (gfx950).
//
// M8.8 "Native Binary and Ternary Transformers", 0x07C (BitNet v2): the input
// of a linear layer is rotated by a fast Walsh-Hadamard transform before its
// activations are quantised to INT4, so that outlier channels are spread over
// the whole block.  For each token row of k channels:
//     B    = largest power of two dividing k, at most 2048 (64 at least)
//     x'   = (H_B / sqrt(B)) x, block by block (Sylvester order)
//     m    = max_k |x'|,  r = 7 / m
//     q    = clip(rint(x' r), -7, 7)                 int8 storage
//     s_x  = m / 7                                    (0 for an all-zero row)
// The codes feed the int8 products unchanged: y = s_w s_x (Q(W) . q).
//
// Bit-exactness.  Each butterfly stage (half-width h = 1, 2, 4, ...) maps a
// pair (a, c) to (a + c, a - c), one fp32 rounding each, and the stages run
// in increasing h, so every value is the same fp32 number whichever lane
// computes it; then one multiply by fp32(1 / sqrt(B)).  The file is built
// with -ffp-contract=off; the cross-lane form fma(p, s, w) with s = +-1 is a
// single rounding of w +- p, the same as the add or subtract (up to a sign
// that rounding to nearest preserves).
//
// Layout.  A wavefront transforms a unit of 256 * E elements (E = B / 256 when
// B >= 256, else 1) held as E float4 per lane: element (c, lane, j) is
// 256 c + 4 lane + j.  Index bits 0-1 are the float4 components (stages
// h = 1, 2 in registers), bits 2-7 the lane (h = 4 .. 128 across lanes, by DPP,
// ds_swizzle and permlane32_swap: no LDS addresses), bits 8 and up the chunk
// c (h = 256 .. B / 2 in registers).  A row is spread
// over WPR wavefronts (1, 4 or 16), each holding UPW units in registers, so
// the row is read from HBM once, reduced, and quantised from the registers.
#include <math.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace lowbit {

namespace {

// clip(rint(v * r), -7, 7) in the low byte: one fp32 multiply, the clip
// (which commutes with rounding to an integer), then an add of 1.5 * 2^23,
// whose sum has a unit ulp, so the add itself rounds to the nearest integer,
// ties to even (as rintf), and the sum's low byte is the code in two's
// complement
__device__ __forceinline__ uint32_t code4_bits(float v, float r) {
    return __builtin_bit_cast(uint32_t, fminf(fmaxf(v * r, -7.0f), 7.0f) + 12582912.0f);
}

// the four codes of a float4 as one little-endian word
__device__ __forceinline__ uint32_t pack4(const float4& a, float r) {
    const uint32_t lo = __builtin_amdgcn_perm(code4_bits(a.y, r), code4_bits(a.x, r), 0x0c0c0400u);
    const uint32_t hi = __builtin_amdgcn_perm(code4_bits(a.w, r), code4_bits(a.z, r), 0x0c0c0400u);
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

__device__ __forceinline__ void bfly(float& a, float& c) {
    const float s = a + c, d = a - c;
    a = s;
    c = d;
}

__device__ __forceinline__ void bfly4(float4& a, float4& c) {
    bfly(a.x, c.x);
    bfly(a.y, c.y);
    bfly(a.z, c.z);
    bfly(a.w, c.w);
}

// Cross-lane stages on lane bits 0-4, with a per-lane sign.  A lane holds
// w = sigma * x for a sign sigma that depends only on the lane bits already
// processed, so the two lanes of a pair share it.  One fused step
// w' = w + s p (p the partner's w, s = -1 on the lane whose bit is set) gives
// sigma (a + c) on the lower lane and sigma (c - a) = -sigma (a - c) on the
// upper one: the same single rounding as a + c and a - c, with the upper
// lane's sign flipped.  The product of the flips is undone exactly when the
// row is multiplied by 1 / sqrt(B).
//   bit 0, 1: DPP quad permutation;  bit 3: DPP rotation of a 16-lane row
//   by 8;  bit 2, 4: ds_swizzle xor (no address register)
template <int M>
__device__ __forceinline__ float partner(float w) {
    const int v = __builtin_bit_cast(int, w);
    int p;
    if constexpr (M == 1) p = __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, true);         // quad_perm 1,0,3,2
    else if constexpr (M == 2) p = __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, true);    // quad_perm 2,3,0,1
    else if constexpr (M == 8) p = __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, true);   // row_ror 8
    else p = __builtin_amdgcn_ds_swizzle(v, (M << 10) | 0x1F);                                   // xor M
    return __builtin_bit_cast(float, p);
}

template <int M>
__device__ __forceinline__ void xstage4(float4& v, float s) {
    v.x = fmaf(partner<M>(v.x), s, v.x);
    v.y = fmaf(partner<M>(v.y), s, v.y);
    v.z = fmaf(partner<M>(v.z), s, v.z);
    v.w = fmaf(partner<M>(v.w), s, v.w);
}

// Lane bit 5: v_permlane32_swap exchanges the upper half of one register
// with the lower half of another, so after swapping (a, b) each lane holds
// both members of a pair (the lower lanes a's, the upper lanes b's), the
// butterfly runs in registers, and a second swap puts the results back.  The
// two lanes of a pair share their sign, and this stage adds none.
__device__ __forceinline__ void xstage32(float& a, float& b) {
    auto t = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, b),
                                              false, false);
    const float x = __builtin_bit_cast(float, (unsigned)t[0]), y = __builtin_bit_cast(float, (unsigned)t[1]);
    const float u = x + y, d = x - y;
    t = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, u), __builtin_bit_cast(unsigned, d), false,
                                         false);
    a = __builtin_bit_cast(float, (unsigned)t[0]);
    b = __builtin_bit_cast(float, (unsigned)t[1]);
}

constexpr int kWaveRow = 8;

template <int E, int UPW, int WPR>
__global__ __launch_bounds__(WPR == 16 ? 1024 : 256) void act_quant_h4_kernel(
    const float* __restrict__ x, int t, int k, int b, float scale, int8_t* __restrict__ q,
    float* __restrict__ sx, int32_t* __restrict__ status) {
    constexpr int WG = WPR == 16 ? 16 : 4;   // wavefronts per workgroup
    constexpr int RPW = WG / WPR;            // rows per workgroup
    constexpr int U4 = 64 * E;               // float4 per unit
    __shared__ float red_m[WG];
    __shared__ int red_bad[WG];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int row = blockIdx.x * RPW + wave / WPR;
    const int wr = wave % WPR;
    if constexpr (WPR == 1) {
        if (row >= t) return;   // no barrier follows
    }
    // with WPR > 1 the waves of a row past t (the last workgroup's second row
    // at WPR = 2) skip every unit but still reach the barrier
    const int k4 = row < t ? k >> 2 : 0;
    const float4* xr = reinterpret_cast<const float4*>(x + (size_t)row * k);

    // units past the row's end (UPW is rounded up) are skipped by a uniform
    // branch: neither loaded, transformed nor stored
    auto unit_ok = [&](int uu) { return (wr + uu * WPR) * U4 < k4; };
    float4 v[UPW][E];
    #pragma unroll
    for (int uu = 0; uu < UPW; ++uu) {
        const int base = (wr + uu * WPR) * U4 + lane;
        if (!unit_ok(uu)) continue;
        #pragma unroll
        for (int c = 0; c < E; ++c) {
            const int i = base + 64 * c;
            // a unit is whole unless B < 256 (E == 1), when a row's last unit
            // may hold fewer than 256 elements (whole blocks of B)
            if (E > 1 || b >= 256 || i < k4) v[uu][c] = xr[i];
            else v[uu][c] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
    }

    // the fused cross-lane steps' signs (-1 on the lane whose bit is set), and
    // the sign a lane's values carry after them: one flip per set bit among
    // the lane bits those steps used (bits 0-3, and 4 when B > 64)
    const float s1 = (lane & 1) ? -1.0f : 1.0f, s2 = (lane & 2) ? -1.0f : 1.0f, s4 = (lane & 4) ? -1.0f : 1.0f,
                s8 = (lane & 8) ? -1.0f : 1.0f, s16 = (lane & 16) ? -1.0f : 1.0f;
    const float sscale = (__popc(lane & (b > 64 ? 0x1F : 0xF)) & 1) ? -scale : scale;

    float m = 0.0f;
    #pragma unroll
    for (int uu = 0; uu < UPW; ++uu) {
        if (!unit_ok(uu)) continue;
        #pragma unroll
        for (int c = 0; c < E; ++c) {   // h = 1, 2
            float4& a = v[uu][c];
            bfly(a.x, a.y);
            bfly(a.z, a.w);
            bfly(a.x, a.z);
            bfly(a.y, a.w);
        }
        // h = 4 .. min(B, 256) / 2 across lanes (b >= 64; b is uniform)
        #pragma unroll
        for (int c = 0; c < E; ++c) {
            float4& a = v[uu][c];
            xstage4<1>(a, s1);
            xstage4<2>(a, s2);
            xstage4<4>(a, s4);
            xstage4<8>(a, s8);
            if (E > 1 || b > 64) xstage4<16>(a, s16);
        }
        if (E > 1 || b > 128) {
            #pragma unroll
            for (int c = 0; c < E; ++c) {
                xstage32(v[uu][c].x, v[uu][c].y);
                xstage32(v[uu][c].z, v[uu][c].w);
            }
        }
        // h = 256 .. B / 2 across the unit's chunks (B = 256 E here)
        #pragma unroll
        for (int cb = 1; cb < E; cb <<= 1) {
            #pragma unroll
            for (int c = 0; c < E; ++c)
                if (!(c & cb)) bfly4(v[uu][c], v[uu][c | cb]);
        }
        #pragma unroll
        for (int c = 0; c < E; ++c) {
            float4& a = v[uu][c];
            a.x *= sscale;
            a.y *= sscale;
            a.z *= sscale;
            a.w *= sscale;
            // IEEE maximum (v_maximum3_f32) keeps a NaN, so one test of m
            // finds every non-finite value of the lane
            m = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m, fabsf(a.x)), fabsf(a.y));
            m = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m, fabsf(a.z)), fabsf(a.w));
        }
    }
    int bad = !isfinite(m);
    m = wave_max(m);
    bad = wave_or(bad);
    if constexpr (WPR > 1) {   // the row's wavefronts are wave0 .. wave0 + WPR - 1
        if (lane == 0) { red_m[wave] = m; red_bad[wave] = bad; }
        __syncthreads();
        const int wave0 = wave - wr;
        #pragma unroll
        for (int i = 0; i < WPR; ++i) {
            m = red_m[wave0 + i] > m ? red_m[wave0 + i] : m;
            bad |= red_bad[wave0 + i];
        }
    }

    float r = 0.0f;
    int flag = 0;
    if (bad) {
        flag = LOWBIT_ACT_NONFINITE;
    } else if (m > 0.0f) {
        r = 7.0f / m;
        if (!isfinite(r)) flag = LOWBIT_ACT_OVERFLOW;
    }
    uint32_t* qr = reinterpret_cast<uint32_t*>(q + (size_t)row * k);
    #pragma unroll
    for (int uu = 0; uu < UPW; ++uu) {
        const int base = (wr + uu * WPR) * U4 + lane;
        if (!unit_ok(uu)) continue;
        #pragma unroll
        for (int c = 0; c < E; ++c) {
            const int i = base + 64 * c;
            if (E > 1 || b >= 256 || i < k4) qr[i] = flag ? 0u : pack4(v[uu][c], r);   // rejected: zero codes
        }
    }
    if (wr == 0 && lane == 0 && row < t) {
        sx[row] = flag ? __builtin_nanf("") : m / 7.0f;
        if (flag && status) atomicOr(status, flag);
    }
}

template <int E, int UPW, int WPR>
hipError_t launch_h4(const float* x, int t, int k, int b, float scale, int8_t* q, float* sx, int32_t* status,
                     hipStream_t stream) {
    constexpr int WG = WPR == 16 ? 16 : 4;
    constexpr int RPW = WG / WPR;
    act_quant_h4_kernel<E, UPW, WPR><<<dim3((unsigned)((t + RPW - 1) / RPW)), dim3(64 * WG), 0, stream>>>(
        x, t, k, b, scale, q, sx, status);
    return hipGetLastError();
}

// units per wavefront rounded up to a power of two with UPW * E <= CAP
template <int E, int WPR, int CAP>
hipError_t launch_h4_upw(int upw, const float* x, int t, int k, int b, float scale, int8_t* q, float* sx,
                         int32_t* status, hipStream_t stream) {
    if (upw <= 1) return launch_h4<E, 1, WPR>(x, t, k, b, scale, q, sx, status, stream);
    if constexpr (2 * E <= CAP)
        if (upw <= 2) return launch_h4<E, 2, WPR>(x, t, k, b, scale, q, sx, status, stream);
    if constexpr (4 * E <= CAP)
        if (upw <= 4) return launch_h4<E, 4, WPR>(x, t, k, b, scale, q, sx, status, stream);
    if constexpr (8 * E <= CAP)
        if (upw <= 8) return launch_h4<E, 8, WPR>(x, t, k, b, scale, q, sx, status, stream);
    if constexpr (16 * E <= CAP)
        if (upw <= 16) return launch_h4<E, 16, WPR>(x, t, k, b, scale, q, sx, status, stream);
    return hipErrorInvalidValue;
}

template <int WPR, int CAP>
hipError_t launch_h4_e(int e, int upw, const float* x, int t, int k, int b, float scale, int8_t* q, float* sx,
                       int32_t* status, hipStream_t stream) {
    switch (e) {
        case 1: return launch_h4_upw<1, WPR, CAP>(upw, x, t, k, b, scale, q, sx, status, stream);
        case 2: return launch_h4_upw<2, WPR, CAP>(upw, x, t, k, b, scale, q, sx, status, stream);
        case 4: return launch_h4_upw<4, WPR, CAP>(upw, x, t, k, b, scale, q, sx, status, stream);
        case 8:
            if constexpr (CAP >= 8) return launch_h4_upw<8, WPR, CAP>(upw, x, t, k, b, scale, q, sx, status, stream);
            return hipErrorInvalidValue;
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int h4_block(int k) {
    if (k <= 0) return 0;
    int b = k & -k;
    b = b > kH4MaxBlock ? kH4MaxBlock : b;
    return b >= 64 ? b : 0;
}

hipError_t launch_act_quant_h4(const float* x, int t, int k, int8_t* q, float* sx, int32_t* status,
                               hipStream_t stream) {
    const int b = h4_block(k);
    if (t < 1 || b == 0 || k > kH4MaxK) return hipErrorInvalidValue;
    const int e = b >= 256 ? b / 256 : 1;
    const int units = (k + 256 * e - 1) / (256 * e);
    const float scale = (float)(1.0 / sqrt((double)b));
    // a wavefront per row while a lane holds at most kWaveRow float4, then
    // two or four wavefronts per row (16 float4 per lane), then 1024 threads
    if (units * e <= kWaveRow) return launch_h4_e<1, kWaveRow>(e, units, x, t, k, b, scale, q, sx, status, stream);
    if ((units + 1) / 2 * e <= 16)
        return launch_h4_e<2, 16>(e, (units + 1) / 2, x, t, k, b, scale, q, sx, status, stream);
    if ((units + 3) / 4 * e <= 16)
        return launch_h4_e<4, 16>(e, (units + 3) / 4, x, t, k, b, scale, q, sx, status, stream);
    return launch_h4_e<16, 16>(e, (units + 15) / 16, x, t, k, b, scale, q, sx, status, stream);
}

}  // namespace lowbit
