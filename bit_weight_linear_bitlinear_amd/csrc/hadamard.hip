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
// with -ffp-contract=off; the cross-lane form fma(s, v, p) with s = +-1 is a
// single rounding of p +- v, the same as the add or subtract.
//
// Layout.  A wavefront transforms a unit of 256 * E elements (E = B / 256 when
// B >= 256, else 1) held as E float4 per lane: element (c, lane, j) is
// 256 c + 4 lane + j.  Index bits 0-1 are the float4 components (stages
// h = 1, 2 in registers), bits 2-7 the lane (h = 4 .. 128 across lanes), bits
// 8 and up the chunk c (h = 256 .. B / 2 in registers).  A row is spread
// over WPR wavefronts (1, 4 or 16), each holding UPW units in registers, so
// the row is read from HBM once, reduced, and quantised from the registers.
#include <math.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace lowbit {

namespace {

// clip(rint(v * r), -7, 7): one fp32 multiply, ties to even
__device__ __forceinline__ uint32_t code4(float v, float r) {
    float c = rintf(v * r);
    c = c < -7.0f ? -7.0f : (c > 7.0f ? 7.0f : c);
    return (uint32_t)(uint8_t)(int8_t)(int)c;
}

__device__ __forceinline__ void bfly(float& a, float& c) {
    const float s = a + c, d = a - c;
    a = s;
    c = d;
}

// one cross-lane stage: partner = lane ^ M; the lane whose bit M is clear
// holds a and keeps a + c, the other holds c and keeps a - c
template <int M>
__device__ __forceinline__ float xstage(float v, float s) {
    return fmaf(s, v, __shfl_xor(v, M, 64));
}

template <int M>
__device__ __forceinline__ void xstage4(float4& v, int lane) {
    const float s = (lane & M) ? -1.0f : 1.0f;
    v.x = xstage<M>(v.x, s);
    v.y = xstage<M>(v.y, s);
    v.z = xstage<M>(v.z, s);
    v.w = xstage<M>(v.w, s);
}

__device__ __forceinline__ void bfly4(float4& a, float4& c) {
    bfly(a.x, c.x);
    bfly(a.y, c.y);
    bfly(a.z, c.z);
    bfly(a.w, c.w);
}

template <int E, int UPW, int WPR>
__global__ __launch_bounds__(WPR == 16 ? 1024 : 256) void act_quant_h4_kernel(
    const float* __restrict__ x, int t, int k, int b, float scale, int8_t* __restrict__ q,
    float* __restrict__ sx, int32_t* __restrict__ status) {
    constexpr int WG = WPR == 16 ? 16 : 4;   // wavefronts per workgroup
    constexpr int RPW = WG / WPR;            // rows per workgroup
    constexpr int U4 = 64 * E;               // float4 per unit
    __shared__ float red_m[WG];
    __shared__ int red_bad[WG];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row = blockIdx.x * RPW + wave / WPR;
    const int wr = wave % WPR;
    if (row >= t) return;   // only when WPR == 1 (RPW > 1): no barrier follows then
    const int k4 = k >> 2;
    const float4* xr = reinterpret_cast<const float4*>(x + (size_t)row * k);

    float4 v[UPW][E];
    #pragma unroll
    for (int uu = 0; uu < UPW; ++uu) {
        const int base = (wr + uu * WPR) * U4 + lane;
        #pragma unroll
        for (int c = 0; c < E; ++c) {
            const int i = base + 64 * c;
            v[uu][c] = i < k4 ? xr[i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
    }

    float m = 0.0f;
    int bad = 0;
    #pragma unroll
    for (int uu = 0; uu < UPW; ++uu) {
        #pragma unroll
        for (int c = 0; c < E; ++c) {   // h = 1, 2
            float4& a = v[uu][c];
            bfly(a.x, a.y);
            bfly(a.z, a.w);
            bfly(a.x, a.z);
            bfly(a.y, a.w);
        }
        // h = 4 .. min(B, 256) / 2 across lanes (b is uniform)
        #pragma unroll
        for (int c = 0; c < E; ++c) {
            float4& a = v[uu][c];
            if (b > 4) xstage4<1>(a, lane);
            if (b > 8) xstage4<2>(a, lane);
            if (b > 16) xstage4<4>(a, lane);
            if (b > 32) xstage4<8>(a, lane);
            if (b > 64) xstage4<16>(a, lane);
            if (b > 128) xstage4<32>(a, lane);
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
            a.x *= scale;
            a.y *= scale;
            a.z *= scale;
            a.w *= scale;
            bad |= !(isfinite(a.x) && isfinite(a.y) && isfinite(a.z) && isfinite(a.w));
            const float a0 = fabsf(a.x), a1 = fabsf(a.y), a2 = fabsf(a.z), a3 = fabsf(a.w);
            m = a0 > m ? a0 : m; m = a1 > m ? a1 : m; m = a2 > m ? a2 : m; m = a3 > m ? a3 : m;
        }
    }
    m = wave_max(m);
    bad = wave_or(bad);
    if constexpr (WPR > 1) {   // RPW == 1: the workgroup is one row
        if (lane == 0) { red_m[wave] = m; red_bad[wave] = bad; }
        __syncthreads();
        #pragma unroll
        for (int i = 0; i < WG; ++i) { m = red_m[i] > m ? red_m[i] : m; bad |= red_bad[i]; }
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
        #pragma unroll
        for (int c = 0; c < E; ++c) {
            const int i = base + 64 * c;
            if (i < k4) {
                const float4 a = v[uu][c];
                uint32_t p = 0u;   // a rejected row gets zero codes
                if (!flag) p = code4(a.x, r) | (code4(a.y, r) << 8) | (code4(a.z, r) << 16) | (code4(a.w, r) << 24);
                qr[i] = p;
            }
        }
    }
    if (wr == 0 && lane == 0) {
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
    // a wavefront per row while a lane holds at most 4 float4, then a
    // 256-thread workgroup per row (16 float4 per lane), then 1024 threads
    if (units * e <= 4) return launch_h4_e<1, 4>(e, units, x, t, k, b, scale, q, sx, status, stream);
    if ((units + 3) / 4 * e <= 16)
        return launch_h4_e<4, 16>(e, (units + 3) / 4, x, t, k, b, scale, q, sx, status, stream);
    return launch_h4_e<16, 16>(e, (units + 15) / 16, x, t, k, b, scale, q, sx, status, stream);
}

}  // namespace lowbit
