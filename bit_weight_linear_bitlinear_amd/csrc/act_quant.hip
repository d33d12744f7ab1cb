// act_quant.hip - per-token absmax int8 activation quantiser (gfx950).
//
// M8.8 "Native Binary and Ternary Transformers", 0x02C and 0x05C (the
// 127-based per-token realisation): for each token row
//     m   = max_k |x|
//     q   = clip(rint(x * (127 / m)), -127, 127)      fp32, ties to even
//     s_x = m / 127                                     (0 for an all-zero row)
// Bit-exactness: 127 / m and m / 127 are IEEE-correct fp32 divisions (the
// default HIP division, no fast-math), x * r is a single fp32 multiply rounded
// once and the file is built with -ffp-contract=off, and rintf maps to
// v_rndne_f32.  Denormals are kept (no flush-to-zero).
//
// HBM-bound stream (4 bytes read, 1 byte written per element): one wavefront
// per row, 16-byte loads, the row max reduced across the wave with lane
// shuffles, then a second pass over the row (served from L2) writes 4 codes
// per 32-bit store.
#include "device_common.hpp"
#include "kernels.hpp"

namespace lowbit {

constexpr int kActWaves = 4;   // rows per 256-thread workgroup

__device__ __forceinline__ int8_t quant1(float v, float r) {
    float p = v * r;
    float c = rintf(p);
    c = c < -127.0f ? -127.0f : (c > 127.0f ? 127.0f : c);
    return (int8_t)(int)c;
}

template <bool VEC>
__global__ __launch_bounds__(256) void act_quant_kernel(const float* __restrict__ x, int t, int k,
                                                        int8_t* __restrict__ q, float* __restrict__ sx,
                                                        int32_t* __restrict__ status) {
    const int row = blockIdx.x * kActWaves + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= t) return;   // whole wavefronts exit together
    const float* xr = x + (size_t)row * k;
    int8_t* qr = q + (size_t)row * k;

    float m = 0.0f;
    int bad = 0;
    if (VEC) {
        const float4* x4 = reinterpret_cast<const float4*>(xr);
        const int k4 = k >> 2;
        for (int i = lane; i < k4; i += 64) {
            float4 v = x4[i];
            float a0 = fabsf(v.x), a1 = fabsf(v.y), a2 = fabsf(v.z), a3 = fabsf(v.w);
            bad |= !(isfinite(v.x) && isfinite(v.y) && isfinite(v.z) && isfinite(v.w));
            m = a0 > m ? a0 : m; m = a1 > m ? a1 : m; m = a2 > m ? a2 : m; m = a3 > m ? a3 : m;
        }
    } else {
        for (int i = lane; i < k; i += 64) {
            float v = xr[i];
            bad |= !isfinite(v);
            float a = fabsf(v);
            m = a > m ? a : m;
        }
    }
    m = wave_max(m);
    bad = wave_or(bad);

    float r = 0.0f;
    int flag = 0;
    if (bad) {
        flag = LOWBIT_ACT_NONFINITE;
    } else if (m > 0.0f) {
        r = 127.0f / m;
        if (!isfinite(r)) flag = LOWBIT_ACT_OVERFLOW;
    }
    if (flag) {   // a rejected row gets zero codes
        if (VEC) {
            uint32_t* q4 = reinterpret_cast<uint32_t*>(qr);
            for (int i = lane; i < (k >> 2); i += 64) q4[i] = 0u;
        } else {
            for (int i = lane; i < k; i += 64) qr[i] = 0;
        }
    } else if (VEC) {
        const float4* x4 = reinterpret_cast<const float4*>(xr);
        uint32_t* q4 = reinterpret_cast<uint32_t*>(qr);
        const int k4 = k >> 2;
        for (int i = lane; i < k4; i += 64) {
            float4 v = x4[i];
            uint32_t p = (uint32_t)(uint8_t)quant1(v.x, r) | ((uint32_t)(uint8_t)quant1(v.y, r) << 8) |
                         ((uint32_t)(uint8_t)quant1(v.z, r) << 16) | ((uint32_t)(uint8_t)quant1(v.w, r) << 24);
            q4[i] = p;
        }
    } else {
        for (int i = lane; i < k; i += 64) qr[i] = quant1(xr[i], r);
    }
    if (lane == 0) {
        sx[row] = flag ? __builtin_nanf("") : m / 127.0f;
        if (flag && status) atomicOr(status, flag);
    }
}

hipError_t launch_act_quant(const float* x, int t, int k, int8_t* q, float* sx, int32_t* status,
                            hipStream_t stream) {
    dim3 grid((unsigned)((t + kActWaves - 1) / kActWaves)), block(256);
    const bool vec = (k % 4 == 0) && ((uintptr_t)x % 16 == 0) && ((uintptr_t)q % 4 == 0);
    if (vec)
        act_quant_kernel<true><<<grid, block, 0, stream>>>(x, t, k, q, sx, status);
    else
        act_quant_kernel<false><<<grid, block, 0, stream>>>(x, t, k, q, sx, status);
    return hipGetLastError();
}

}  // namespace lowbit
