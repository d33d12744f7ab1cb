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
// HBM-bound stream (4 bytes read, 1 byte written per element).  Aligned rows
// of up to 16384 elements are read once into registers by a wavefront (k <=
// 2048) or a whole workgroup, reduced, and quantised from the registers;
// longer or unaligned rows take a two-pass loop (one wavefront per row, the
// second pass served from L2).
#include <algorithm>

#include "device_common.hpp"
#include "kernels.hpp"

namespace lowbit {

constexpr int kActWaves = 4;   // rows per 256-thread workgroup

// The inputs of one launch: up to kActQuantMaxSrc matrices [t, k] of equal
// shape (blockIdx.y picks one), so that several products' inputs are
// quantised by one launch.
struct ActQuantTable {
    int t;
    const float* x[kActQuantMaxSrc];
    int8_t* q[kActQuantMaxSrc];
    float* sx[kActQuantMaxSrc];
    float eps;                    // MODE 1, 2: the encoder epsilon
    const uint32_t* tensor;       // MODE 2: [0] fp32 bits of the tensor's max |x|, [1] non-finite flag
};

// The code rule of a launch (M8.8 "Native Binary and Ternary Transformers"):
//   MODE 0  the per-token absmax int8 rule of 0x02C / 0x05C: r = 127 / m,
//           code = clip(rint(x r), -127, 127), s_x = m / 127;
//   MODE 1  the original BitNet forward of 0x02E, Q_b = 128: d = m + eps,
//           code = clip(rint((128 x) / d), -128, 127) (one exact multiply and
//           one IEEE division, in that order), s_x = m / 128; a zero row
//           codes to 0; a row whose 128 m overflows is rejected;
//   MODE 2  MODE 1 with the tensor-wide m of a prior reduction;
//   MODE 3  BitNet a4.8's 4-bit input codes (0x07B): the INT4 counterpart of
//           MODE 0, r = 7 / m, code = clip(rint(x r), -7, 7), s_x = m / 7.
// rowdiv() returns the row's flag and sets rr (MODE 0: r; MODE 1, 2: d).
template <int MODE>
__device__ __forceinline__ int rowdiv(float m, int bad, float eps, float& rr) {
    rr = 0.0f;
    if (bad) return LOWBIT_ACT_NONFINITE;
    if constexpr (MODE == 0 || MODE == 3) {
        if (m > 0.0f) {
            rr = (MODE == 0 ? 127.0f : 7.0f) / m;
            if (!isfinite(rr)) return LOWBIT_ACT_OVERFLOW;
        }
    } else {
        if (!isfinite(m * 128.0f)) return LOWBIT_ACT_OVERFLOW;
        rr = m + eps;
    }
    return 0;
}

template <int MODE>
__device__ __forceinline__ int8_t code_of(float v, float rr, float m) {
    if constexpr (MODE == 0) {
        return quant1(v, rr);
    } else if constexpr (MODE == 3) {
        float c = rintf(v * rr);
        c = c < -7.0f ? -7.0f : (c > 7.0f ? 7.0f : c);
        return (int8_t)(int)c;
    } else {
        if (m == 0.0f) return 0;
        float c = rintf((v * 128.0f) / rr);
        c = c < -128.0f ? -128.0f : (c > 127.0f ? 127.0f : c);
        return (int8_t)(int)c;
    }
}

template <int MODE>
__device__ __forceinline__ float scale_of(float m) {
    if constexpr (MODE == 0) return m / 127.0f;
    else if constexpr (MODE == 3) return m / 7.0f;
    else return m / 128.0f;
}

template <bool VEC, int MODE>
__global__ __launch_bounds__(256) void act_quant_kernel(const ActQuantTable tab, int k,
                                                        int32_t* __restrict__ status) {
    const float* __restrict__ x = tab.x[blockIdx.y];
    int8_t* __restrict__ q = tab.q[blockIdx.y];
    float* __restrict__ sx = tab.sx[blockIdx.y];
    const int t = tab.t;
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
    if constexpr (MODE == 2) {
        m = __uint_as_float(tab.tensor[0]);
        bad = tab.tensor[1] != 0u;
    }

    float r;
    const int flag = rowdiv<MODE>(m, bad, tab.eps, r);
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
            uint32_t p = (uint32_t)(uint8_t)code_of<MODE>(v.x, r, m) |
                         ((uint32_t)(uint8_t)code_of<MODE>(v.y, r, m) << 8) |
                         ((uint32_t)(uint8_t)code_of<MODE>(v.z, r, m) << 16) |
                         ((uint32_t)(uint8_t)code_of<MODE>(v.w, r, m) << 24);
            q4[i] = p;
        }
    } else {
        for (int i = lane; i < k; i += 64) qr[i] = code_of<MODE>(xr[i], r, m);
    }
    if (lane == 0) {
        sx[row] = flag ? __builtin_nanf("") : scale_of<MODE>(m);
        if (flag && status) atomicOr(status, flag);
    }
}

// Register-resident variant for rows of up to TPR * 4 * R floats (16-byte
// aligned, k % 4 == 0): TPR threads (8, 16 or 32 lanes of a wavefront, a
// wavefront, or a whole 256-thread workgroup) share one row, every element is
// read from HBM exactly once into registers, the row max is reduced with lane
// shuffles (and LDS across the workgroup's wavefronts), and the codes are
// written from the same registers.  All loads of a thread are issued before
// any is consumed.  Short rows share a wavefront so that a launch is not
// thousands of nearly idle workgroups.
template <int TPR, int R, int MODE>
__global__ __launch_bounds__(256) void act_quant_reg_kernel(const ActQuantTable tab, int k,
                                                            int32_t* __restrict__ status) {
    const float* __restrict__ x = tab.x[blockIdx.y];
    int8_t* __restrict__ q = tab.q[blockIdx.y];
    float* __restrict__ sx = tab.sx[blockIdx.y];
    const int t = tab.t;
    constexpr int RPW = 256 / TPR;                           // rows per workgroup
    __shared__ float red_m[4];
    __shared__ int red_bad[4];
    const int row = blockIdx.x * RPW + (int)threadIdx.x / TPR;
    const int sub = threadIdx.x % TPR;
    const int lane = threadIdx.x & 63;
    if constexpr (TPR <= 64) {                               // whole wavefronts exit together
        if (blockIdx.x * RPW + (int)(threadIdx.x >> 6) * (64 / TPR) >= t) return;
    }
    const bool row_ok = row < t;                             // (a wavefront's rows may run past t)
    const int rowc = row_ok ? row : t - 1;
    const int k4 = k >> 2;
    const float4* x4 = reinterpret_cast<const float4*>(x + (size_t)rowc * k);
    float4 v[R];
    #pragma unroll
    for (int i = 0; i < R; ++i) {
        const int idx = sub + i * TPR;
        v[i] = idx < k4 ? x4[idx] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
    float m = 0.0f;
    int bad = 0;
    #pragma unroll
    for (int i = 0; i < R; ++i) {
        bad |= !(isfinite(v[i].x) && isfinite(v[i].y) && isfinite(v[i].z) && isfinite(v[i].w));
        const float a0 = fabsf(v[i].x), a1 = fabsf(v[i].y), a2 = fabsf(v[i].z), a3 = fabsf(v[i].w);
        m = a0 > m ? a0 : m; m = a1 > m ? a1 : m; m = a2 > m ? a2 : m; m = a3 > m ? a3 : m;
    }
    if constexpr (TPR < 64) {                                // the row's lanes only
        #pragma unroll
        for (int off = TPR / 2; off > 0; off >>= 1) {
            const float o = __shfl_xor(m, off, 64);
            m = o > m ? o : m;
            bad |= __shfl_xor(bad, off, 64);
        }
    } else {
        m = wave_max(m);
        bad = wave_or(bad);
    }
    if constexpr (TPR == 256) {
        const int w = threadIdx.x >> 6;
        if (lane == 0) { red_m[w] = m; red_bad[w] = bad; }
        __syncthreads();
        #pragma unroll
        for (int i = 0; i < 4; ++i) { m = red_m[i] > m ? red_m[i] : m; bad |= red_bad[i]; }
    }
    if constexpr (MODE == 2) {
        m = __uint_as_float(tab.tensor[0]);
        bad = tab.tensor[1] != 0u;
    }
    float r;
    const int flag = rowdiv<MODE>(m, bad, tab.eps, r);
    uint32_t* q4 = reinterpret_cast<uint32_t*>(q + (size_t)rowc * k);
    #pragma unroll
    for (int i = 0; i < R; ++i) {
        const int idx = sub + i * TPR;
        if (idx < k4 && row_ok) {
            uint32_t p = 0u;   // a rejected row gets zero codes
            if (!flag)
                p = (uint32_t)(uint8_t)code_of<MODE>(v[i].x, r, m) |
                    ((uint32_t)(uint8_t)code_of<MODE>(v[i].y, r, m) << 8) |
                    ((uint32_t)(uint8_t)code_of<MODE>(v[i].z, r, m) << 16) |
                    ((uint32_t)(uint8_t)code_of<MODE>(v[i].w, r, m) << 24);
            q4[idx] = p;
        }
    }
    if (sub == 0 && row_ok) {
        sx[row] = flag ? __builtin_nanf("") : scale_of<MODE>(m);
        if (flag && status) atomicOr(status, flag);
    }
}

// One launch of the rule MODE over the table's n inputs.
template <int MODE>
hipError_t launch_table(const ActQuantTable& tab, int n, int t, int k, bool vec, int32_t* status,
                        hipStream_t stream) {
    const int k4 = k / 4;
    if (vec && k4 <= 8 * 8) {
        act_quant_reg_kernel<8, 8, MODE><<<dim3((unsigned)((t + 31) / 32), n), dim3(256), 0, stream>>>(tab, k, status);
    } else if (vec && k4 <= 16 * 8) {
        act_quant_reg_kernel<16, 8, MODE><<<dim3((unsigned)((t + 15) / 16), n), dim3(256), 0, stream>>>(tab, k, status);
    } else if (vec && k4 <= 32 * 8) {
        act_quant_reg_kernel<32, 8, MODE><<<dim3((unsigned)((t + 7) / 8), n), dim3(256), 0, stream>>>(tab, k, status);
    } else if (vec && k4 <= 64 * 8) {
        act_quant_reg_kernel<64, 8, MODE><<<dim3((unsigned)((t + 3) / 4), n), dim3(256), 0, stream>>>(tab, k, status);
    } else if (vec && k4 <= 256 * 4) {
        act_quant_reg_kernel<256, 4, MODE><<<dim3((unsigned)t, n), dim3(256), 0, stream>>>(tab, k, status);
    } else if (vec && k4 <= 256 * 16) {
        act_quant_reg_kernel<256, 16, MODE><<<dim3((unsigned)t, n), dim3(256), 0, stream>>>(tab, k, status);
    } else {
        dim3 grid((unsigned)((t + kActWaves - 1) / kActWaves), n), block(256);
        if (vec)
            act_quant_kernel<true, MODE><<<grid, block, 0, stream>>>(tab, k, status);
        else
            act_quant_kernel<false, MODE><<<grid, block, 0, stream>>>(tab, k, status);
    }
    return hipGetLastError();
}

hipError_t launch_act_quant_group(const float* const* x, int8_t* const* q, float* const* sx, int count, int t,
                                  int k, int32_t* status, hipStream_t stream) {
    for (int b = 0; b < count; b += kActQuantMaxSrc) {
        const int n = std::min(kActQuantMaxSrc, count - b);
        ActQuantTable tab{};
        tab.t = t;
        bool vec = k % 4 == 0;
        for (int i = 0; i < n; ++i) {
            tab.x[i] = x[b + i];
            tab.q[i] = q[b + i];
            tab.sx[i] = sx[b + i];
            vec = vec && (uintptr_t)x[b + i] % 16 == 0 && (uintptr_t)q[b + i] % 4 == 0;
        }
        hipError_t e = launch_table<0>(tab, n, t, k, vec, status, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_act_quant_v1(const float* x, int t, int k, float eps, const uint32_t* tensor, int8_t* q,
                               float* sx, int32_t* status, hipStream_t stream) {
    ActQuantTable tab{};
    tab.t = t;
    tab.x[0] = x;
    tab.q[0] = q;
    tab.sx[0] = sx;
    tab.eps = eps;
    tab.tensor = tensor;
    const bool vec = k % 4 == 0 && (uintptr_t)x % 16 == 0 && (uintptr_t)q % 4 == 0;
    return tensor ? launch_table<2>(tab, 1, t, k, vec, status, stream)
                  : launch_table<1>(tab, 1, t, k, vec, status, stream);
}

hipError_t launch_act_quant_a4(const float* x, int t, int k, int8_t* q, float* sx, int32_t* status,
                               hipStream_t stream) {
    ActQuantTable tab{};
    tab.t = t;
    tab.x[0] = x;
    tab.q[0] = q;
    tab.sx[0] = sx;
    const bool vec = k % 4 == 0 && (uintptr_t)x % 16 == 0 && (uintptr_t)q % 4 == 0;
    return launch_table<3>(tab, 1, t, k, vec, status, stream);
}

hipError_t launch_act_quant(const float* x, int t, int k, int8_t* q, float* sx, int32_t* status,
                            hipStream_t stream) {
    return launch_act_quant_group(&x, &q, &sx, 1, t, k, status, stream);
}

}  // namespace lowbit
