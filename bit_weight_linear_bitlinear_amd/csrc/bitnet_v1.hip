// bitnet_v1.hip - the pieces of the original BitNet BitLinear forward that
// the int8 path does not already have (gfx950).
//
// M8.8 "Native Binary and Ternary Transformers", 0x02B-0x02E: the input of a
// BitLinear is normalised by a sub-layer LayerNorm, then coded with Q_b = 128
// against its max |x| - per token at inference, per tensor in training - and
// multiplied by centered-sign binary weights.  The codes come from the int8
// quantiser's kernels (act_quant.hip, rules MODE 1 and 2) and the product from
// the existing GEMV / GEMM; here are
//  - the tensor-wide max |x| for the per-tensor rule: a workspace is cleared
//    by a one-wavefront kernel (not a memset, so a captured graph replays it),
//    then each of at most 512 workgroups reduces a grid-strided share and
//    merges it with one atomicMax on the fp32 bits (|x| >= 0 orders like its
//    bits) and one atomicOr of a non-finite flag;
//  - LayerNorm without (or with) an affine map: a wavefront per row, fp32
//    sums reduced across lanes, mean first, then the centred second moment.
#include <math.h>

#include <algorithm>

#include "device_common.hpp"
#include "kernels.hpp"

namespace lowbit {

namespace {

__global__ void clear_tensor_max_kernel(uint32_t* __restrict__ w) {
    if (threadIdx.x < 2) w[threadIdx.x] = 0u;
}

template <bool VEC>
__global__ __launch_bounds__(256) void tensor_absmax_kernel(const float* __restrict__ x, int64_t n,
                                                            uint32_t* __restrict__ w) {
    float m = 0.0f;
    int bad = 0;
    const int64_t stride = (int64_t)gridDim.x * 256;
    if (VEC) {
        const float4* x4 = reinterpret_cast<const float4*>(x);
        for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n / 4; i += stride) {
            const float4 v = x4[i];
            bad |= !(isfinite(v.x) && isfinite(v.y) && isfinite(v.z) && isfinite(v.w));
            m = fmaxf(fmaxf(m, fabsf(v.x)), fmaxf(fabsf(v.y), fmaxf(fabsf(v.z), fabsf(v.w))));
        }
    } else {
        for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
            const float v = x[i];
            bad |= !isfinite(v);
            m = fmaxf(m, fabsf(v));
        }
    }
    // one atomic per workgroup: the wavefronts' results meet in LDS first
    // (thousands of atomics on one address serialise at the L2)
    __shared__ float red_m[4];
    __shared__ int red_bad[4];
    m = wave_max(m);
    bad = wave_or(bad);
    if ((threadIdx.x & 63) == 0) { red_m[threadIdx.x >> 6] = m; red_bad[threadIdx.x >> 6] = bad; }
    __syncthreads();
    if (threadIdx.x == 0) {
        m = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));
        bad = red_bad[0] | red_bad[1] | red_bad[2] | red_bad[3];
        if (bad) atomicOr(&w[1], 1u);
        atomicMax(&w[0], __float_as_uint(m));
    }
}

// a wavefront per row; four rows per 256-thread workgroup
// (x and out may be one buffer: each lane reads an element before it writes it)
__global__ __launch_bounds__(256) void layernorm_kernel(const float* x, int t, int d, float eps,
                                                        const float* __restrict__ g, const float* __restrict__ b,
                                                        float* out) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (row >= t) return;
    const float* xr = x + (size_t)row * d;
    float* yr = out + (size_t)row * d;
    float s = 0.0f;
    for (int i = lane; i < d; i += 64) s += xr[i];
    #pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    const float mean = s / (float)d;
    float v = 0.0f;
    for (int i = lane; i < d; i += 64) {
        const float c = xr[i] - mean;
        v += c * c;
    }
    #pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    const float inv = 1.0f / sqrtf(v / (float)d + eps);
    for (int i = lane; i < d; i += 64) {
        float y = (xr[i] - mean) * inv;
        if (g) y = y * g[i];
        if (b) y = y + b[i];
        yr[i] = y;
    }
}

}  // namespace

hipError_t launch_tensor_absmax(const float* x, int64_t n, uint32_t* work, hipStream_t stream) {
    clear_tensor_max_kernel<<<1, 64, 0, stream>>>(work);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const bool vec = n % 4 == 0 && (uintptr_t)x % 16 == 0;
    const int64_t items = vec ? n / 4 : n;
    const unsigned grid = (unsigned)std::min<int64_t>(std::max<int64_t>((items + 1023) / 1024, 1), 512);
    if (vec)
        tensor_absmax_kernel<true><<<grid, 256, 0, stream>>>(x, n, work);
    else
        tensor_absmax_kernel<false><<<grid, 256, 0, stream>>>(x, n, work);
    return hipGetLastError();
}

hipError_t launch_layernorm(const float* x, int t, int d, float eps, const float* g, const float* b, float* out,
                            hipStream_t stream) {
    layernorm_kernel<<<(unsigned)((t + 3) / 4), 256, 0, stream>>>(x, t, d, eps, g, b, out);
    return hipGetLastError();
}

}  // namespace lowbit
