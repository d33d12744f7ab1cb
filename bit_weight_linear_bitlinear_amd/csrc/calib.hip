// calib.hip - the two ceilings the products' roofline fractions are read
// against, measured on the device itself (the published figures are 8 TB/s
// of HBM and 5.0 POPS of dense int8 matrix-core work):
//  - a read stream: two workgroups per CU, each streaming its own contiguous
//    slab in 16-byte words with eight loads in flight per lane,
//    non-temporal (the data is used once), XOR-reduced so the loads cannot be
//    dropped; bytes / time is the achievable HBM read rate when the buffer is
//    several times the 256 MB last-level cache.  Over 2 GiB a grid-stride
//    walk measured 5.7-6.3 TB/s and slabs 6.9-7.1; the closing atomics cost
//    little only while they are few (one per workgroup of 512 workgroups:
//    7.0 TB/s; one per wavefront of 16384: 5.5);
//  - an int8 matrix-core loop: two wavefronts per SIMD on every CU, each
//    issuing v_mfma_i32_32x32x32_i8 back to back on eight independent
//    accumulators held in registers (no memory traffic); 65536 operations per
//    MFMA.
// Each kernel folds its result into one word with atomic XORs (one per
// workgroup for the read stream, per wavefront for the matrix-core loop),
// which the caller ignores.
#include "device_common.hpp"
#include "kernels.hpp"

namespace lowbit {

typedef int32_t i32x16c __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t wave_xor(uint32_t v) {
    #pragma unroll
    for (int off = 32; off > 0; off >>= 1) v ^= (uint32_t)__shfl_xor((int)v, off, 64);
    return v;
}

__global__ __launch_bounds__(256) void calib_read_kernel(const u32x4* __restrict__ src, int64_t words,
                                                         uint32_t* __restrict__ sink) {
    // each workgroup streams its own contiguous slab (the last one also the
    // remainder), eight 16-byte loads in flight per lane
    constexpr int U = 8;
    const int64_t per = words / gridDim.x;
    const int64_t begin = per * blockIdx.x;
    const int64_t end = blockIdx.x + 1 == gridDim.x ? words : begin + per;
    const u32x4* p = src + begin;
    const int64_t n = end - begin;
    uint32_t acc = 0;
    int64_t i = threadIdx.x;
    for (; i + (U - 1) * 256 < n; i += U * 256) {
        u32x4 v[U];
        #pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * 256);
        #pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < n; i += 256) {
        const u32x4 a = __builtin_nontemporal_load(p + i);
        acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
    }
    __shared__ uint32_t part[4];
    acc = wave_xor(acc);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) atomicXor(sink, part[0] ^ part[1] ^ part[2] ^ part[3]);
}

__global__ __launch_bounds__(256) void calib_mfma_i8_kernel(int iters, uint32_t* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    i32x4 a = {lane, lane * 3, lane * 5, lane * 7};
    i32x4 b = {lane * 11, lane * 13, lane * 17, lane * 19};
    i32x16c c0 = {}, c1 = {}, c2 = {}, c3 = {}, c4 = {}, c5 = {}, c6 = {}, c7 = {};
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c3, 0, 0, 0);
        c4 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c4, 0, 0, 0);
        c5 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c5, 0, 0, 0);
        c6 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c6, 0, 0, 0);
        c7 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c7, 0, 0, 0);
    }
    int r = 0;
    #pragma unroll
    for (int e = 0; e < 16; ++e) r ^= c0[e] ^ c1[e] ^ c2[e] ^ c3[e] ^ c4[e] ^ c5[e] ^ c6[e] ^ c7[e];
    const uint32_t rx = wave_xor((uint32_t)r);
    if (lane == 0) atomicXor(sink, rx);
}

hipError_t launch_calib_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
    const int grid = device_cu_count() * 2;
    calib_read_kernel<<<grid, 256, 0, stream>>>(static_cast<const u32x4*>(src), bytes / 16, sink);
    return hipGetLastError();
}

int64_t calib_mfma_i8_ops_per_iter() { return (int64_t)device_cu_count() * 2 * 4 * 8 * 65536; }

hipError_t launch_calib_mfma_i8(int32_t iters, uint32_t* sink, hipStream_t stream) {
    calib_mfma_i8_kernel<<<device_cu_count() * 2, 256, 0, stream>>>(iters, sink);
    return hipGetLastError();
}

}  // namespace lowbit
