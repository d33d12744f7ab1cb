// sparse8.hip - BitNet a4.8's sparse 8-bit codes for intermediate states
// (gfx950).
//
// M8.8 "Native Binary and Ternary Transformers", 0x07B: the states in front of
// the attention output and FFN down projections are sparsified, then given
// 8-bit codes.  For each token row of x [t, k]:
//     keep the `keep` entries of largest |x| (at the threshold magnitude, the
//     lower channels first), set the others to zero,
//     m   = max |x| (always kept),  r = 127 / m,
//     q   = clip(rint(x r), -127, 127) where kept, else 0;  s_x = m / 127
// so the kept codes are exactly the dense per-token INT8 codes.
//
// One workgroup per row; the row stays in registers from load to store (up
// to 10 float4 per thread; 1024 threads per row when there are at most 64
// rows, for latency).  The threshold is a radix select over the 31-bit
// magnitude keys (the fp32 bits without the sign order like the magnitudes):
// three passes of 11, 10 and 10 bits from the top, each an LDS histogram of
// the keys that still match the chosen prefix, then a workgroup scan of the
// bins from the top finds the digit where the count of larger keys reaches
// the number still to keep.  Keys above the threshold are kept; keys equal to it
// are kept in channel order up to the remaining count, which needs a
// workgroup scan per register slot only when more keys tie at the threshold
// than may be kept (rare for real-valued rows).
//
// HBM-bound: 4 bytes read and 1 byte written per element, as the dense
// quantiser; the select runs on registers and LDS.
#include "device_common.hpp"
#include "kernels.hpp"

namespace lowbit {

namespace {

__device__ __forceinline__ float comp(const float4& v, int c) {
    return c == 0 ? v.x : (c == 1 ? v.y : (c == 2 ? v.z : v.w));
}

// |v|'s fp32 bits, recomputed at every use: as an ordinary expression the
// compiler keeps one key per element live beside the element itself (80 more
// registers at 40 elements per thread, and fewer rows per compute unit)
__device__ __forceinline__ uint32_t mag_key(float v) {
    uint32_t r;
    asm volatile("v_and_b32 %0, 0x7fffffff, %1" : "=v"(r) : "v"(v));
    return r;
}

constexpr int kBins = 2048;                     // the first digit's; the others use 1024

// The workgroup finds the bin, counted from the top, where the running count
// reaches rem (1 <= rem <= the histogram's total of NT BPT bins): thread i
// sums its BPT bins (the highest BPT for thread 0), a workgroup scan places
// the thread whose range holds the crossing, and that thread walks its bins.
// sel receives the bin, the count of keys above it and the count in it.
// Ends with the workgroup synchronised and sel visible to all.
template <int NT, int BPT>
__device__ __forceinline__ void pick_bin(const uint32_t* hist, uint32_t rem, uint32_t* wtot, uint32_t* sel) {
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lo = (NT - 1 - tid) * BPT;             // this thread's lowest bin
    uint32_t h[BPT];
    uint32_t s = 0u;
    #pragma unroll
    for (int j = 0; j < BPT; ++j) { h[j] = hist[lo + j]; s += h[j]; }
    uint32_t inc = s;
    #pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_up(inc, off, 64);
        if (lane >= off) inc += o;
    }
    if (lane == 63) wtot[w] = inc;
    __syncthreads();
    #pragma unroll
    for (int j = 0; j < NW; ++j) inc += j < w ? wtot[j] : 0u;
    const uint32_t exc = inc - s;
    if (exc < rem && rem <= inc) {                  // exactly one thread
        uint32_t above = exc, d = 0u, he = 0u;
        bool found = false;
        #pragma unroll
        for (int j = BPT - 1; j >= 0; --j) {
            if (!found) {
                if (above + h[j] >= rem) { found = true; d = (uint32_t)(lo + j); he = h[j]; }
                else above += h[j];
            }
        }
        sel[0] = d; sel[1] = above; sel[2] = he;
    }
    __syncthreads();
}

template <int NT, int R>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(6))) void sparse8_kernel(
        const float* __restrict__ x, int k, int keep, int8_t* __restrict__ q, float* __restrict__ sx,
        int32_t* __restrict__ status) {
    constexpr int NW = NT / 64;
    // two histograms: the first digit's 2048 bins (its lower half serves the
    // third digit), the second digit's 1024; each is cleared a pass ahead
    __shared__ __align__(16) uint32_t hist_a[kBins];
    __shared__ __align__(16) uint32_t hist_b[kBins / 2];
    __shared__ float red_m[NW];
    __shared__ int red_bad[NW];
    __shared__ uint32_t wtot[NW];
    __shared__ uint32_t sel[3];                 // chosen digit, keys above it, keys equal to it
    const int row = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int k4 = k >> 2;
    const float4* x4 = reinterpret_cast<const float4*>(x + (size_t)row * k);
    float4 v[R];
    #pragma unroll
    for (int i = 0; i < R; ++i) {
        const int idx = tid + i * NT;
        v[i] = idx < k4 ? x4[idx] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
    for (int i = tid; i < kBins / 4; i += NT) reinterpret_cast<uint4*>(hist_a)[i] = make_uint4(0u, 0u, 0u, 0u);
    for (int i = tid; i < kBins / 8; i += NT) reinterpret_cast<uint4*>(hist_b)[i] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    // the row max, finiteness, and the first digit's histogram (key bits
    // 30-20: the exponent and three mantissa bits, so that magnitudes of one
    // binade spread over eight bins and a wavefront's atomics rarely meet)
    float m = 0.0f;
    int bad = 0;
    #pragma unroll
    for (int i = 0; i < R; ++i) {
        bad |= !(isfinite(v[i].x) && isfinite(v[i].y) && isfinite(v[i].z) && isfinite(v[i].w));
        const float a0 = fabsf(v[i].x), a1 = fabsf(v[i].y), a2 = fabsf(v[i].z), a3 = fabsf(v[i].w);
        m = a0 > m ? a0 : m; m = a1 > m ? a1 : m; m = a2 > m ? a2 : m; m = a3 > m ? a3 : m;
        if (tid + i * NT < k4) {
            #pragma unroll
            for (int c = 0; c < 4; ++c) atomicAdd(&hist_a[mag_key(comp(v[i], c)) >> 20], 1u);
        }
    }
    m = wave_max(m);
    bad = wave_or(bad);
    if (lane == 0) { red_m[w] = m; red_bad[w] = bad; }
    __syncthreads();
    #pragma unroll
    for (int i = 0; i < NW; ++i) { m = red_m[i] > m ? red_m[i] : m; bad |= red_bad[i]; }
    int flag = 0;
    float r = 0.0f;
    if (bad) {
        flag = LOWBIT_ACT_NONFINITE;
    } else if (m > 0.0f) {
        r = 127.0f / m;
        if (!isfinite(r)) flag = LOWBIT_ACT_OVERFLOW;
    }

    // The threshold key T: keys above it are kept, and of the keys equal to
    // it the first `need` in channel order (all of them unless ranked).  A
    // pass whose chosen bin is kept whole ends the search, T then being the
    // digits so far with the lower bits zero.
    uint32_t T = 0u;
    uint32_t need = 0u;
    bool ranked = false;
    const bool select = !flag && m > 0.0f && keep < k;   // the same for every thread
    if (select) {
        uint32_t rem = (uint32_t)keep;
        pick_bin<NT, kBins / NT>(hist_a, rem, wtot, sel);
        T = sel[0] << 20;
        rem -= sel[1];
        if (rem != sel[2]) {                         // the second digit, key bits 19-10
            for (int i = tid; i < kBins / 8; i += NT)  // (the third digit's bins)
                reinterpret_cast<uint4*>(hist_a)[i] = make_uint4(0u, 0u, 0u, 0u);
            #pragma unroll
            for (int i = 0; i < R; ++i) {
                if (tid + i * NT < k4) {
                    #pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const uint32_t key = mag_key(comp(v[i], c));
                        if ((key & 0xfff00000u) == T) atomicAdd(&hist_b[(key >> 10) & 1023u], 1u);
                    }
                }
            }
            __syncthreads();
            pick_bin<NT, kBins / 2 / NT>(hist_b, rem, wtot, sel);
            T |= sel[0] << 10;
            rem -= sel[1];
            if (rem != sel[2]) {                     // the third digit, key bits 9-0
                #pragma unroll
                for (int i = 0; i < R; ++i) {
                    if (tid + i * NT < k4) {
                        #pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const uint32_t key = mag_key(comp(v[i], c));
                            if ((key & 0xfffffc00u) == T) atomicAdd(&hist_a[key & 1023u], 1u);
                        }
                    }
                }
                __syncthreads();
                pick_bin<NT, kBins / 2 / NT>(hist_a, rem, wtot, sel);
                T |= sel[0];
                rem -= sel[1];
                need = rem;
                ranked = sel[2] > rem && T != 0u;    // (zero magnitudes code to 0 kept or not)
            }
        }
    }

    // Kept: keys above T, and keys equal to T unless ranked; ranked ties are
    // kept by their channel order, their bits (4 per register slot) in rk.
    static_assert(R <= 16, "rk holds 4 bits per register slot");
    uint64_t rk = 0u;
    if (ranked) {
        // channel order is slot-major: channel 4 (tid + i NT) + c.  The ties
        // in slot i ahead of this thread's come from the slots before it
        // (base) and from lower threads in slot i (a workgroup scan).
        uint32_t base = 0u;
        #pragma unroll
        for (int i = 0; i < R; ++i) {
            uint32_t tie = 0u;
            if (tid + i * NT < k4) {
                #pragma unroll
                for (int c = 0; c < 4; ++c) tie |= (uint32_t)(mag_key(comp(v[i], c)) == T) << c;
            }
            const uint32_t cnt = __builtin_popcount(tie);
            uint32_t inc = cnt;
            #pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const uint32_t o = __shfl_up(inc, off, 64);
                if (lane >= off) inc += o;
            }
            if (lane == 63) wtot[w] = inc;
            __syncthreads();
            uint32_t before = base + inc - cnt, total = 0u;
            #pragma unroll
            for (int j = 0; j < NW; ++j) {
                const uint32_t tw = wtot[j];
                before += j < w ? tw : 0u;
                total += tw;
            }
            __syncthreads();                        // wtot is rewritten by the next slot
            #pragma unroll
            for (int c = 0; c < 4; ++c) {
                if ((tie >> c) & 1u) {
                    if (before < need) rk |= (uint64_t)1u << (4 * i + c);
                    ++before;
                }
            }
            base += total;
        }
    }

    uint32_t* q4 = reinterpret_cast<uint32_t*>(q + (size_t)row * k);
    #pragma unroll
    for (int i = 0; i < R; ++i) {
        const int idx = tid + i * NT;
        if (idx < k4) {
            uint32_t p = 0u;   // a rejected row gets zero codes
            if (!flag) {
                #pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float xv = comp(v[i], c);
                    const uint32_t key = mag_key(xv);
                    const bool kept = !select || key > T ||
                                      (key == T && (!ranked || ((rk >> (4 * i + c)) & 1u)));
                    if (kept) p |= (uint32_t)(uint8_t)quant1(xv, r) << (8 * c);
                }
            }
            q4[idx] = p;
        }
    }
    if (tid == 0) {
        sx[row] = flag ? __builtin_nanf("") : m / 127.0f;
        if (flag && status) atomicOr(status, flag);
    }
}

}  // namespace

hipError_t launch_act_quant_sparse8(const float* x, int t, int k, int keep, int8_t* q, float* sx, int32_t* status,
                                    hipStream_t stream) {
    const int k4 = k / 4;
    if (t <= 64 && k4 <= 1024 * 3) {
        // few rows (decode): a row's latency is the launch's, so spread each
        // row over 16 wavefronts (fewer serial atomics per thread)
        if (k4 <= 1024)
            sparse8_kernel<1024, 1><<<dim3((unsigned)t), dim3(1024), 0, stream>>>(x, k, keep, q, sx, status);
        else
            sparse8_kernel<1024, 3><<<dim3((unsigned)t), dim3(1024), 0, stream>>>(x, k, keep, q, sx, status);
        return hipGetLastError();
    }
    if (k4 <= 256 * 3)
        sparse8_kernel<256, 3><<<dim3((unsigned)t), dim3(256), 0, stream>>>(x, k, keep, q, sx, status);
    else if (k4 <= 256 * 10)
        sparse8_kernel<256, 10><<<dim3((unsigned)t), dim3(256), 0, stream>>>(x, k, keep, q, sx, status);
    else if (k4 <= 512 * 8)
        sparse8_kernel<512, 8><<<dim3((unsigned)t), dim3(512), 0, stream>>>(x, k, keep, q, sx, status);
    else
        sparse8_kernel<1024, 8><<<dim3((unsigned)t), dim3(1024), 0, stream>>>(x, k, keep, q, sx, status);
    return hipGetLastError();
}

}  // namespace lowbit
