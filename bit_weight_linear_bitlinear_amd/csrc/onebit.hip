// onebit.hip - OneBit's W1A16 projection on the gfx950 matrix cores.
//
// M8.8 "Native Binary and Ternary Transformers", 0x06A: a sign matrix S
// (+1 / -1, packed one bit per weight in the binary layout), an FP16 input
// vector g and an FP16 output vector h:
//     y[t, n] = h[n] * sum_k S[n, k] * fp16(x[t, k] * g[k])
// (the LayerNorm that follows is lowbit_layernorm).  The activations stay
// 16-bit, so the contraction is v_mfma_f32_16x16x32_f16: fp16 products,
// exact for +-1 times an fp16 value, accumulated in fp32.
//
// Sign decode.  A packed word holds 32 sign bits of one row (bit c set =
// code -1).  Shifting the word left by 15 - c puts bit c at bit 15 and bit
// c + 16 at bit 31, the sign bits of the two halves of a dword; one AND-OR
// with 0x80008000 and 1.0 in both halves (0x3C003C00) yields the operand pair
// (code c, code c + 16): two instructions per two codes, no table.  MFMA m of
// a word takes pairs c = 4m .. 4m + 3.
//
// Activation operand.  x * g is rounded to fp16 once and staged in LDS for
// the workgroup's 16 tokens, each 32-code chunk permuted so that the eight
// halves an MFMA lane needs - codes c, c + 16 for c = 4m .. 4m + 3, in that
// order - are contiguous (position 8 (c / 4) + 2 (c % 4), + 1 for c + 16).
// An MFMA sums over whichever k its lanes supply as long as the two
// operands name the same k: lane quarter q takes the packed lane group q's
// words (k offsets 32q .. 32q + 31 of each 128-code block) and the staged
// halves of the same codes.  Codes past k stage as 0, so the padding signs
// (+1) add nothing.
//
// Work split.  A 256-thread workgroup owns one 16-row tile and 16 tokens;
// its four wavefronts take every fourth packed k-step, and their fp32
// partials meet in LDS.  The workgroup stages 1024 codes of x * g at a time
// (32 KB of LDS, so that several workgroups share a CU).
#include <algorithm>

#include "device_common.hpp"
#include "kernels.hpp"

namespace lowbit {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kObChunk = 1024;                    // codes of x * g staged at a time (32 KB)

struct OneBitArgs {
    const uint8_t* packed;
    const uint16_t* g;
    const uint16_t* h;
    const uint16_t* x;
    float* y;
    int n, k, t;
    int wpl, step_k, n_steps;
};

__device__ __forceinline__ int perm32(int c) {    // staged position of code c of a 32-code chunk
    return c < 16 ? 8 * (c >> 2) + 2 * (c & 3) : 8 * ((c - 16) >> 2) + 2 * (c & 3) + 1;
}

template <int WPL>
__global__ __launch_bounds__(256) void onebit_kernel(const OneBitArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    _Float16* xs = reinterpret_cast<_Float16*>(smem);      // [16 tokens][kObChunk]
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4, r = lane & 15;
    const int tile = blockIdx.x, t0 = blockIdx.y * 16;
    const int K = a.k, SK = a.step_k;
    const uint8_t* pk = a.packed + (size_t)tile * a.n_steps * (256 * WPL) + (size_t)(q * 16 + r) * WPL * 4;

    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    const int kpad = a.n_steps * SK;
    for (int c0 = 0; c0 < kpad; c0 += kObChunk) {
        const int cl = min(kObChunk, kpad - c0);           // a multiple of SK (kObChunk is)
        // stage fp16(x * g) for the 16 tokens, permuted within 32-code chunks
        for (int e = tid; e < 16 * cl; e += 256) {
            const int ti = e / cl, kk = e - ti * cl, kg = c0 + kk, tt = t0 + ti;
            _Float16 v = (_Float16)0.0f;
            if (tt < a.t && kg < K) {
                const float xf = (float)__builtin_bit_cast(_Float16, a.x[(size_t)tt * K + kg]);
                const float gf = (float)__builtin_bit_cast(_Float16, a.g[kg]);
                v = (_Float16)(xf * gf);                   // exact in fp32, one rounding to fp16
            }
            xs[ti * kObChunk + (kk & ~31) + perm32(kk & 31)] = v;
        }
        __syncthreads();
        const int s_end = c0 / SK + cl / SK;
        for (int s = c0 / SK + wave; s < s_end; s += 4) {
            uint32_t w[WPL];
            if constexpr (WPL == 4) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(pk + (size_t)s * (256 * WPL));
                w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
            } else if constexpr (WPL == 2) {
                const u32x2 v = *reinterpret_cast<const u32x2*>(pk + (size_t)s * (256 * WPL));
                w[0] = v[0]; w[1] = v[1];
            } else {
                w[0] = *reinterpret_cast<const uint32_t*>(pk + (size_t)s * (256 * WPL));
            }
            #pragma unroll
            for (int ww = 0; ww < WPL; ++ww) {
                // this lane quarter's 32 codes of block ww: k = s SK + 128 ww + 32 q
                const _Float16* arow = xs + r * kObChunk + (s * SK - c0) + 128 * ww + 32 * q;
                #pragma unroll
                for (int m = 0; m < 4; ++m) {
                    u32x4 b;
                    #pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int c = 4 * m + i;
                        b[i] = ((w[ww] << (15 - c)) & 0x80008000u) | 0x3C003C00u;
                    }
                    const half8 av = *reinterpret_cast<const half8*>(arow + 8 * m);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, __builtin_bit_cast(half8, b), acc, 0, 0, 0);
                }
            }
        }
        __syncthreads();                                   // before the next chunk overwrites xs
    }
    // the four wavefronts' partials: acc element e of lane (q, r) is token
    // 4q + e of the tile's 16, row r of its 16
    f32x4* red = reinterpret_cast<f32x4*>(smem);
    red[wave * 64 + lane] = acc;
    __syncthreads();
    if (wave == 0) {
        const f32x4 s1 = red[64 + lane], s2 = red[128 + lane], s3 = red[192 + lane];
        const int n = tile * 16 + r;
        if (n < a.n) {
            const float hv = (float)__builtin_bit_cast(_Float16, a.h[n]);
            #pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int tt = t0 + 4 * q + e;
                if (tt < a.t) a.y[(size_t)tt * a.n + n] = (((acc[e] + s1[e]) + s2[e]) + s3[e]) * hv;
            }
        }
    }
}

}  // namespace

hipError_t launch_onebit(const uint8_t* packed, const uint16_t* g, const uint16_t* h, const uint16_t* x, float* y,
                         int n, int k, int t, int wpl, int step_k, int n_steps, hipStream_t stream) {
    OneBitArgs a{packed, g, h, x, y, n, k, t, wpl, step_k, n_steps};
    const dim3 grid((unsigned)((n + 15) / 16), (unsigned)((t + 15) / 16));
    const size_t lds = (size_t)16 * kObChunk * 2;
    switch (wpl) {
        case 4: onebit_kernel<4><<<grid, 256, lds, stream>>>(a); break;
        case 2: onebit_kernel<2><<<grid, 256, lds, stream>>>(a); break;
        default: onebit_kernel<1><<<grid, 256, lds, stream>>>(a); break;
    }
    return hipGetLastError();
}

}  // namespace lowbit
