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
// Work split.  A workgroup of four (or eight) wavefronts owns 16 TT tokens
// and 64 R (128 R) rows: each
// wavefront streams R 16-row tiles over all of k (R = 1 at decode; R = 4 at
// prefill, so that one staged operand serves 256 rows, or 8 with eight
// wavefronts per workgroup and 1024 rows where that still fills every CU:
// 8 x 4 accumulator tiles need two wavefronts per SIMD asked for, at a few
// spilled registers, and two staged groups in flight per thread instead of
// four), reusing each
// activation operand for its R tiles and each decoded sign operand for its
// TT token tiles (TT = 2 or 4 at prefill).  At decode with fewer than 1024
// tiles a workgroup instead owns one tile and its wavefronts split k four
// ways.  x * g of the tile's real tokens is staged up to 32 KB at a time (a
// decode row of up to 16384 codes in one pass; 64 KB at prefill), written as
// whole 16-byte groups of the permuted chunk.
#include <algorithm>

#include "device_common.hpp"
#include "kernels.hpp"

namespace lowbit {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kObLds = 32768;                     // bytes of staged x * g per workgroup
// Halves of padding after each staged token row.  The operand reads take 16
// token rows at one column (lane quarters 64 bytes apart); with rows of a
// whole number of kilobytes they met on the same banks.  Counters at 4096
// tokens: bank-conflict cycles 0.82 of the LDS's active cycles unpadded, 0.40
// with a pad of 8, 16 or 24 halves (16 the fastest: 4096^3 in 203 against
// ~230 us unpadded).
constexpr int kObPad = 16;
constexpr int kObBatch = 4;                       // staged 16-byte groups per thread whose loads fly together

struct OneBitArgs {
    const uint8_t* packed;
    const uint16_t* g;
    const uint16_t* h;
    const uint16_t* x;
    float* y;
    int n, k, t;
    int wpl, step_k, n_steps, n_tiles;
    int chunk;                                     // codes staged at a time: a multiple of 512
    int vec;                                       // x and g 16-byte aligned and k % 8 == 0
};

// R 16-row tiles per wavefront, four wavefronts: 64 R rows x 16 tokens; or
// (KS) one 16-row tile per workgroup whose four wavefronts take every fourth
// k-step, their fp32 partials summed in LDS
template <int WPL, int R, bool KS, int TT, int NWV>
__global__ __launch_bounds__(64 * NWV) __attribute__((amdgpu_waves_per_eu(R == 8 ? 2 : 1))) void onebit_kernel(const OneBitArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    _Float16* xs = reinterpret_cast<_Float16*>(smem);      // [tokens of this tile][chunk + kObPad]
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = lane >> 4, r = lane & 15;
    const int t0 = blockIdx.y * 16 * TT, tv = min(16 * TT, a.t - t0);   // tokens of this tile
    const int K = a.k, SK = a.step_k, CH = a.chunk;
    const int RS = CH + kObPad;                               // staged row stride (halves)
    constexpr int NB = R == 8 ? 2 : kObBatch;                  // (eight row tiles: fewer registers in flight)
    constexpr int NT = 64 * NWV;                              // threads per workgroup
    static_assert(!KS || NWV == 4, "k split over four wavefronts");
    const int tile0 = KS ? (int)blockIdx.x : (blockIdx.x * NWV + wave) * R;   // this wavefront's first row tile
    const uint8_t* pk[R];
    #pragma unroll
    for (int i = 0; i < R; ++i)
        pk[i] = a.packed + (size_t)min(tile0 + i, a.n_tiles - 1) * a.n_steps * (256 * WPL) +
                (size_t)(q * 16 + r) * WPL * 4;
    const bool x_vec = a.vec != 0;                            // rows of x and g 16-byte aligned

    f32x4 acc[R][TT];
    #pragma unroll
    for (int i = 0; i < R; ++i)
        #pragma unroll
        for (int u = 0; u < TT; ++u) acc[i][u] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const int kpad = a.n_steps * SK;
    for (int c0 = 0; c0 < kpad; c0 += CH) {
        const int cl = min(CH, kpad - c0);                    // a multiple of SK
        // stage fp16(x * g) of the real tokens; token rows past t are never
        // staged (their outputs, which depend only on their own row of the
        // operand, are not stored).  One unit is a 16-byte group of the
        // permuted chunk: positions 8 m .. 8 m + 7 of chunk c hold codes
        // 32 c + 4 m + j and 32 c + 16 + 4 m + j (j = 0 .. 3) interleaved, so a
        // thread reads two 8-byte runs of x and of g, multiplies them as fp16
        // pairs (the product of two fp16 values rounded once, as fp16(x * g)
        // computed in fp32 would be: that product is exact in fp32) and writes
        // one 16-byte word.  Each thread issues the loads of kObBatch units
        // before using any.
        const int n_pos = cl / 8;                             // groups per token row of this pass
        const int units = tv * n_pos;
        for (int e0 = 0; e0 < units; e0 += NT * NB) {
            u32x2 xl[NB], xh[NB], gl[NB], gh[NB];
            int ti[NB], kc[NB];
            bool fast[NB];
            #pragma unroll
            for (int u = 0; u < NB; ++u) {
                const int e = e0 + NT * u + tid;
                ti[u] = e / n_pos;
                const int pos = e - ti[u] * n_pos;
                kc[u] = c0 + 32 * (pos >> 2) + 4 * (pos & 3);   // code of the group's first half
                fast[u] = e < units && x_vec && kc[u] + 20 <= K;
                if (fast[u]) {
                    const uint16_t* xr = a.x + (size_t)(t0 + ti[u]) * K;
                    xl[u] = *reinterpret_cast<const u32x2*>(xr + kc[u]);
                    xh[u] = *reinterpret_cast<const u32x2*>(xr + kc[u] + 16);
                    gl[u] = *reinterpret_cast<const u32x2*>(a.g + kc[u]);
                    gh[u] = *reinterpret_cast<const u32x2*>(a.g + kc[u] + 16);
                }
            }
            #pragma unroll
            for (int u = 0; u < NB; ++u) {
                const int e = e0 + NT * u + tid;
                if (e >= units) continue;
                u32x4 o;
                if (fast[u]) {
                    // products of codes (kc, kc+1), (kc+2, kc+3), (kc+16, kc+17), (kc+18, kc+19)
                    uint32_t pr[4];
                    // (vector elements are copied out first: a bit_cast of an
                    // element expression compiled to the element 0 here)
                    #pragma unroll
                    for (int w2 = 0; w2 < 2; ++w2) {
                        const uint32_t xa = xl[u][w2], ga = gl[u][w2], xb = xh[u][w2], gb = gh[u][w2];
                        pr[w2] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2, xa) * __builtin_bit_cast(half2, ga));
                        pr[2 + w2] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2, xb) * __builtin_bit_cast(half2, gb));
                    }
                    // interleave: dword j = (code kc + j, code kc + 16 + j)
                    o[0] = __builtin_amdgcn_perm(pr[2], pr[0], 0x05040100u);
                    o[1] = __builtin_amdgcn_perm(pr[2], pr[0], 0x07060302u);
                    o[2] = __builtin_amdgcn_perm(pr[3], pr[1], 0x05040100u);
                    o[3] = __builtin_amdgcn_perm(pr[3], pr[1], 0x07060302u);
                } else {
                    auto prod = [](uint16_t xb, uint16_t gb) {
                        const _Float16 v = __builtin_bit_cast(_Float16, xb) * __builtin_bit_cast(_Float16, gb);
                        return (uint32_t)__builtin_bit_cast(uint16_t, v);
                    };
                    const uint16_t* xr = a.x + (size_t)(t0 + ti[u]) * K;
                    #pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int kl = kc[u] + j, kh = kc[u] + 16 + j;   // codes past k stage as 0: their +1 signs add nothing
                        const uint32_t lo = kl < K ? prod(xr[kl], a.g[kl]) : 0u;
                        const uint32_t hi = kh < K ? prod(xr[kh], a.g[kh]) : 0u;
                        o[j] = lo | (hi << 16);
                    }
                }
                const int pos = e - ti[u] * n_pos;
                *reinterpret_cast<u32x4*>(xs + ti[u] * RS + 32 * (pos >> 2) + 8 * (pos & 3)) = o;
            }
        }
        __syncthreads();
        const int s0 = c0 / SK, s1 = s0 + cl / SK;
        for (int s = s0 + (KS ? wave : 0); s < s1; s += KS ? 4 : 1) {
            uint32_t w[R][WPL];
            #pragma unroll
            for (int i = 0; i < R; ++i) {
                const uint8_t* p = pk[i] + (size_t)s * (256 * WPL);
                if constexpr (WPL == 4) {
                    const u32x4 v = *reinterpret_cast<const u32x4*>(p);
                    w[i][0] = v[0]; w[i][1] = v[1]; w[i][2] = v[2]; w[i][3] = v[3];
                } else if constexpr (WPL == 2) {
                    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
                    w[i][0] = v[0]; w[i][1] = v[1];
                } else {
                    w[i][0] = *reinterpret_cast<const uint32_t*>(p);
                }
            }
            #pragma unroll
            for (int ww = 0; ww < WPL; ++ww) {
                // this lane quarter's 32 codes of block ww: k = s SK + 128 ww + 32 q
                // (token rows past t read the last staged row: their outputs are dropped)
                const int kof = (s * SK - c0) + 128 * ww + 32 * q;
                #pragma unroll
                for (int m = 0; m < 4; ++m) {
                    half8 av[TT];
                    #pragma unroll
                    for (int u = 0; u < TT; ++u)
                        av[u] = *reinterpret_cast<const half8*>(xs + min(16 * u + r, tv - 1) * RS + kof + 8 * m);
                    #pragma unroll
                    for (int i = 0; i < R; ++i) {
                        u32x4 b;                                  // decoded once, used by the TT token tiles
                        #pragma unroll
                        for (int jj = 0; jj < 4; ++jj) {
                            const int c = 4 * m + jj;
                            b[jj] = ((w[i][ww] << (15 - c)) & 0x80008000u) | 0x3C003C00u;
                        }
                        #pragma unroll
                        for (int u = 0; u < TT; ++u)
                            acc[i][u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[u], __builtin_bit_cast(half8, b),
                                                                              acc[i][u], 0, 0, 0);
                    }
                }
            }
        }
        __syncthreads();                                   // before the next chunk overwrites xs
    }
    if constexpr (KS) {                                       // the four partials, in wave order
        f32x4* red = reinterpret_cast<f32x4*>(smem);
        red[wave * 64 + lane] = acc[0][0];
        __syncthreads();
        if (wave != 0) return;
        acc[0][0] = ((acc[0][0] + red[64 + lane]) + red[128 + lane]) + red[192 + lane];
    }
    // acc[i][u] element e of lane (q, r): token 16 u + 4q + e, row r of tile tile0 + i
    #pragma unroll
    for (int i = 0; i < R; ++i) {
        const int n = (tile0 + i) * 16 + r;
        if (n < a.n) {
            const float hv = (float)__builtin_bit_cast(_Float16, a.h[n]);
            #pragma unroll
            for (int u = 0; u < TT; ++u)
                #pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int tt = t0 + 16 * u + 4 * q + e;
                    if (tt < a.t) a.y[(size_t)tt * a.n + n] = acc[i][u][e] * hv;
                }
        }
    }
}

template <int R, bool KS, int TT, int NWV = 4>
void launch_r(const OneBitArgs& a, dim3 grid, size_t lds, hipStream_t stream) {
    switch (a.wpl) {
        case 4: onebit_kernel<4, R, KS, TT, NWV><<<grid, 64 * NWV, lds, stream>>>(a); break;
        case 2: onebit_kernel<2, R, KS, TT, NWV><<<grid, 64 * NWV, lds, stream>>>(a); break;
        default: onebit_kernel<1, R, KS, TT, NWV><<<grid, 64 * NWV, lds, stream>>>(a); break;
    }
}

}  // namespace

hipError_t launch_onebit(const uint8_t* packed, const uint16_t* g, const uint16_t* h, const uint16_t* x, float* y,
                         int n, int k, int t, int wpl, int step_k, int n_steps, hipStream_t stream) {
    const int tiles = (n + 15) / 16;
    const bool prefill = t > 16;                   // two (or four) 16-token tiles per workgroup
    // four token tiles per workgroup (each decoded sign operand feeds four
    // MFMAs) while that still leaves two workgroups per CU
    const bool tt4 = prefill && (int64_t)((tiles + 15) / 16) * ((t + 63) / 64) >= 2LL * device_cu_count();
    const int tv = std::min(t, prefill ? (tt4 ? 64 : 32) : 16);
    // staged codes per pass: what the stage (32 KB, 64 KB at prefill) holds
    // for the tile's tokens, a multiple of 512 (every k-step size divides it)
    const int budget = prefill ? 2 * kObLds : kObLds;
    const int chunk = std::max(512, (budget / (2 * tv)) / 512 * 512);
    const int vec = k % 8 == 0 && (uintptr_t)x % 16 == 0 && (uintptr_t)g % 16 == 0;
    OneBitArgs a{packed, g, h, x, y, n, k, t, wpl, step_k, n_steps, tiles, chunk, vec};
    const size_t lds = (size_t)2 * tv * (chunk + kObPad);
    // prefill: 256 rows and 32 or 64 tokens per workgroup, so that one staged
    // operand serves 256 rows and one decoded sign operand two or four token
    // tiles; decode: 64 rows, or one tile with k split four ways when that
    // leaves under 256 workgroups, so that small and short-wide matrices
    // spread over the chip
    // eight row tiles per wavefront and eight wavefronts per workgroup (1024
    // rows per staged operand: a quarter of the staging per row; one
    // workgroup per CU) while that still fills every CU
    const bool w8 = tt4 && (int64_t)((tiles + 63) / 64) * ((t + 63) / 64) >= device_cu_count();
    if (w8) launch_r<8, false, 4, 8>(a, dim3((unsigned)((tiles + 63) / 64), (unsigned)((t + 63) / 64)), lds, stream);
    else if (tt4) launch_r<4, false, 4>(a, dim3((unsigned)((tiles + 15) / 16), (unsigned)((t + 63) / 64)), lds, stream);
    else if (prefill) launch_r<4, false, 2>(a, dim3((unsigned)((tiles + 15) / 16), (unsigned)((t + 31) / 32)), lds, stream);
    else if (tiles < 1024) launch_r<1, true, 1>(a, dim3((unsigned)tiles, (unsigned)((t + 15) / 16)), lds, stream);
    else launch_r<1, false, 1>(a, dim3((unsigned)((tiles + 3) / 4), (unsigned)((t + 15) / 16)), lds, stream);
    return hipGetLastError();
}

}  // namespace lowbit
