// gemm.hip - prefill-shaped low-bit product on the gfx950 matrix cores.
//
// What it computes (M8.8 "Native Binary and Ternary Transformers", 0x02D,
// 0x09C): acc[t, n] = sum_k q[t, k] * code[n, k] exactly in int32 (per scale
// group in group mode), then the fp32 rescale.  Prefill is a genuine dense
// contraction ("prefill ... competes with highly optimised dense GEMMs",
// 0x09B), so it runs on v_mfma_i32_16x16x64_i8.
//
// Tiling.  A 256-thread workgroup owns a 128-token x 128-row output tile and
// walks k in steps of 128.  Each step stages the token tile (128 x 128 int8
// codes, rows padded to 144 B against bank conflicts) and the *packed* weight
// tile (128 rows x 16/32/64 B for binary/ternary/int4) in LDS, double
// buffered, with the next step's global loads in flight during the MFMAs.
// The four wavefronts are a 2 x 2 grid of 64 x 64 sub-tiles (4 x 4 MFMA
// blocks of 16 x 16).  Weight codes are decoded from packed LDS words into
// operand registers right before their MFMAs (shift + mask per 4 codes), so
// LDS holds and serves the packed bytes only.  Binary activations are
// permuted within each 32-byte chunk while being staged, to match the page's
// packbits code order.
#include "device_common.hpp"
#include "kernels.hpp"

namespace lowbit {

struct GemmArgs {
    const uint8_t* packed;
    const float* scales;
    const int8_t* q;
    const float* sx;
    float* y;
    int32_t* acc;
    int wpl;            // packed layout: words per (lane group, row) per layout k-step
    int lay_steps;      // packed layout: k-steps per row
    int n_rows_pad;     // 16 * ceil(N / 16): rows present in the packed buffer
    int T, N, K;
    int n_steps;        // ceil(K / 128)
    int group;          // group mode: columns per group
    int G;              // group mode: groups per row (else 1)
    int scale_per_row;
    int q_aligned;      // K % 16 == 0 and q 16-byte aligned
};

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int A_STRIDE = BK + 16;   // bytes per staged token row

template <int FMT> struct GemmFmt {
    static constexpr int kRowBytes = BK / Fmt<FMT>::kCodesPerWord * 4;   // packed bytes per row per step
    static constexpr int kBStride = kRowBytes + 8;                       // staged row stride
};

template <int FMT, bool GROUP>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs a) {
    constexpr int SHIFT = Fmt<FMT>::kShift;
    constexpr int WB = GemmFmt<FMT>::kRowBytes;
    constexpr int BS = GemmFmt<FMT>::kBStride;
    constexpr int A_BYTES = BM * A_STRIDE;
    constexpr int B_BYTES = BN * BS;
    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (A_BYTES + B_BYTES)];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, rl = lane & 15;
    const int wm = wave >> 1, wn = wave & 1;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const bool q_aligned = a.q_aligned != 0;

    // ---- global -> register staging: 4 x 16 B of activations per thread
    // (binary: 2 x 32 B chunks), and the weight tile's packed words gathered
    // from the tiled layout into per-row order (word i of a row's 128-k slice:
    // block i / (4 * WB), lane-group quarter, half).
    constexpr int B_WORDS = BN * WB / 4;                   // words in the weight tile
    constexpr int B_PER_THREAD = B_WORDS / 256;
    constexpr int KBLK = FMT == FMT_BINARY ? 128 : 64;     // k per layout block
    constexpr int WBW = FMT == FMT_INT4 ? 2 : 1;           // words per lane group per block
    i32x4 ra[4];
    uint32_t rb[B_PER_THREAD];

    // activation pieces: 16 B (ternary, int4) or 32 B (binary, so one thread
    // can permute a whole 32-code word's worth of activations)
    constexpr int PB = FMT == FMT_BINARY ? 32 : 16;
    constexpr int PIECES_PER_ROW = BK / PB;
    constexpr int PIECES_PER_THREAD = BM * BK / PB / 256;      // 4 or 2
    auto load_a = [&](int step) {
        #pragma unroll
        for (int i = 0; i < PIECES_PER_THREAD; ++i) {
            const int c = tid + 256 * i;
            const int r = c / PIECES_PER_ROW, kk = (c % PIECES_PER_ROW) * PB;
            const int t = m0 + r;
            #pragma unroll
            for (int h = 0; h < PB / 16; ++h) {
                const int k0 = step * BK + kk + 16 * h;
                i32x4 v = {0, 0, 0, 0};
                if (t < a.T && k0 < a.K) {
                    const int8_t* p = a.q + (size_t)t * a.K + k0;
                    if (q_aligned) {
                        v = *reinterpret_cast<const i32x4*>(p);
                    } else {
                        const int valid = a.K - k0;
                        #pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int vj = valid - 4 * j;
                            v[j] = vj <= 0 ? 0 : (int32_t)load_u32_partial(reinterpret_cast<const uint8_t*>(p) + 4 * j, vj < 4 ? vj : 4);
                        }
                    }
                }
                ra[i * (PB / 16) + h] = v;
            }
        }
    };
    auto load_b = [&](int step) {
        const int nb_step = a.wpl / WBW;                   // layout blocks per layout k-step
        #pragma unroll
        for (int i = 0; i < B_PER_THREAD; ++i) {
            const int c = tid + 256 * i;
            const int r = c / (WB / 4), wi = c % (WB / 4);
            const int b = wi / (4 * WBW), gq = (wi / WBW) % 4, h = wi % WBW;
            const int blk = step * (BK / KBLK) + b;          // layout block along k
            const int ls = blk / nb_step, w = (blk % nb_step) * WBW + h;
            const int n = n0 + r;
            uint32_t v = 0;
            if (n < a.n_rows_pad && ls < a.lay_steps) {
                const size_t off = ((((size_t)(n >> 4) * a.lay_steps + ls) * 4 + gq) * 16 + (n & 15)) * a.wpl + w;
                v = reinterpret_cast<const uint32_t*>(a.packed)[off];
            }
            rb[i] = v;
        }
    };
    auto store_tiles = [&](int buf) {
        uint8_t* As = smem + buf * (A_BYTES + B_BYTES);
        uint8_t* Bs = As + A_BYTES;
        #pragma unroll
        for (int i = 0; i < PIECES_PER_THREAD; ++i) {
            const int c = tid + 256 * i;
            const int r = c / PIECES_PER_ROW, kk = (c % PIECES_PER_ROW) * PB;
            if constexpr (FMT == FMT_BINARY) {
                const uint32_t X[8] = {(uint32_t)ra[2 * i][0], (uint32_t)ra[2 * i][1], (uint32_t)ra[2 * i][2],
                                       (uint32_t)ra[2 * i][3], (uint32_t)ra[2 * i + 1][0], (uint32_t)ra[2 * i + 1][1],
                                       (uint32_t)ra[2 * i + 1][2], (uint32_t)ra[2 * i + 1][3]};
                i32x4 a0, a1;
                perm_binary_a(X, a0, a1);
                *reinterpret_cast<i32x4*>(As + r * A_STRIDE + kk) = a0;
                *reinterpret_cast<i32x4*>(As + r * A_STRIDE + kk + 16) = a1;
            } else {
                *reinterpret_cast<i32x4*>(As + r * A_STRIDE + kk) = ra[i];
            }
        }
        #pragma unroll
        for (int i = 0; i < B_PER_THREAD; ++i) {
            const int c = tid + 256 * i;
            const int r = c / (WB / 4), wi = c % (WB / 4);
            *reinterpret_cast<uint32_t*>(Bs + r * BS + 4 * wi) = rb[i];
        }
    };

    i32x4 C[4][4];
    float yp[GROUP ? 4 : 1][GROUP ? 4 : 1][4];
    #pragma unroll
    for (int i = 0; i < 4; ++i)
        #pragma unroll
        for (int j = 0; j < 4; ++j) C[i][j] = i32x4{0, 0, 0, 0};
    if constexpr (GROUP) {
        #pragma unroll
        for (int i = 0; i < 4; ++i)
            #pragma unroll
            for (int j = 0; j < 4; ++j)
                #pragma unroll
                for (int r = 0; r < 4; ++r) yp[i][j][r] = 0.0f;
    }

    // group epilogue after the codes of columns < kdone have been summed
    auto group_epilogue = [&](int kdone) {
        const int gi = (kdone - 1) / a.group;
        #pragma unroll
        for (int tj = 0; tj < 4; ++tj) {
            const int n = n0 + wn * 64 + tj * 16 + rl;
            const float sg = n < a.N ? a.scales[((size_t)(n >> 4) * a.G + gi) * 16 + (n & 15)] : 0.0f;   // tiled
            #pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                #pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int32_t av = C[ti][tj][r] >> SHIFT;
                    yp[ti][tj][r] = yp[ti][tj][r] + sg * (float)av;
                    if (a.acc) {
                        const int t = m0 + wm * 64 + ti * 16 + 4 * g + r;
                        if (t < a.T && n < a.N) a.acc[((size_t)t * a.N + n) * a.G + gi] = av;
                    }
                }
                C[ti][tj] = i32x4{0, 0, 0, 0};
            }
        }
    };

    load_a(0);
    load_b(0);
    for (int s = 0; s < a.n_steps; ++s) {
        const int buf = s & 1;
        store_tiles(buf);
        __syncthreads();
        if (s + 1 < a.n_steps) {   // next step's loads fly during this step's MFMAs
            load_a(s + 1);
            load_b(s + 1);
        }
        const uint8_t* As = smem + buf * (A_BYTES + B_BYTES);
        const uint8_t* Bs = As + A_BYTES;

        #pragma unroll
        for (int slot = 0; slot < 2; ++slot) {
            i32x4 Aop[4], Bop[4];
            #pragma unroll
            for (int ti = 0; ti < 4; ++ti) {
                const int r = wm * 64 + ti * 16 + rl;
                int koff;
                if constexpr (FMT == FMT_BINARY) koff = 32 * g + 16 * slot;   // permuted 32 B pieces
                else koff = 64 * slot + 16 * g;
                Aop[ti] = *reinterpret_cast<const i32x4*>(As + r * A_STRIDE + koff);
            }
            #pragma unroll
            for (int tj = 0; tj < 4; ++tj) {
                const uint8_t* brow = Bs + (wn * 64 + tj * 16 + rl) * BS;
                if constexpr (FMT == FMT_TERNARY) {
                    const uint32_t w = *reinterpret_cast<const uint32_t*>(brow + 4 * (4 * slot + g));
                    Bop[tj] = decode_ternary(w);
                } else if constexpr (FMT == FMT_INT4) {
                    const u32x2 w = *reinterpret_cast<const u32x2*>(brow + 4 * (8 * slot + 2 * g));
                    Bop[tj] = decode_int4(w[0], w[1]);
                } else {
                    const uint32_t w = *reinterpret_cast<const uint32_t*>(brow + 4 * g);
                    i32x4 o0, o1;
                    decode_binary(w, o0, o1);
                    Bop[tj] = slot == 0 ? o0 : o1;
                }
            }
            #pragma unroll
            for (int ti = 0; ti < 4; ++ti)
                #pragma unroll
                for (int tj = 0; tj < 4; ++tj) C[ti][tj] = mfma16(Aop[ti], Bop[tj], C[ti][tj]);

            if constexpr (GROUP) {
                // k covered so far: ternary/int4 slots are 64-column blocks;
                // a binary step's two slots share all 128 columns
                // (only a slot that holds valid columns can close a group)
                int kbeg, kdone;
                if constexpr (FMT == FMT_BINARY) { kbeg = s * BK; kdone = slot == 1 ? (s + 1) * BK : 0; }
                else { kbeg = s * BK + 64 * slot; kdone = kbeg + 64; }
                if (kdone > 0 && kbeg < a.K) {
                    if (kdone > a.K) kdone = a.K;
                    if (kdone % a.group == 0 || kdone == a.K) group_epilogue(kdone);
                }
            }
        }
    }

    // ---- epilogue
    #pragma unroll
    for (int tj = 0; tj < 4; ++tj) {
        const int n = n0 + wn * 64 + tj * 16 + rl;
        if (n >= a.N) continue;
        const float sw = GROUP ? 0.0f : a.scales[a.scale_per_row ? n : 0];
        #pragma unroll
        for (int ti = 0; ti < 4; ++ti) {
            #pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = m0 + wm * 64 + ti * 16 + 4 * g + r;
                if (t >= a.T) continue;
                if constexpr (GROUP) {
                    a.y[(size_t)t * a.N + n] = a.sx[t] * yp[ti][tj][r];
                } else {
                    const int32_t av = C[ti][tj][r] >> SHIFT;
                    a.y[(size_t)t * a.N + n] = (float)av * (a.sx[t] * sw);
                    if (a.acc) a.acc[(size_t)t * a.N + n] = av;
                }
            }
        }
    }
}

// the general path: any k, any alignment (ragged tails read byte by byte)
hipError_t launch_gemm_generic(const LinearArgs& a, hipStream_t stream) {
    GemmArgs ga;
    ga.packed = a.packed; ga.scales = a.scales; ga.q = a.q; ga.sx = a.sx; ga.y = a.y; ga.acc = a.acc;
    ga.wpl = a.wpl; ga.lay_steps = a.n_steps; ga.n_rows_pad = (a.n + 15) / 16 * 16;
    ga.T = a.t; ga.N = a.n; ga.K = a.k;
    ga.n_steps = (a.k + BK - 1) / BK;
    ga.group = a.scale == LOWBIT_SCALE_GROUP ? a.group : 0;
    ga.G = a.scale == LOWBIT_SCALE_GROUP ? a.n_groups : 1;
    ga.scale_per_row = a.scale == LOWBIT_SCALE_ROW;
    ga.q_aligned = (a.k % 16 == 0) && ((uintptr_t)a.q % 16 == 0);
    dim3 grid((unsigned)((a.n + BN - 1) / BN), (unsigned)((a.t + BM - 1) / BM));
    const bool group = a.scale == LOWBIT_SCALE_GROUP;
    switch (a.fmt) {
        case FMT_TERNARY:
            if (group) gemm_kernel<FMT_TERNARY, true><<<grid, dim3(256), 0, stream>>>(ga);
            else gemm_kernel<FMT_TERNARY, false><<<grid, dim3(256), 0, stream>>>(ga);
            break;
        case FMT_INT4:
            if (group) gemm_kernel<FMT_INT4, true><<<grid, dim3(256), 0, stream>>>(ga);
            else gemm_kernel<FMT_INT4, false><<<grid, dim3(256), 0, stream>>>(ga);
            break;
        default:
            if (group) gemm_kernel<FMT_BINARY, true><<<grid, dim3(256), 0, stream>>>(ga);
            else gemm_kernel<FMT_BINARY, false><<<grid, dim3(256), 0, stream>>>(ga);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_gemm(const LinearArgs& a, hipStream_t stream) {
    return gemm_mfma_supported(a) ? launch_gemm_mfma(a, stream) : launch_gemm_generic(a, stream);
}

hipError_t launch_gemm_group(const LinearArgs* mats, int count, hipStream_t stream) {
    bool all = true;
    for (int i = 0; i < count; ++i) all = all && gemm_mfma_supported(mats[i]);
    if (all) return launch_gemm_mfma_group(mats, count, stream);
    for (int i = 0; i < count; ++i) {                        // the general path: one launch each
        hipError_t e = launch_gemm(mats[i], stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace lowbit
