// gemv.hip - decode-shaped low-bit product (t <= 16 tokens per launch row).
//
// What it computes (M8.8 "Native Binary and Ternary Transformers", 0x02D,
// 0x05D, 0x09C):  acc[t, n] = sum_k q[t, k] * code[n, k] exactly in int32,
// then y = fp32 rescale (tensor/row scales) or a sum of per-group rescaled
// partials (group scales).
//
// Why this shape: decode streams each packed weight byte once ("decode often
// has a small token dimension and repeatedly streams large weight matrices",
// 0x09B), so the kernel is HBM-bound and the work per packed byte must stay
// under the chip's ~5 lane-ops per byte of bandwidth.  Per 16 codes it spends
// 7 VALU ops (shift+mask decode) and hands the multiply-accumulate to one
// quarter of an i8 MFMA; the token dimension (<= 16, zero-padded) rides in the
// MFMA's M side, so t = 1 and t = 16 cost the same weight traffic.
//
// Mapping.  A 16-row tile of W is one MFMA column block: lane l holds weight
// row (l % 16); its lane group (l / 16) streams a quarter of each k-step of that
// row with one 4/8/16-byte load.  The A operand (tokens x k) is 16 consecutive
// bytes of q read straight from the L2-resident activation codes (masked for
// tokens >= t and k >= K).  A workgroup is 4 wavefronts; they either split one
// tile's k-steps (long rows, `ksplit` = 4 or 2) or take separate tiles.
// Partial sums from a k-split are combined in LDS in a fixed order.
#include "device_common.hpp"
#include "kernels.hpp"

namespace lowbit {

struct GemvArgs {
    const uint8_t* packed;
    const float* scales;
    const int8_t* q;
    const float* sx;
    float* y;
    int32_t* acc;
    int64_t row_bytes;
    int T, N, K;
    int n_steps;        // k-steps per row
    int group_steps;    // group mode: k-steps per scale group
    int G;              // group mode: scale groups per row
    int ksplit;         // wavefronts sharing one 16-row tile (1, 2 or 4)
    int scale_per_row;  // tensor/row mode: 1 = scales[n], 0 = scales[0]
    int q_aligned;      // K % 16 == 0 and q 16-byte aligned
};

// 16 activation bytes q[tok, k0 .. k0+16), zero outside [0, K)
__device__ __forceinline__ i32x4 load_a16(const int8_t* qrow, int k0, int K, bool tok_ok, bool aligned) {
    i32x4 v = {0, 0, 0, 0};
    if (tok_ok && k0 < K) {
        if (aligned) {
            v = *reinterpret_cast<const i32x4*>(qrow + k0);
        } else {
            const uint8_t* p = reinterpret_cast<const uint8_t*>(qrow + k0);
            int valid = K - k0;
            #pragma unroll
            for (int i = 0; i < 4; ++i) {
                int vi = valid - 4 * i;
                v[i] = vi <= 0 ? 0 : (int32_t)load_u32_partial(p + 4 * i, vi < 4 ? vi : 4);
            }
        }
    }
    return v;
}

// One k-step of one 16-row tile: WPL packed words per lane -> NM MFMAs.
template <int FMT, int WPL>
__device__ __forceinline__ void gemv_step(const uint32_t* wv, int step, int g, const int8_t* qrow, int K,
                                          bool tok_ok, bool q_aligned, i32x4& C) {
    const int word0 = step * 4 * WPL + g * WPL;   // first packed word of this lane in the row
    if constexpr (FMT == FMT_TERNARY) {
        #pragma unroll
        for (int i = 0; i < WPL; ++i) {
            i32x4 a = load_a16(qrow, 16 * (word0 + i), K, tok_ok, q_aligned);
            C = mfma16(a, decode_ternary(wv[i]), C);
        }
    } else if constexpr (FMT == FMT_INT4) {
        #pragma unroll
        for (int i = 0; i < WPL / 2; ++i) {
            i32x4 a = load_a16(qrow, 8 * (word0 + 2 * i), K, tok_ok, q_aligned);
            C = mfma16(a, decode_int4(wv[2 * i], wv[2 * i + 1]), C);
        }
    } else {
        #pragma unroll
        for (int i = 0; i < WPL; ++i) {
            const int k0 = 32 * (word0 + i);
            i32x4 lo = load_a16(qrow, k0, K, tok_ok, q_aligned);
            i32x4 hi = load_a16(qrow, k0 + 16, K, tok_ok, q_aligned);
            uint32_t X[8] = {(uint32_t)lo[0], (uint32_t)lo[1], (uint32_t)lo[2], (uint32_t)lo[3],
                             (uint32_t)hi[0], (uint32_t)hi[1], (uint32_t)hi[2], (uint32_t)hi[3]};
            i32x4 a0, a1, b0, b1;
            perm_binary_a(X, a0, a1);
            decode_binary(wv[i], b0, b1);
            C = mfma16(a0, b0, C);
            C = mfma16(a1, b1, C);
        }
    }
}

template <int FMT, int WPL, int NR, bool GROUP, bool W_ALIGNED>
__global__ __launch_bounds__(256) void gemv_kernel(GemvArgs a) {
    constexpr int BPL = 4 * WPL;          // packed bytes per lane per k-step
    constexpr int SHIFT = Fmt<FMT>::kShift;
    __shared__ int32_t red[4][4][64];     // [wave][C register][lane], k-split partials

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;              // lane group: quarter of the k-step
    const int rl = lane & 15;             // weight row within the tile
    const int tiles_per_wg = 4 / a.ksplit;
    const int tile = blockIdx.x * tiles_per_wg + wave / a.ksplit;
    const int part = wave % a.ksplit;
    const int t0 = blockIdx.y * 16;

    const int row = tile * 16 + rl;
    const bool row_ok = row < a.N;
    const uint8_t* wrow = a.packed + (size_t)(row_ok ? row : 0) * (size_t)a.row_bytes;
    const int tq = t0 + rl;               // token of this lane's A operand row
    const bool tok_ok = tq < a.T;
    const int8_t* qrow = a.q + (size_t)(tok_ok ? tq : 0) * (size_t)a.K;
    const bool q_aligned = a.q_aligned != 0;

    float yp[NR];
    #pragma unroll
    for (int r = 0; r < NR; ++r) yp[r] = 0.0f;
    i32x4 C = {0, 0, 0, 0};

    auto load_step = [&](int s, uint32_t* wv) {
        const int64_t off = (int64_t)s * 4 * BPL + g * BPL;
        const int64_t rem = row_ok ? a.row_bytes - off : 0;
        const int valid = rem <= 0 ? 0 : (rem >= BPL ? BPL : (int)rem);
        load_words<WPL>(wrow + (rem > 0 ? off : 0), valid, W_ALIGNED && valid == BPL, wv);
    };

    // this wavefront's k-steps: whole scale groups in group mode
    int sb, se;
    if constexpr (GROUP) {
        const int gb = part * a.G / a.ksplit, ge = (part + 1) * a.G / a.ksplit;
        sb = gb * a.group_steps;
        se = min(ge * a.group_steps, a.n_steps);
    } else {
        sb = part * a.n_steps / a.ksplit;
        se = (part + 1) * a.n_steps / a.ksplit;
    }

    constexpr int U = 4;                  // k-steps whose loads are issued together
    for (int s = sb; s < se; s += U) {
        uint32_t wv[U][WPL];
        #pragma unroll
        for (int u = 0; u < U; ++u)
            if (s + u < se) load_step(s + u, wv[u]);
        #pragma unroll
        for (int u = 0; u < U; ++u) {
            if (s + u < se) {
                gemv_step<FMT, WPL>(wv[u], s + u, g, qrow, a.K, tok_ok, q_aligned, C);
                if constexpr (GROUP) {
                    const int sn = s + u + 1;
                    if (sn % a.group_steps == 0 || sn == a.n_steps) {   // scale group complete
                        const int gi = (s + u) / a.group_steps;
                        const float sg = row_ok ? a.scales[(size_t)row * a.G + gi] : 0.0f;
                        #pragma unroll
                        for (int r = 0; r < NR; ++r) {
                            const int32_t av = C[r] >> SHIFT;
                            yp[r] = yp[r] + sg * (float)av;
                            if (a.acc) {
                                const int t = t0 + 4 * g + r;
                                if (t < a.T && row_ok) a.acc[((size_t)t * a.N + row) * a.G + gi] = av;
                            }
                        }
                        C = i32x4{0, 0, 0, 0};
                    }
                }
            }
        }
    }

    if constexpr (GROUP) {
        if (a.ksplit > 1) {
            #pragma unroll
            for (int r = 0; r < NR; ++r) red[wave][r][lane] = __float_as_int(yp[r]);
            __syncthreads();
            if (part == 0) {
                for (int p = 1; p < a.ksplit; ++p) {
                    #pragma unroll
                    for (int r = 0; r < NR; ++r) yp[r] = yp[r] + __int_as_float(red[wave + p][r][lane]);
                }
            }
        }
        if (part == 0) {
            #pragma unroll
            for (int r = 0; r < NR; ++r) {
                const int t = t0 + 4 * g + r;
                if (t < a.T && row_ok) a.y[(size_t)t * a.N + row] = a.sx[t] * yp[r];
            }
        }
    } else {
        int32_t av[NR];
        #pragma unroll
        for (int r = 0; r < NR; ++r) av[r] = C[r] >> SHIFT;
        if (a.ksplit > 1) {
            #pragma unroll
            for (int r = 0; r < NR; ++r) red[wave][r][lane] = av[r];
            __syncthreads();
            if (part == 0) {
                for (int p = 1; p < a.ksplit; ++p) {
                    #pragma unroll
                    for (int r = 0; r < NR; ++r) av[r] += red[wave + p][r][lane];
                }
            }
        }
        if (part == 0) {
            const float sw = row_ok ? a.scales[a.scale_per_row ? row : 0] : 0.0f;
            #pragma unroll
            for (int r = 0; r < NR; ++r) {
                const int t = t0 + 4 * g + r;
                if (t < a.T && row_ok) {
                    a.y[(size_t)t * a.N + row] = (float)av[r] * (a.sx[t] * sw);
                    if (a.acc) a.acc[(size_t)t * a.N + row] = av[r];
                }
            }
        }
    }
}

// ------------------------------------------------------------------ dispatch

template <int FMT, int WPL, int NR, bool GROUP>
static void launch_gemv_t(const GemvArgs& ga, dim3 grid, bool w_aligned, hipStream_t st) {
    if (w_aligned)
        gemv_kernel<FMT, WPL, NR, GROUP, true><<<grid, dim3(256), 0, st>>>(ga);
    else
        gemv_kernel<FMT, WPL, NR, GROUP, false><<<grid, dim3(256), 0, st>>>(ga);
}

template <int FMT, int WPL>
static void launch_gemv_nr(const GemvArgs& ga, dim3 grid, int nr, bool group, bool w_aligned, hipStream_t st) {
    if (group) {
        if (nr == 1) launch_gemv_t<FMT, WPL, 1, true>(ga, grid, w_aligned, st);
        else if (nr == 2) launch_gemv_t<FMT, WPL, 2, true>(ga, grid, w_aligned, st);
        else launch_gemv_t<FMT, WPL, 4, true>(ga, grid, w_aligned, st);
    } else {
        if (nr == 1) launch_gemv_t<FMT, WPL, 1, false>(ga, grid, w_aligned, st);
        else if (nr == 2) launch_gemv_t<FMT, WPL, 2, false>(ga, grid, w_aligned, st);
        else launch_gemv_t<FMT, WPL, 4, false>(ga, grid, w_aligned, st);
    }
}

hipError_t launch_gemv(const LinearArgs& a, hipStream_t stream) {
    const int cpw = a.fmt == FMT_TERNARY ? 16 : (a.fmt == FMT_INT4 ? 8 : 32);
    const bool group = a.scale == LOWBIT_SCALE_GROUP;
    // bytes per lane per step: the widest of 16/8/4 that keeps a scale group a
    // whole number of steps and that the row length divides (else the
    // byte-safe loader handles every step)
    const int min_bpl = a.fmt == FMT_INT4 ? 8 : 4;   // one int4 MFMA operand is 2 words
    auto step_k = [&](int b) { return 4 * (b / 4) * cpw; };
    int bpl = 16;
    if (group) {   // describe() guarantees group % 64 (128 binary) == 0, so min_bpl fits
        while (bpl > min_bpl && (a.group % step_k(bpl)) != 0) bpl /= 2;
    } else {
        while (bpl > min_bpl && a.row_bytes % bpl != 0) bpl /= 2;
    }
    const int wpl = bpl / 4;
    const int64_t step_bytes = 4 * (int64_t)bpl;
    const int n_steps = (int)((a.row_bytes + step_bytes - 1) / step_bytes);
    const bool w_aligned = (a.row_bytes % bpl == 0) && ((uintptr_t)a.packed % 16 == 0);

    GemvArgs ga;
    ga.packed = a.packed; ga.scales = a.scales; ga.q = a.q; ga.sx = a.sx; ga.y = a.y; ga.acc = a.acc;
    ga.row_bytes = a.row_bytes; ga.T = a.t; ga.N = a.n; ga.K = a.k;
    ga.n_steps = n_steps;
    ga.group_steps = group ? a.group / step_k(bpl) : 0;
    ga.G = group ? a.n_groups : 1;
    ga.scale_per_row = a.scale == LOWBIT_SCALE_ROW;
    ga.q_aligned = (a.k % 16 == 0) && ((uintptr_t)a.q % 16 == 0);

    const int units = group ? ga.G : n_steps;           // what the waves split
    ga.ksplit = units >= 8 ? 4 : (units >= 2 ? 2 : 1);
    const int tiles = (a.n + 15) / 16;
    const int tiles_per_wg = 4 / ga.ksplit;
    const int nr = a.t == 1 ? 1 : (a.t == 2 ? 2 : 4);
    dim3 grid((unsigned)((tiles + tiles_per_wg - 1) / tiles_per_wg), (unsigned)((a.t + 15) / 16));

    switch (a.fmt) {
        case FMT_TERNARY:
            if (wpl == 4) launch_gemv_nr<FMT_TERNARY, 4>(ga, grid, nr, group, w_aligned, stream);
            else if (wpl == 2) launch_gemv_nr<FMT_TERNARY, 2>(ga, grid, nr, group, w_aligned, stream);
            else launch_gemv_nr<FMT_TERNARY, 1>(ga, grid, nr, group, w_aligned, stream);
            break;
        case FMT_INT4:
            if (wpl == 4) launch_gemv_nr<FMT_INT4, 4>(ga, grid, nr, group, w_aligned, stream);
            else launch_gemv_nr<FMT_INT4, 2>(ga, grid, nr, group, w_aligned, stream);
            break;
        default:
            if (wpl == 4) launch_gemv_nr<FMT_BINARY, 4>(ga, grid, nr, group, w_aligned, stream);
            else if (wpl == 2) launch_gemv_nr<FMT_BINARY, 2>(ga, grid, nr, group, w_aligned, stream);
            else launch_gemv_nr<FMT_BINARY, 1>(ga, grid, nr, group, w_aligned, stream);
            break;
    }
    return hipGetLastError();
}

}  // namespace lowbit
