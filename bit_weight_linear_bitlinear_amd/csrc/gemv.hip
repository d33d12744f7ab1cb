// gemv.hip - decode-shaped low-bit product: t <= 16 tokens per launch, one
// or many weight matrices of equal k per launch.
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
// bytes of q read from the L2-resident activation codes (masked for tokens
// >= t and k >= K).  A workgroup is 4 wavefronts; `ksplit` of them share one
// tile's k-range (combined in LDS in a fixed order), the rest take other
// tiles.  Workgroups are persistent: each walks tile groups
// blockIdx.x, blockIdx.x + gridDim.x, ... and every wavefront runs one flat
// sequence of (tile, k-step) pairs with the loads of the next D steps
// (weights, activation operands, group scales) always in flight, across tile
// and matrix boundaries.
#include <algorithm>

#include "device_common.hpp"
#include "gemv.hpp"
#include "kernels.hpp"

namespace lowbit {

// 16 activation bytes q[tok, k0 .. k0+16), zero outside [0, K).  FAST: K is a
// multiple of 16 and q 16-byte aligned, so a chunk is wholly inside or outside.
template <bool FAST>
__device__ __forceinline__ i32x4 load_a16(const int8_t* qrow, int k0, int K, bool tok_ok) {
    i32x4 v = {0, 0, 0, 0};
    if (tok_ok && k0 < K) {
        if constexpr (FAST) {
            v = *reinterpret_cast<const i32x4*>(qrow + k0);
        } else {
            const uint8_t* p = reinterpret_cast<const uint8_t*>(qrow + k0);
            const int valid = K - k0;
            #pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int vi = valid - 4 * i;
                v[i] = vi <= 0 ? 0 : (int32_t)load_u32_partial(p + 4 * i, vi < 4 ? vi : 4);
            }
        }
    }
    return v;
}

template <int FMT, int WPL> struct StepShape {
    // 16-byte activation chunks one k-step of one lane needs
    static constexpr int kChunks = FMT == FMT_TERNARY ? WPL : (FMT == FMT_INT4 ? WPL / 2 : 2 * WPL);
    // k offset (within the row) of chunk c for a lane whose first word is word0
    static __device__ __forceinline__ int chunk_k(int word0, int c) {
        if constexpr (FMT == FMT_TERNARY) return 16 * (word0 + c);
        else if constexpr (FMT == FMT_INT4) return 8 * (word0 + 2 * c);
        else return 32 * (word0 + c / 2) + 16 * (c % 2);
    }
};

// MFMAs of one k-step (decoded weights x activation chunks)
template <int FMT, int WPL>
__device__ __forceinline__ void step_mfma(const uint32_t* wv, const i32x4* a, i32x4& C) {
    if constexpr (FMT == FMT_TERNARY) {
        #pragma unroll
        for (int i = 0; i < WPL; ++i) C = mfma16(a[i], decode_ternary(wv[i]), C);
    } else if constexpr (FMT == FMT_INT4) {
        #pragma unroll
        for (int i = 0; i < WPL / 2; ++i) C = mfma16(a[i], decode_int4(wv[2 * i], wv[2 * i + 1]), C);
    } else {
        #pragma unroll
        for (int i = 0; i < WPL; ++i) {
            const uint32_t X[8] = {(uint32_t)a[2 * i][0], (uint32_t)a[2 * i][1], (uint32_t)a[2 * i][2],
                                   (uint32_t)a[2 * i][3], (uint32_t)a[2 * i + 1][0], (uint32_t)a[2 * i + 1][1],
                                   (uint32_t)a[2 * i + 1][2], (uint32_t)a[2 * i + 1][3]};
            i32x4 a0, a1, b0, b1;
            perm_binary_a(X, a0, a1);
            decode_binary(wv[i], b0, b1);
            C = mfma16(a0, b0, C);
            C = mfma16(a1, b1, C);
        }
    }
}

// Position of a wavefront in its flat (tile, k-step) sequence.  All fields
// are wavefront-uniform.
struct Cursor {
    int it;      // tile-group iteration of this workgroup
    int j;       // k-step within this wavefront's part of the row
    int tile;    // global tile index (across matrices)
    int mi;      // matrix of that tile
};

// FAST: every row is a whole number of BPL-byte chunks, packed and q are
// 16-byte aligned and K % 16 == 0 - loads are single vector loads masked per
// lane; otherwise byte-safe loaders handle ragged rows and tails.
template <int FMT, int WPL, int NR, bool GROUP, bool FAST>
__global__ __launch_bounds__(256) void gemv_kernel(const GemvParams p) {
    constexpr int BPL = 4 * WPL;                 // packed bytes per lane per k-step
    constexpr int SHIFT = Fmt<FMT>::kShift;
    constexpr int NA = StepShape<FMT, WPL>::kChunks;
    constexpr int D = 4;                         // k-steps of loads in flight per wavefront
    __shared__ int32_t red[4][4][64];            // [wave][C register][lane], k-split partials

    // the wavefront index is uniform; saying so keeps every value derived
    // from it (tile, matrix, k-range) in scalar registers and scalar loads
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;                     // lane group: quarter of the k-step
    const int rl = lane & 15;                    // weight row within the tile
    const int part = wave % p.ksplit;
    const int wslot = wave / p.ksplit;
    const bool tok_ok = rl < p.T;

    const int n_iter = (p.n_tile_groups - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
    const int F = n_iter * p.part_steps;
    const int s_begin = part * p.part_steps;                       // first row k-step of this part
    const int s_end = min(p.n_steps, s_begin + p.part_steps);

    auto set_iter = [&](Cursor& c, int it) {
        c.it = it;
        c.j = 0;
        c.tile = ((int)blockIdx.x + it * (int)gridDim.x) * p.tpw + wslot;
        while (c.mi + 1 < p.n_mats && c.tile >= p.m[c.mi + 1].tile0) ++c.mi;
    };
    auto advance = [&](Cursor& c) {
        if (++c.j == p.part_steps) set_iter(c, c.it + 1);
    };

    // ring of D prefetched k-steps
    uint32_t wv[D][WPL];
    i32x4 av[D][NA];
    float sg[D];           // group scale (group mode) or the row's scale (tensor/row mode)
    float sxs[D][NR];      // activation scales of the tokens this lane's C registers hold

    auto load_slot = [&](int u, const Cursor& c) {
        const int s = s_begin + c.j;
        const bool live = c.it < n_iter && s < s_end && c.tile < p.total_tiles;   // uniform
        const GemvMat& m = p.m[c.mi];
        const int row = (c.tile - m.tile0) * 16 + rl;
        const bool row_ok = live && row < m.n;
        const int64_t off = (int64_t)s * 4 * BPL + g * BPL;
        const int word0 = s * 4 * WPL + g * WPL;
        if constexpr (FAST) {
            // Every load is issued unconditionally and nothing is done with
            // its value here, so the compiler's wait counting never assumes a
            // skipped load and never waits on a load right after issuing it.
            // Lanes with nothing to read use clamped, valid addresses: a row
            // past n or a token past t only pollutes outputs that are never
            // stored, and weights past the row are zeroed when consumed.
            const bool wok = row_ok && off < p.row_bytes;
            load_words<WPL>(m.packed + (wok ? (size_t)row * (size_t)p.row_bytes + off : 0), BPL, true, wv[u]);
            #pragma unroll
            for (int i = 0; i < NA; ++i) {
                const int k0 = StepShape<FMT, WPL>::chunk_k(word0, i);
                const bool aok = live && tok_ok && k0 < p.K;
                av[u][i] = *reinterpret_cast<const i32x4*>(m.q + (aok ? (size_t)rl * (size_t)p.K + k0 : 0));
            }
            // scale of the group this step belongs to / of the row; the
            // tokens' activation scales ride along so the tile's last step has
            // every epilogue operand in the ring
            if constexpr (GROUP)
                sg[u] = m.scales[row_ok ? (size_t)row * p.G + s / p.spu : 0];
            else
                sg[u] = m.scales[p.scale_per_row && row_ok ? row : 0];
            #pragma unroll
            for (int r = 0; r < NR; ++r) sxs[u][r] = m.sx[min(4 * g + r, p.T - 1)];
        } else {
            #pragma unroll
            for (int i = 0; i < WPL; ++i) wv[u][i] = 0u;
            #pragma unroll
            for (int i = 0; i < NA; ++i) av[u][i] = i32x4{0, 0, 0, 0};
            sg[u] = 0.0f;
            if (!live) return;
            const int64_t rem = row_ok ? p.row_bytes - off : 0;
            const int valid = rem <= 0 ? 0 : (rem >= BPL ? BPL : (int)rem);
            if (valid > 0)
                load_words<WPL>(m.packed + (size_t)(row_ok ? row : 0) * (size_t)p.row_bytes + off, valid, false, wv[u]);
            const int8_t* qrow = m.q + (size_t)(tok_ok ? rl : 0) * (size_t)p.K;
            #pragma unroll
            for (int i = 0; i < NA; ++i)
                av[u][i] = load_a16<false>(qrow, StepShape<FMT, WPL>::chunk_k(word0, i), p.K, tok_ok);
            if constexpr (GROUP) {
                const int sn = s + 1;
                if ((sn % p.spu == 0 || sn == p.n_steps) && row_ok)
                    sg[u] = m.scales[(size_t)row * p.G + s / p.spu];
            } else {
                sg[u] = m.scales[p.scale_per_row && row_ok ? row : 0];
            }
            #pragma unroll
            for (int r = 0; r < NR; ++r) sxs[u][r] = m.sx[min(4 * g + r, p.T - 1)];
        }
    };

    i32x4 C = {0, 0, 0, 0};
    float yp[NR];
    #pragma unroll
    for (int r = 0; r < NR; ++r) yp[r] = 0.0f;

    auto compute_slot = [&](int u, const Cursor& c) {
        const int s = s_begin + c.j;
        const bool live = s < s_end;             // c.it < n_iter holds here
        const GemvMat& m = p.m[c.mi];
        const int row = (c.tile - m.tile0) * 16 + rl;
        const bool row_ok = c.tile < p.total_tiles && row < m.n;
        if (live) {
            if constexpr (FAST) {
                // weights past the end of the row pair with clamped (garbage)
                // activations: zero them (binary: after decoding, a zero word
                // means +1 codes)
                const bool wok = (int64_t)s * 4 * BPL + g * BPL < p.row_bytes;
                if constexpr (FMT != FMT_BINARY) {
                    #pragma unroll
                    for (int i = 0; i < WPL; ++i) wv[u][i] = wok ? wv[u][i] : 0u;
                } else {
                    #pragma unroll
                    for (int i = 0; i < NA; ++i) av[u][i] = wok ? av[u][i] : i32x4{0, 0, 0, 0};
                }
            }
            step_mfma<FMT, WPL>(wv[u], av[u], C);
            if constexpr (GROUP) {
                const int sn = s + 1;
                if (sn % p.spu == 0 || sn == p.n_steps) {        // a scale group is complete
                    const int gi = s / p.spu;
                    #pragma unroll
                    for (int r = 0; r < NR; ++r) {
                        const int32_t a = C[r] >> SHIFT;
                        yp[r] = yp[r] + sg[u] * (float)a;
                        if (m.acc) {
                            const int t = 4 * g + r;
                            if (t < p.T && row_ok) m.acc[((size_t)t * m.n + row) * p.G + gi] = a;
                        }
                    }
                    C = i32x4{0, 0, 0, 0};
                }
            }
        }
        if (c.j == p.part_steps - 1) {           // end of this tile's k-range
            if constexpr (GROUP) {
                if (p.ksplit > 1) {
                    #pragma unroll
                    for (int r = 0; r < NR; ++r) red[wave][r][lane] = __float_as_int(yp[r]);
                    __syncthreads();
                    if (part == 0) {
                        for (int q = 1; q < p.ksplit; ++q) {
                            #pragma unroll
                            for (int r = 0; r < NR; ++r) yp[r] = yp[r] + __int_as_float(red[wave + q][r][lane]);
                        }
                    }
                    __syncthreads();
                }
                if (part == 0) {
                    #pragma unroll
                    for (int r = 0; r < NR; ++r) {
                        const int t = 4 * g + r;
                        if (t < p.T && row_ok) m.y[(size_t)t * m.n + row] = sxs[u][r] * yp[r];
                    }
                }
            } else {
                int32_t a[NR];
                #pragma unroll
                for (int r = 0; r < NR; ++r) a[r] = C[r] >> SHIFT;
                if (p.ksplit > 1) {
                    #pragma unroll
                    for (int r = 0; r < NR; ++r) red[wave][r][lane] = a[r];
                    __syncthreads();
                    if (part == 0) {
                        for (int q = 1; q < p.ksplit; ++q) {
                            #pragma unroll
                            for (int r = 0; r < NR; ++r) a[r] += red[wave + q][r][lane];
                        }
                    }
                    __syncthreads();
                }
                if (part == 0 && row_ok) {
                    #pragma unroll
                    for (int r = 0; r < NR; ++r) {
                        const int t = 4 * g + r;
                        if (t < p.T) {
                            m.y[(size_t)t * m.n + row] = (float)a[r] * (sxs[u][r] * sg[u]);
                            if (m.acc) m.acc[(size_t)t * m.n + row] = a[r];
                        }
                    }
                }
            }
            C = i32x4{0, 0, 0, 0};
            #pragma unroll
            for (int r = 0; r < NR; ++r) yp[r] = 0.0f;
        }
    };

    Cursor pc, cc;
    pc.mi = 0;
    cc.mi = 0;
    set_iter(pc, 0);
    set_iter(cc, 0);
    #pragma unroll
    for (int u = 0; u < D; ++u) {
        load_slot(u, pc);
        advance(pc);
    }
    for (int f = 0; f < F; f += D) {
        #pragma unroll
        for (int u = 0; u < D; ++u) {
            if (f + u < F) {
                compute_slot(u, cc);
                advance(cc);
                load_slot(u, pc);
                advance(pc);
            }
        }
    }
}

// ------------------------------------------------------------------ dispatch

namespace {

template <int FMT, int WPL, int NR, bool GROUP>
void launch_t(const GemvParams& gp, int grid, bool fast, hipStream_t st) {
    if (fast)
        gemv_kernel<FMT, WPL, NR, GROUP, true><<<dim3(grid), dim3(256), 0, st>>>(gp);
    else
        gemv_kernel<FMT, WPL, NR, GROUP, false><<<dim3(grid), dim3(256), 0, st>>>(gp);
}

template <int FMT, int WPL>
void launch_nr(const GemvParams& gp, int grid, int nr, bool group, bool fast, hipStream_t st) {
    if (group) {
        if (nr == 1) launch_t<FMT, WPL, 1, true>(gp, grid, fast, st);
        else if (nr == 2) launch_t<FMT, WPL, 2, true>(gp, grid, fast, st);
        else launch_t<FMT, WPL, 4, true>(gp, grid, fast, st);
    } else {
        if (nr == 1) launch_t<FMT, WPL, 1, false>(gp, grid, fast, st);
        else if (nr == 2) launch_t<FMT, WPL, 2, false>(gp, grid, fast, st);
        else launch_t<FMT, WPL, 4, false>(gp, grid, fast, st);
    }
}

int device_cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        cached[dev] = cus;
    }
    return cached[dev];
}

}  // namespace

// Launch one gemv over `count` matrices that share fmt, scale mode, group, k
// and the token count t <= 16.  Tile indices run over the matrices in order.
hipError_t launch_gemv_group(const LinearArgs* mats, int count, hipStream_t stream) {
    const LinearArgs& a = mats[0];
    const int cpw = a.fmt == FMT_TERNARY ? 16 : (a.fmt == FMT_INT4 ? 8 : 32);
    const bool group = a.scale == LOWBIT_SCALE_GROUP;
    const int min_bpl = a.fmt == FMT_INT4 ? 8 : 4;   // one int4 MFMA operand is 2 words
    auto step_k = [&](int b) { return 4 * (b / 4) * cpw; };
    // bytes per lane per k-step: the widest of 16/8/4 that keeps a scale
    // group a whole number of steps and that the row length divides (else
    // the byte-safe loader handles every step)
    int bpl = 16;
    if (group) {   // describe() guarantees group % 64 (128 binary) == 0, so min_bpl fits
        while (bpl > min_bpl && (a.group % step_k(bpl)) != 0) bpl /= 2;
    } else {
        while (bpl > min_bpl && a.row_bytes % bpl != 0) bpl /= 2;
    }
    const int wpl = bpl / 4;
    const int64_t step_bytes = 4 * (int64_t)bpl;
    const int n_steps = (int)((a.row_bytes + step_bytes - 1) / step_bytes);
    bool w_aligned = a.row_bytes % bpl == 0;

    GemvParams gp;
    gp.n_mats = count;
    gp.K = a.k;
    gp.T = a.t;
    gp.row_bytes = a.row_bytes;
    gp.n_steps = n_steps;
    gp.spu = group ? a.group / step_k(bpl) : 1;
    gp.G = group ? a.n_groups : 1;
    gp.scale_per_row = a.scale == LOWBIT_SCALE_ROW;
    gp.q_aligned = a.k % 16 == 0;
    int tiles = 0;
    for (int i = 0; i < count; ++i) {
        const LinearArgs& b = mats[i];
        GemvMat& m = gp.m[i];
        m.packed = b.packed; m.scales = b.scales; m.q = b.q; m.sx = b.sx; m.y = b.y; m.acc = b.acc;
        m.n = b.n;
        m.tile0 = tiles;
        tiles += (b.n + 15) / 16;
        w_aligned = w_aligned && ((uintptr_t)b.packed % 16 == 0);
        gp.q_aligned = gp.q_aligned && ((uintptr_t)b.q % 16 == 0);
    }
    gp.total_tiles = tiles;
    const bool fast = w_aligned && gp.q_aligned;

    // k-split: enough wavefronts to fill the chip, whole scale groups per part
    const int cus = device_cu_count();
    const int units = (n_steps + gp.spu - 1) / gp.spu;
    int ksplit = 1;
    if (tiles < 4 * cus && units >= 4) ksplit = 2;
    if (tiles < 2 * cus && units >= 8) ksplit = 4;
    gp.ksplit = ksplit;
    gp.tpw = 4 / ksplit;
    const int upp = (units + ksplit - 1) / ksplit;
    gp.part_steps = upp * gp.spu;
    gp.n_tile_groups = (tiles + gp.tpw - 1) / gp.tpw;
    const int grid = std::min(gp.n_tile_groups, cus * 8);
    const int nr = a.t == 1 ? 1 : (a.t == 2 ? 2 : 4);

    switch (a.fmt) {
        case FMT_TERNARY:
            if (wpl == 4) launch_nr<FMT_TERNARY, 4>(gp, grid, nr, group, fast, stream);
            else if (wpl == 2) launch_nr<FMT_TERNARY, 2>(gp, grid, nr, group, fast, stream);
            else launch_nr<FMT_TERNARY, 1>(gp, grid, nr, group, fast, stream);
            break;
        case FMT_INT4:
            if (wpl == 4) launch_nr<FMT_INT4, 4>(gp, grid, nr, group, fast, stream);
            else launch_nr<FMT_INT4, 2>(gp, grid, nr, group, fast, stream);
            break;
        default:
            if (wpl == 4) launch_nr<FMT_BINARY, 4>(gp, grid, nr, group, fast, stream);
            else if (wpl == 2) launch_nr<FMT_BINARY, 2>(gp, grid, nr, group, fast, stream);
            else launch_nr<FMT_BINARY, 1>(gp, grid, nr, group, fast, stream);
            break;
    }
    return hipGetLastError();
}

// One matrix, any t: 16 tokens per launch.
hipError_t launch_gemv(const LinearArgs& a, hipStream_t stream) {
    for (int t0 = 0; t0 < a.t; t0 += 16) {
        LinearArgs c = a;
        c.t = std::min(16, a.t - t0);
        c.q = a.q + (size_t)t0 * a.k;
        c.sx = a.sx + t0;
        c.y = a.y + (size_t)t0 * a.n;
        c.acc = a.acc ? a.acc + (size_t)t0 * a.n * a.n_groups : nullptr;
        hipError_t e = launch_gemv_group(&c, 1, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace lowbit
