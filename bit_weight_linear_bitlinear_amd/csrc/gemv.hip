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

// MFMAs of one k-step (decoded weights x activation chunks).  FRESH: the
// step starts a new accumulation (its first MFMA adds to zero, not to C).
template <int FMT, int WPL, bool FRESH = false>
__device__ __forceinline__ void step_mfma(const uint32_t* wv, const i32x4* a, i32x4& C) {
    const i32x4 zero = {0, 0, 0, 0};
    if constexpr (FMT == FMT_TERNARY) {
        #pragma unroll
        for (int i = 0; i < WPL; ++i) C = mfma16(a[i], decode_ternary(wv[i]), (FRESH && i == 0) ? zero : C);
    } else if constexpr (FMT == FMT_INT4) {
        #pragma unroll
        for (int i = 0; i < WPL / 2; ++i)
            C = mfma16(a[i], decode_int4(wv[2 * i], wv[2 * i + 1]), (FRESH && i == 0) ? zero : C);
    } else {
        #pragma unroll
        for (int i = 0; i < WPL; ++i) {
            const uint32_t X[8] = {(uint32_t)a[2 * i][0], (uint32_t)a[2 * i][1], (uint32_t)a[2 * i][2],
                                   (uint32_t)a[2 * i][3], (uint32_t)a[2 * i + 1][0], (uint32_t)a[2 * i + 1][1],
                                   (uint32_t)a[2 * i + 1][2], (uint32_t)a[2 * i + 1][3]};
            i32x4 a0, a1, b0, b1;
            perm_binary_a(X, a0, a1);
            decode_binary(wv[i], b0, b1);
            C = mfma16(a0, b0, (FRESH && i == 0) ? zero : C);
            C = mfma16(a1, b1, C);
        }
    }
}

// Where one wavefront reads one 16-row tile: uniform base pointers of its
// part of the k-range, set up once per tile.
struct TileCtx {
    const uint8_t* w;     // packed row (row0) at this part's first k-step
    const int8_t* q;      // activation codes at this part's first k
    const float* sc;      // group mode: scales[row0, first group]; else scales (+ row0 if per row)
    const float* sx;
    float* y;             // y + row0
    int32_t* acc;         // acc + row0 * G (nullable)
    int n;                // rows of the matrix (y row stride)
    int rows;             // valid rows of the tile (<= 0: padding tile)
};

// FAST: every row is a whole number of k-steps, k % 16 == 0, scale groups are
// a power-of-two number of k-steps and pointers are 16-byte aligned - so no
// load ever needs a bounds mask; otherwise byte-safe loaders handle ragged
// rows and tails.  D: k-steps of loads in flight per wavefront.
// ACC: also write the exact integer products (the acc output); kept out of
// the streaming instantiations because optional stores inside the k-loop
// would make the compiler's wait counting conservative.
template <int FMT, int WPL, int NR, bool GROUP, bool FAST, int D, bool ACC>
__global__ __launch_bounds__(256) void gemv_kernel(const GemvParams p) {
    constexpr int BPL = 4 * WPL;                             // packed bytes per lane per k-step
    constexpr int SB = 4 * BPL;                              // packed bytes per row per k-step
    constexpr int KS = 4 * WPL * Fmt<FMT>::kCodesPerWord;     // k per k-step
    constexpr int SHIFT = Fmt<FMT>::kShift;
    constexpr int NA = StepShape<FMT, WPL>::kChunks;
    __shared__ int32_t red[4][4][64];                        // [wave][C register][lane], k-split partials

    // the wavefront index is uniform; saying so keeps every value derived
    // from it (tile, matrix, k-range) in scalar registers and scalar loads
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;                                 // lane group: quarter of each k-step
    const int rl = lane & 15;                                // weight row within the tile
    const int part = wave % p.ksplit;
    const int wslot = wave / p.ksplit;
    const bool tok_ok = rl < p.T;

    const int n_iter = (p.n_tile_groups - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
    const int s_begin = part * p.part_len;                   // first row k-step of this part
    const int s_real = max(0, min(p.n_steps, s_begin + p.part_len) - s_begin);
    const int S = p.loop_steps;                              // part_len rounded up to D

    // per-lane offsets, fixed for the whole kernel
    const uint32_t lw_row = (uint32_t)rl * (uint32_t)p.row_bytes + (uint32_t)(g * BPL);
    const uint32_t lw_row0 = (uint32_t)(g * BPL);
    const uint32_t la = (tok_ok ? (uint32_t)rl * (uint32_t)p.K : 0u) + (uint32_t)((KS / 4) * g);
    const uint32_t ls_row = GROUP ? (uint32_t)rl * (uint32_t)p.G : (p.scale_per_row ? (uint32_t)rl : 0u);
    int sxi[NR];
    #pragma unroll
    for (int r = 0; r < NR; ++r) sxi[r] = min(4 * g + r, p.T - 1);

    auto make_ctx = [&](int it, int& mi) -> TileCtx {
        const int tile = ((int)blockIdx.x + it * (int)gridDim.x) * p.tpw + wslot;
        TileCtx c;
        if (it >= n_iter || tile >= p.total_tiles) {     // padding: valid addresses, nothing stored
            const GemvMat& m0 = p.m[0];
            c.w = m0.packed; c.q = m0.q; c.sc = m0.scales; c.sx = m0.sx; c.y = m0.y; c.acc = nullptr;
            c.n = m0.n; c.rows = 0;
            return c;
        }
        while (mi + 1 < p.n_mats && tile >= p.m[mi + 1].tile0) ++mi;
        const GemvMat& m = p.m[mi];
        const int row0 = (tile - m.tile0) * 16;
        c.w = m.packed + (size_t)row0 * (size_t)p.row_bytes + (size_t)s_begin * SB;
        c.q = m.q + (size_t)s_begin * KS;
        if constexpr (GROUP) c.sc = m.scales + (size_t)row0 * p.G + (s_begin >> p.spu_shift);
        else c.sc = m.scales + (p.scale_per_row ? row0 : 0);
        c.sx = m.sx;
        c.y = m.y + row0;
        c.acc = m.acc ? m.acc + (size_t)row0 * p.G : nullptr;
        c.n = m.n;
        c.rows = min(16, m.n - row0);
        return c;
    };

    // ring of D prefetched k-steps
    uint32_t wv[D][WPL];
    i32x4 av[D][NA];
    float sg[D];           // group scale (group mode) or the row's scale (tensor/row mode)
    float sxs[D][NR];      // activation scales of the tokens this lane's C registers hold

    auto load_slot = [&](int u, const TileCtx& c, int j) {
        const bool row_ok = rl < c.rows;
        if constexpr (FAST) {
            // Unconditional loads, values untouched until consumed: the
            // compiler's wait counting then keeps all D steps in flight.
            // Rows past n use the tile's first row (outputs never stored);
            // dead steps past this part re-read its first step (never used).
            const int jj = j < s_real ? j : 0;
            load_words<WPL>(c.w + (row_ok ? lw_row : lw_row0) + (size_t)jj * SB, BPL, true, wv[u]);
            #pragma unroll
            for (int i = 0; i < NA; ++i)
                av[u][i] = *reinterpret_cast<const i32x4*>(c.q + la + (size_t)jj * KS + 16 * i);
            if constexpr (GROUP) sg[u] = c.sc[(row_ok ? ls_row : 0u) + (uint32_t)(jj >> p.spu_shift)];
            else sg[u] = c.sc[row_ok ? ls_row : 0u];
        } else {
            #pragma unroll
            for (int i = 0; i < WPL; ++i) wv[u][i] = 0u;
            #pragma unroll
            for (int i = 0; i < NA; ++i) av[u][i] = i32x4{0, 0, 0, 0};
            sg[u] = 0.0f;
            if (j < s_real && row_ok) {
                const int64_t off = (int64_t)(s_begin + j) * SB + g * BPL;    // within the row
                const int64_t rem = p.row_bytes - off;
                const int valid = rem <= 0 ? 0 : (rem >= BPL ? BPL : (int)rem);
                if (valid > 0) load_words<WPL>(c.w + (size_t)rl * (size_t)p.row_bytes + (size_t)j * SB + g * BPL,
                                               valid, false, wv[u]);
                if constexpr (GROUP) sg[u] = c.sc[ls_row + (uint32_t)(j / p.spu)];
                else sg[u] = c.sc[ls_row];
            }
            if (j < s_real) {
                const int8_t* qrow = c.q - (size_t)s_begin * KS + (size_t)(tok_ok ? rl : 0) * (size_t)p.K;
                const int kbase = (s_begin + j) * KS + (KS / 4) * g;
                #pragma unroll
                for (int i = 0; i < NA; ++i) av[u][i] = load_a16<false>(qrow, kbase + 16 * i, p.K, tok_ok);
            }
        }
        #pragma unroll
        for (int r = 0; r < NR; ++r) sxs[u][r] = c.sx[sxi[r]];
    };

    i32x4 C = {0, 0, 0, 0};
    float yp[NR];
    #pragma unroll
    for (int r = 0; r < NR; ++r) yp[r] = 0.0f;

    auto compute_slot = [&](int u, const TileCtx& c, int j) {
        if (j >= s_real) return;                             // dead step (uniform)
        if (GROUP && FAST && p.spu_shift == 0)               // one k-step per scale group
            step_mfma<FMT, WPL, true>(wv[u], av[u], C);
        else
            step_mfma<FMT, WPL, false>(wv[u], av[u], C);
        if constexpr (GROUP) {
            const int sn = s_begin + j + 1;
            bool group_end;
            if constexpr (FAST) group_end = (sn & ((1 << p.spu_shift) - 1)) == 0 || sn == p.n_steps;
            else group_end = sn % p.spu == 0 || sn == p.n_steps;
            if (group_end) {
                const int gi = FAST ? (s_begin + j) >> p.spu_shift : (s_begin + j) / p.spu;
                const bool row_ok = rl < c.rows;
                #pragma unroll
                for (int r = 0; r < NR; ++r) {
                    const int32_t a = C[r] >> SHIFT;
                    yp[r] = yp[r] + sg[u] * (float)a;
                    if constexpr (ACC) {
                        const int t = 4 * g + r;
                        if (c.acc && t < p.T && row_ok) c.acc[((size_t)t * c.n + rl) * p.G + gi] = a;
                    }
                }
                if (!(FAST && p.spu_shift == 0)) C = i32x4{0, 0, 0, 0};
            }
        }
    };

    float ep_sx[NR], ep_sw = 0.0f;                           // epilogue operands of the tile
    auto tile_end = [&](const TileCtx& c) {
        const bool row_ok = rl < c.rows;
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
            if (part == 0 && row_ok) {
                #pragma unroll
                for (int r = 0; r < NR; ++r) {
                    const int t = 4 * g + r;
                    if (t < p.T) c.y[(size_t)t * c.n + rl] = ep_sx[r] * yp[r];
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
                        c.y[(size_t)t * c.n + rl] = (float)a[r] * (ep_sx[r] * ep_sw);
                        if constexpr (ACC) {
                            if (c.acc) c.acc[(size_t)t * c.n + rl] = a[r];
                        }
                    }
                }
            }
        }
        C = i32x4{0, 0, 0, 0};
        #pragma unroll
        for (int r = 0; r < NR; ++r) yp[r] = 0.0f;
    };

    int mi_cur = 0;
    TileCtx cur = make_ctx(0, mi_cur);
    int mi_nxt = mi_cur;
    TileCtx nxt = make_ctx(1, mi_nxt);
    #pragma unroll
    for (int u = 0; u < D; ++u) load_slot(u, cur, u);         // S >= D: all in the first tile
    for (int it = 0; it < n_iter; ++it) {
        for (int j = 0; j < S; j += D) {
            #pragma unroll
            for (int u = 0; u < D; ++u) {
                compute_slot(u, cur, j + u);
                if (u == D - 1 && j + D == S) {                  // the tile's last step: keep its
                    #pragma unroll                                // epilogue operands before the
                    for (int r = 0; r < NR; ++r) ep_sx[r] = sxs[u][r];   // slot is refilled
                    ep_sw = sg[u];
                }
                const int jn = j + u + D;                        // step this slot is refilled with
                if (jn < S) load_slot(u, cur, jn);
                else load_slot(u, nxt, jn - S);
            }
        }
        tile_end(cur);
        cur = nxt;
        mi_cur = mi_nxt;
        nxt = make_ctx(it + 2, mi_nxt);
    }
}

// ------------------------------------------------------------------ dispatch

namespace {

template <int FMT, int WPL, int NR, bool GROUP>
void launch_t(const GemvParams& gp, int grid, bool fast, int d, bool acc, hipStream_t st) {
    if (fast && !acc) {
        if (d == 4) gemv_kernel<FMT, WPL, NR, GROUP, true, 4, false><<<dim3(grid), dim3(256), 0, st>>>(gp);
        else gemv_kernel<FMT, WPL, NR, GROUP, true, 1, false><<<dim3(grid), dim3(256), 0, st>>>(gp);
    } else if (fast) {
        if (d == 4) gemv_kernel<FMT, WPL, NR, GROUP, true, 4, true><<<dim3(grid), dim3(256), 0, st>>>(gp);
        else gemv_kernel<FMT, WPL, NR, GROUP, true, 1, true><<<dim3(grid), dim3(256), 0, st>>>(gp);
    } else {
        gemv_kernel<FMT, WPL, NR, GROUP, false, 1, true><<<dim3(grid), dim3(256), 0, st>>>(gp);
    }
}

template <int FMT, int WPL>
void launch_nr(const GemvParams& gp, int grid, int nr, bool group, bool fast, int d, bool acc, hipStream_t st) {
    if (group) {
        if (nr == 1) launch_t<FMT, WPL, 1, true>(gp, grid, fast, d, acc, st);
        else launch_t<FMT, WPL, 4, true>(gp, grid, fast, d, acc, st);
    } else {
        if (nr == 1) launch_t<FMT, WPL, 1, false>(gp, grid, fast, d, acc, st);
        else launch_t<FMT, WPL, 4, false>(gp, grid, fast, d, acc, st);
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

int log2_exact(int v) {   // log2 of a power of two, else -1
    if (v <= 0 || (v & (v - 1)) != 0) return -1;
    int l = 0;
    while ((1 << l) < v) ++l;
    return l;
}

}  // namespace

// Launch one gemv over `count` matrices that share fmt, scale mode, group, k
// and the token count t <= 16.  Tile indices run over the matrices in order.
hipError_t launch_gemv_group(const LinearArgs* mats, int count, hipStream_t stream) {
    const LinearArgs& a = mats[0];
    const int cpw = a.fmt == FMT_TERNARY ? 16 : (a.fmt == FMT_INT4 ? 8 : 32);
    const bool group = a.scale == LOWBIT_SCALE_GROUP;
    const int min_bpl = a.fmt == FMT_INT4 ? 8 : 4;           // one int4 MFMA operand is 2 words
    auto step_k = [&](int b) { return b * cpw; };            // k per k-step = 4 lanes x b bytes
    auto group_ok = [&](int b) { return !group || a.group % step_k(b) == 0; };
    // bytes per lane per k-step: the widest of 16/8/4 whose k-step tiles the
    // scale groups and the row exactly (FAST path); failing the row, the
    // widest that tiles the groups (byte-safe path)
    int bpl = 0;
    for (int b = 16; b >= min_bpl; b /= 2)
        if (group_ok(b) && a.row_bytes % (4 * b) == 0) { bpl = b; break; }
    const bool rows_whole = bpl != 0;
    if (!rows_whole)
        for (int b = 16; b >= min_bpl; b /= 2)
            if (group_ok(b)) { bpl = b; break; }
    const int wpl = bpl / 4;
    const int64_t step_bytes = 4 * (int64_t)bpl;
    const int n_steps = (int)((a.row_bytes + step_bytes - 1) / step_bytes);

    GemvParams gp;
    gp.n_mats = count;
    gp.K = a.k;
    gp.T = a.t;
    gp.row_bytes = a.row_bytes;
    gp.n_steps = n_steps;
    gp.spu = group ? a.group / step_k(bpl) : 1;
    gp.spu_shift = std::max(0, log2_exact(gp.spu));
    gp.G = group ? a.n_groups : 1;
    gp.scale_per_row = a.scale == LOWBIT_SCALE_ROW;
    bool fast = rows_whole && a.k % 16 == 0 && log2_exact(gp.spu) >= 0;
    int tiles = 0;
    for (int i = 0; i < count; ++i) {
        const LinearArgs& b = mats[i];
        GemvMat& m = gp.m[i];
        m.packed = b.packed; m.scales = b.scales; m.q = b.q; m.sx = b.sx; m.y = b.y; m.acc = b.acc;
        m.n = b.n;
        m.tile0 = tiles;
        tiles += (b.n + 15) / 16;
        fast = fast && ((uintptr_t)b.packed % 16 == 0) && ((uintptr_t)b.q % 16 == 0);
    }
    gp.total_tiles = tiles;
    bool any_acc = false;
    for (int i = 0; i < count; ++i) any_acc = any_acc || mats[i].acc != nullptr;

    // k-split: enough wavefronts to fill the chip, whole scale groups per part
    const int cus = device_cu_count();
    const int units = (n_steps + gp.spu - 1) / gp.spu;
    int ksplit = 1;
    if (tiles < 4 * cus && units >= 4) ksplit = 2;
    if (tiles < 2 * cus && units >= 8) ksplit = 4;
    gp.ksplit = ksplit;
    gp.tpw = 4 / ksplit;
    gp.part_len = ((units + ksplit - 1) / ksplit) * gp.spu;
    const int d = fast && gp.part_len >= 4 ? 4 : 1;
    gp.loop_steps = (gp.part_len + d - 1) / d * d;
    gp.n_tile_groups = (tiles + gp.tpw - 1) / gp.tpw;
    const int grid = std::min(gp.n_tile_groups, cus * 8);
    const int nr = a.t == 1 ? 1 : 4;

    switch (a.fmt) {
        case FMT_TERNARY:
            if (wpl == 4) launch_nr<FMT_TERNARY, 4>(gp, grid, nr, group, fast, d, any_acc, stream);
            else if (wpl == 2) launch_nr<FMT_TERNARY, 2>(gp, grid, nr, group, fast, d, any_acc, stream);
            else launch_nr<FMT_TERNARY, 1>(gp, grid, nr, group, fast, d, any_acc, stream);
            break;
        case FMT_INT4:
            if (wpl == 4) launch_nr<FMT_INT4, 4>(gp, grid, nr, group, fast, d, any_acc, stream);
            else launch_nr<FMT_INT4, 2>(gp, grid, nr, group, fast, d, any_acc, stream);
            break;
        default:
            if (wpl == 4) launch_nr<FMT_BINARY, 4>(gp, grid, nr, group, fast, d, any_acc, stream);
            else if (wpl == 2) launch_nr<FMT_BINARY, 2>(gp, grid, nr, group, fast, d, any_acc, stream);
            else launch_nr<FMT_BINARY, 1>(gp, grid, nr, group, fast, d, any_acc, stream);
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
