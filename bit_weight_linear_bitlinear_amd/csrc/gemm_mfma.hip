// gemm_mfma.hip - prefill-shaped low-bit product on the gfx950 matrix cores,
// the streaming path (k a multiple of 16, activation codes 16-byte aligned).
//
// What it computes (M8.8 "Native Binary and Ternary Transformers", 0x02D,
// 0x09C): acc[t, n] = sum_k q[t, k] * code[n, k] exactly in int32 (per scale
// group in group mode), then the fp32 rescale.  Prefill is a dense contraction
// (0x09B), so the work is v_mfma_i32_32x32x32_i8 with the packed codes decoded
// in registers right before each MFMA.
//
// Tiling.  A 512-thread workgroup owns a 256-token x 256-row output tile; its
// eight wavefronts (two per SIMD) are a 4 x 2 grid of 64 x 128 sub-tiles, i.e.
// 2 x 4 blocks of 32 x 32 (each staged activation byte is read by two
// wavefronts, each packed weight byte by four).  (TILE 0: 128 x 128 with four wavefronts of 64 x 64,
// two workgroups per CU; TILE 2: 128 x 192 with four of 64 x 96.)  k advances one packed-layout k-step (SK codes) at a
// time.  Each step's operands are copied global -> LDS by the memory unit itself
// (16-byte direct-to-LDS loads: no registers, no LDS write instructions), NS
// steps in flight:
//  - activations: row-major [tile token][SK bytes], every copy reading whole
//    128-byte lines (a copy of 1 KB covers 1024 / SK rows), the 16-byte chunks
//    of a row XOR-swizzled with the row number so that the operand reads - 32
//    rows at one k offset - hit 16 different bank groups;
//  - weights: the packed (16-row tile, k-step) blocks as they are.
// MFMA operand lanes: lane l holds token / row l % 32 and 16 k values of half
// h = l / 32.  Half h takes the packed lane groups 2h and 2h + 1 of a 16-row
// tile, i.e. k offsets 32h .. 32h + 31 of each 64-code chunk (binary: 64h ..
// 64h + 63 of each 128-code chunk, bit order matched by perm_binary_a).
// The compiler does not track the LDS side of the copies, so the pipeline waits
// with explicit vmcnt counts (every copy of a step is unconditional) followed
// by a workgroup barrier.  Tokens past t and rows past n read clamped (valid)
// addresses; their results are never stored.  Binary activations past k are
// zeroed in registers (binary padding codes decode as +1; ternary and int4
// padding codes are 0).
//
// Workgroups are numbered so that each XCD (workgroup i runs on XCD i % 8)
// owns a contiguous run of output tiles, token-block-major: the weight matrix
// and a few activation blocks stay in that XCD's L2.
#include <algorithm>
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace lowbit {

typedef int32_t i32x16 __attribute__((ext_vector_type(16)));

// One launch: up to kGemmMaxMats products of equal k, token count, format and
// scale mode; workgroups run over the matrices' output tiles in order.
constexpr int kGemmMaxMats = 64;

struct GemmMat {
    const uint8_t* packed;
    const float* scales;
    const int8_t* q;
    const float* sx;
    float* y;
    int32_t* acc;
    int N;
    int n_tiles;        // ceil(N / 16)
    int nb;             // row blocks of the launch's tile
};

struct GemmFastArgs {
    int T, K;
    int n_steps;        // packed-layout k-steps
    int group;          // group mode: columns per group
    int G;              // group mode: groups per row
    int scale_per_row;
    int mb;             // token blocks
    int n_mats;
    int wg_start[kGemmMaxMats + 1];   // first workgroup of each matrix; [n_mats] = all; INT_MAX past it
    GemmMat m[kGemmMaxMats];
};

// Workgroup tile configurations (blocks of 32 x 32 per wavefront).
template <int TILE> struct TileCfg;
template <> struct TileCfg<0> {
    static constexpr int WAVES_M = 2, WAVES_N = 2, WMB = 2, WNB = 2, BUDGET = 73728;
};
template <> struct TileCfg<1> {
    static constexpr int WAVES_M = 4, WAVES_N = 2, WMB = 2, WNB = 4, BUDGET = 163840;
};
// TILE 2: 128 x 192 with four wavefronts of 64 x 96, one workgroup per CU (a
// whole number of rounds for row counts such as 1280 where 256-wide tiles
// leave CUs idle)
template <> struct TileCfg<2> {
    static constexpr int WAVES_M = 2, WAVES_N = 2, WMB = 2, WNB = 3, BUDGET = 163840;
};

template <int FMT, int WPL, int TILE> struct GemmShape {
    using TC = TileCfg<TILE>;
    static constexpr int WAVES_M = TC::WAVES_M, WAVES_N = TC::WAVES_N, WMB = TC::WMB, WNB = TC::WNB;
    static constexpr int NW = WAVES_M * WAVES_N;             // wavefronts per workgroup
    static constexpr int CPW = Fmt<FMT>::kCodesPerWord;
    static constexpr int SK = 4 * WPL * CPW;                // k per packed-layout step
    static constexpr int CK = FMT == FMT_BINARY ? 128 : 64;  // k per chunk (one packed word per lane group)
    static constexpr int KC = SK / CK;                       // chunks per step
    static constexpr int BM = 32 * WMB * WAVES_M, BN = 32 * WNB * WAVES_N;
    static constexpr int NTILE = BN / 16;                    // 16-row tiles
    static constexpr int A_BYTES = BM * SK;
    static constexpr int B_BYTES = NTILE * 256 * WPL;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int NS = 3 * STAGE <= TC::BUDGET ? 3 : 2;   // steps in flight
    static constexpr int A_PIECES = A_BYTES / 1024;          // 1 KB direct loads per step
    static constexpr int B_PIECES = B_BYTES / 1024;
    static constexpr bool FITS = NS * STAGE <= 163840;
    // room beside the stages for the tile's s_x and weight scales
    static constexpr bool XS_FITS = NS * STAGE + 4 * (BM + BN) <= 163840;
    static constexpr int CPR = SK / 16;                      // 16-byte chunks per activation row
    static constexpr int RPP = 64 / CPR;                     // activation rows per 1 KB piece
    // swizzle: chunk c of row r sits at chunk c ^ swz(r); 16 consecutive rows
    // read at one chunk then fall on 16 distinct 16-byte bank groups
    static constexpr int SW_DIV = CPR >= 16 ? 1 : 16 / CPR, SW_MOD = CPR >= 16 ? 16 : CPR;
    static_assert(A_PIECES % NW == 0, "activation copies per wavefront");
};

template <int N>
__device__ __forceinline__ void wait_vm() {
    // the direct loads write LDS behind the compiler's back: wait explicitly,
    // and keep every LDS access on its side of the wait
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// one 1 KB direct-to-LDS copy: lane l's 16 bytes land at lds + 16 * l
__device__ __forceinline__ void dma16(const void* src, void* lds) {
    __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
}

// one 256-byte direct-to-LDS copy: lane l's 4 bytes land at lds + 4 * l
__device__ __forceinline__ void dma4(const void* src, void* lds) {
    __builtin_amdgcn_global_load_lds(src, lds, 4, 0, 0);
}

// cache-policy operand of a buffer store: the non-temporal bit
constexpr int kStoreNT = 2;

__device__ __forceinline__ i32x16 mfma32(const i32x4& a, const i32x4& b, const i32x16& c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// The 128 x 128 tile is asked for two wavefronts per SIMD (two workgroups
// per CU): with group scales the compiler otherwise took 194 VGPRs and 128
// accumulation registers for the partials and one workgroup per CU; at 256
// registers per lane the group-128 products of the 4B-class layer at 4096
// tokens ran 1.7x faster (573 -> 989 TOPS).  (Binary operands at four words
// per lane still take one.)
template <int FMT, int WPL, int TILE, bool GROUP, bool ACC>
__global__ __launch_bounds__(TILE == 1 ? 512 : 256) __attribute__((amdgpu_waves_per_eu(TILE == 0 ? 2 : 1)))
void gemm_mfma_kernel(const GemmFastArgs a) {
    using S = GemmShape<FMT, WPL, TILE>;
    constexpr int SK = S::SK, CK = S::CK, KC = S::KC, NS = S::NS, STAGE = S::STAGE, A_BYTES = S::A_BYTES;
    constexpr int BM = S::BM, BN = S::BN, NW = S::NW, CPR = S::CPR, RPP = S::RPP;
    constexpr int WMB = S::WMB, WNB = S::WNB;
    constexpr int SHIFT = Fmt<FMT>::kShift;
    // direct loads per wave per step: the fewest any wave issues (waits are
    // then exact or conservative for every wave)
    constexpr int LA = S::A_PIECES / NW;
    constexpr int LB = (S::B_PIECES + NW - 1) / NW;          // past the last piece: a copy of it again
    constexpr int L = LA + LB;
    // the stages, then (row and tensor scales, where they fit) the tile's s_x
    // and weight scales, copied in the prologue so that the epilogue reads
    // them from LDS rather than wait for a global round trip
    constexpr bool XSL = !GROUP && S::XS_FITS;
    constexpr int XS_BYTES = XSL ? 4 * (BM + BN) : 0;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * STAGE + XS_BYTES];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, h = lane >> 5, j = lane & 31;
    const int wm = wave / S::WAVES_N, wn = wave % S::WAVES_N;

    // XCD-aware tile order: XCD x runs a contiguous run of the launch's tiles
    // (matrix after matrix); then this tile's matrix
    const int total = a.wg_start[a.n_mats];
    const int xcd = (int)blockIdx.x % 8, jx = (int)blockIdx.x / 8;
    const int glogical = xcd * (total / 8) + min(xcd, total % 8) + jx;
    int mi = 0, hi = a.n_mats - 1;                          // binary search of the ascending starts
    while (mi < hi) {
        const int mid = (mi + hi + 1) >> 1;
        if (glogical >= a.wg_start[mid]) mi = mid;
        else hi = mid - 1;
    }
    const GemmMat& mat = a.m[mi];
    const uint8_t* const m_packed = mat.packed;
    const float* const m_scales = mat.scales;
    const int8_t* const m_q = mat.q;
    const float* const m_sx = mat.sx;
    float* const m_y = mat.y;
    int32_t* const m_acc = mat.acc;
    const int m_N = mat.N, m_ntiles = mat.n_tiles, m_nb = mat.nb;
    const int logical = glogical - a.wg_start[mi];
    const int tb_m = logical / m_nb, tb_n = logical % m_nb;
    const int m0 = tb_m * BM, n0 = tb_n * BN;
    const int K = a.K, T = a.T;
    auto swz = [](int r) { return (r / S::SW_DIV) % S::SW_MOD; };

    // ---- per-lane sources of this workgroup's direct loads
    // activation piece p: rows p * RPP .. of the tile, lane i reading chunk
    // (i % CPR) ^ swz(row) of row p * RPP + i / CPR, which lands at LDS byte
    // p * 1024 + 16 i = row * SK + 16 * ((i % CPR)): the swizzled position
    const int8_t* const qt = m_q + (size_t)m0 * K;
    int aoff[LA], akc[LA];                                   // row offset in the tile, chunk byte offset
    #pragma unroll
    for (int ii = 0; ii < LA; ++ii) {
        const int p = wave + NW * ii;
        const int r = p * RPP + lane / CPR;
        aoff[ii] = (min(m0 + r, T - 1) - m0) * K;
        akc[ii] = 16 * ((lane % CPR) ^ swz(r));
    }
    // weight piece p: 16-byte chunk c = 64 p + lane of the stage's row tiles;
    // every wave issues LB pieces, those past the last one repeat it (same
    // bytes to the same place), so all waves wait for the same counts
    const uint8_t* b_src[LB];
    int b_dst[LB];
    #pragma unroll
    for (int i = 0; i < LB; ++i) {
        const int p = min(wave + NW * i, S::B_PIECES - 1);
        b_dst[i] = A_BYTES + p * 1024;
        const int c = 64 * p + lane;
        const int tt = c / (16 * WPL), cc = c % (16 * WPL);
        const int tile = min(tb_n * S::NTILE + tt, m_ntiles - 1);
        b_src[i] = m_packed + (size_t)tile * a.n_steps * (256 * WPL) + cc * 16;
    }

    // The direct loads of one step, numbered 0 .. NDMA-1 for this wave:
    // activation pieces first, then weight pieces.
    constexpr int NDMA = LA + LB;
    auto issue_one = [&](int s, int d) {
        uint8_t* st = smem + (s % NS) * STAGE;
        if (d < LA) {
            const int k = s * SK + akc[d];
            dma16(qt + aoff[d] + (k < K ? k : 0), st + (wave + NW * d) * 1024);
        } else {
            const int i = d - LA;
            dma16(b_src[i] + (size_t)s * (256 * WPL), st + b_dst[i]);
        }
    };
    auto issue = [&](int s) {                                // all direct loads of step s
        #pragma unroll
        for (int d = 0; d < NDMA; ++d) issue_one(s, d);
    };

    // this lane's activation rows (one per 32-token block) and their swizzle
    const int sw = swz(j);                                   // rows are 32 apart between blocks: same swizzle
    const int arow0 = (wm * (32 * WMB) + j) * SK;

    i32x16 C[WMB][WNB];
    #pragma unroll
    for (int i = 0; i < WMB; ++i)
        #pragma unroll
        for (int jb = 0; jb < WNB; ++jb) C[i][jb] = i32x16{};
    float yp[GROUP ? WMB : 1][GROUP ? WNB : 1][16];
    if constexpr (GROUP) {
        #pragma unroll
        for (int i = 0; i < WMB; ++i)
            #pragma unroll
            for (int jb = 0; jb < WNB; ++jb)
                #pragma unroll
                for (int r = 0; r < 16; ++r) yp[i][jb][r] = 0.0f;
    }

    // group mode: the chunks ending at kend close a group
    auto close_groups = [&](int kend) {
        const int gi = (min(kend, K) - 1) / a.group;
        #pragma unroll
        for (int jb = 0; jb < WNB; ++jb) {
            const int n = n0 + wn * (32 * WNB) + jb * 32 + j;
            const int nc = min(n, m_N - 1);
            const float sg = m_scales[((size_t)(nc >> 4) * a.G + gi) * 16 + (nc & 15)];
            #pragma unroll
            for (int i = 0; i < WMB; ++i) {
                #pragma unroll
                for (int r = 0; r < 16; ++r) {
                    // C holds 2^SHIFT times the group's partial: converted
                    // directly it is exactly 2^SHIFT times fp32(partial), and
                    // scaling by a power of two commutes with fp32 rounding,
                    // so yp is kept 2^SHIFT times larger bit for bit (one
                    // shift fewer per register and group; the epilogue scales
                    // back)
                    yp[i][jb][r] = yp[i][jb][r] + sg * (float)C[i][jb][r];
                    if constexpr (ACC) {
                        const int t = m0 + wm * (32 * WMB) + i * 32 + 8 * (r / 4) + 4 * h + (r % 4);
                        if (m_acc && t < T && n < m_N) m_acc[((size_t)t * m_N + n) * a.G + gi] = C[i][jb][r] >> SHIFT;
                    }
                }
                C[i][jb] = i32x16{};
            }
        }
    };

    // s_x of the tile's tokens and the scales of its rows (clamped indices;
    // unused past t and n), as 256-byte pieces spread over the wavefronts.
    // They precede step 0's copies, so step 0's wait and barrier cover them.
    float* const xs_x = reinterpret_cast<float*>(smem + NS * STAGE);
    float* const xs_w = xs_x + BM;
    if constexpr (XSL) {
        constexpr int PX = BM / 64, PW = BN / 64;
        static_assert(BM % 64 == 0 && BN % 64 == 0, "scale pieces");
        for (int p = wave; p < PX + PW; p += NW) {           // uniform
            if (p < PX) {
                dma4(m_sx + min(m0 + 64 * p + lane, T - 1), xs_x + 64 * p);
            } else {
                const int n = min(n0 + 64 * (p - PX) + lane, m_N - 1);
                dma4(m_scales + (a.scale_per_row ? n : 0), xs_w + 64 * (p - PX));
            }
        }
    }

    const int n_steps = a.n_steps;
    #pragma unroll
    for (int s = 0; s < NS - 1; ++s)
        if (s < n_steps) issue(s);

    // One k-step.  FETCH: the loads of step s+NS-1 are issued during it (the
    // main part of the loop); the last NS-1 steps fetch nothing.
    auto k_step = [&](int s, auto fetch_tag) {
        constexpr bool FETCH = decltype(fetch_tag)::value;
        // step s has landed once at most the later steps' loads are in flight
        if constexpr (FETCH) {
            wait_vm<(NS - 2) * L>();
        } else {
            const int later = min(NS - 2, n_steps - 1 - s);  // uniform
            if (later >= 2) wait_vm<2 * L>();
            else if (later == 1) wait_vm<L>();
            else wait_vm<0>();
        }
        // Everyone's copies of step s have landed and step s-1 is consumed.
        // A bare s_barrier: __syncthreads() would also drain every later
        // step's loads (its fence waits for all memory operations).
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");                       // (the direct loads below stay after the barrier)
        // Step s+NS-1 goes into the buffer step s-1 used.  Its loads are
        // spread over this step's MFMA groups: issued all at once, every wave
        // would stall behind the others' requests.
        const int sf = s + NS - 1;

        const uint8_t* st = smem + (s % NS) * STAGE;
        const uint8_t* bs = st + A_BYTES;
        // this lane's packed words of the step: groups 2h, 2h + 1 of row
        // j % 16 in tile 2 jb + j / 16 of the wave's rows
        uint32_t bw[WNB][2][WPL];
        #pragma unroll
        for (int jb = 0; jb < WNB; ++jb) {
            #pragma unroll
            for (int gg = 0; gg < 2; ++gg) {
                const uint8_t* p = bs + (wn * (2 * WNB) + 2 * jb + (j >> 4)) * (256 * WPL) +
                                   (((2 * h + gg) * 16 + (j & 15)) * WPL) * 4;
                if constexpr (WPL == 4) {
                    const u32x4 v = *reinterpret_cast<const u32x4*>(p);
                    bw[jb][gg][0] = v[0]; bw[jb][gg][1] = v[1]; bw[jb][gg][2] = v[2]; bw[jb][gg][3] = v[3];
                } else if constexpr (WPL == 2) {
                    const u32x2 v = *reinterpret_cast<const u32x2*>(p);
                    bw[jb][gg][0] = v[0]; bw[jb][gg][1] = v[1];
                } else {
                    bw[jb][gg][0] = *reinterpret_cast<const uint32_t*>(p);
                }
            }
        }
        const bool tail = (s + 1) * SK > K;                  // uniform: the step holds padding k
        #pragma unroll
        for (int cc = 0; cc < KC; ++cc) {
            if constexpr (FMT == FMT_BINARY) {
                // lane half h: the 64 activations at 64h of the chunk, as the
                // operands of lane groups 2h (gg 0) and 2h + 1 (gg 1)
                i32x4 Ap[WMB][2][2];
                #pragma unroll
                for (int i = 0; i < WMB; ++i) {
                    i32x4 X[4];
                    #pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int c = 8 * cc + 4 * h + e;    // logical 16-byte chunk of the row
                        X[e] = *reinterpret_cast<const i32x4*>(st + arow0 + i * 32 * SK + 16 * (c ^ sw));
                        if (tail && s * SK + 16 * c >= K) X[e] = i32x4{0, 0, 0, 0};
                    }
                    #pragma unroll
                    for (int gg = 0; gg < 2; ++gg) {
                        const uint32_t Xw[8] = {(uint32_t)X[2 * gg][0], (uint32_t)X[2 * gg][1],
                                                (uint32_t)X[2 * gg][2], (uint32_t)X[2 * gg][3],
                                                (uint32_t)X[2 * gg + 1][0], (uint32_t)X[2 * gg + 1][1],
                                                (uint32_t)X[2 * gg + 1][2], (uint32_t)X[2 * gg + 1][3]};
                        perm_binary_a(Xw, Ap[i][gg][0], Ap[i][gg][1]);
                    }
                }
                #pragma unroll
                for (int gg = 0; gg < 2; ++gg) {
                    #pragma unroll
                    for (int op = 0; op < 2; ++op) {
                        #pragma unroll
                        for (int jb = 0; jb < WNB; ++jb) {
                            const i32x4 B = decode_binary_half(bw[jb][gg][cc], op);
                            #pragma unroll
                            for (int i = 0; i < WMB; ++i) C[i][jb] = mfma32(Ap[i][gg][op], B, C[i][jb]);
                        }
                    }
                }
            } else {
                i32x4 A[WMB][2];
                #pragma unroll
                for (int i = 0; i < WMB; ++i) {
                    #pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int c = 4 * cc + 2 * h + e;    // logical 16-byte chunk of the row
                        A[i][e] = *reinterpret_cast<const i32x4*>(st + arow0 + i * 32 * SK + 16 * (c ^ sw));
                    }
                }
                #pragma unroll
                for (int gg = 0; gg < 2; ++gg) {
                    #pragma unroll
                    for (int jb = 0; jb < WNB; ++jb) {
                        i32x4 B;
                        if constexpr (FMT == FMT_TERNARY) B = decode_ternary(bw[jb][gg][cc]);
                        else B = decode_int4(bw[jb][gg][2 * cc], bw[jb][gg][2 * cc + 1]);
                        #pragma unroll
                        for (int i = 0; i < WMB; ++i) C[i][jb] = mfma32(A[i][gg], B, C[i][jb]);
                        // this group's share of the next loads
                        const int d = (cc * 2 + gg) * WNB + jb;
                        if constexpr (FETCH) {
                            if (d < NDMA) {
                                issue_one(sf, d);
                            }
                        }
                    }
                }
            }
            if constexpr (FMT == FMT_BINARY) {
                #pragma unroll
                for (int jb = 0; jb < WNB; ++jb) {
                    const int d = cc * WNB + jb;
                    if constexpr (FETCH) {
                        if (d < NDMA) {
                            issue_one(sf, d);
                        }
                    }
                }
            }
            if constexpr (GROUP) {
                const int kbeg = s * SK + cc * CK;
                const int kend = kbeg + CK;
                if (kbeg < K && (kend % a.group == 0 || kend >= K)) close_groups(kend);   // uniform
            }
        }
        constexpr int SLOTS = FMT == FMT_BINARY ? KC * WNB : KC * 2 * WNB;
        #pragma unroll
        for (int d = SLOTS; d < NDMA; ++d)                   // loads beyond the MFMA groups
            if constexpr (FETCH) issue_one(sf, d);
    };
    int s = 0;
    for (; s + NS - 1 < n_steps; ++s) k_step(s, std::true_type{});
    for (; s < n_steps; ++s) k_step(s, std::false_type{});

    // ---- epilogue (every scale is loaded before the first store: the
    // compiler cannot tell y from sx and would otherwise wait per element).
    // Accumulator register r of block (i, jb) is token 32 i + 8 (r / 4) +
    // 4 h + r % 4 and row 32 jb + j of the wave's sub-tile.
    float sxv[WMB][16], swv[WNB];
    #pragma unroll
    for (int i = 0; i < WMB; ++i)
        #pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int tl = wm * (32 * WMB) + i * 32 + 8 * (r / 4) + 4 * h + (r % 4);
            if constexpr (XSL) sxv[i][r] = xs_x[tl];
            else sxv[i][r] = m_sx[min(m0 + tl, T - 1)];
        }
    #pragma unroll
    for (int jb = 0; jb < WNB; ++jb) {
        if constexpr (GROUP) {
            swv[jb] = 0.0f;
        } else if constexpr (XSL) {
            swv[jb] = xs_w[wn * (32 * WNB) + jb * 32 + j];
        } else {
            const int nc = min(n0 + wn * (32 * WNB) + jb * 32 + j, m_N - 1);
            swv[jb] = m_scales[a.scale_per_row ? nc : 0];
        }
    }
    if constexpr (GROUP) {
        #pragma unroll
        for (int jb = 0; jb < WNB; ++jb) {
            const int n = n0 + wn * (32 * WNB) + jb * 32 + j;
            #pragma unroll
            for (int i = 0; i < WMB; ++i)
                #pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int t = m0 + wm * (32 * WMB) + i * 32 + 8 * (r / 4) + 4 * h + (r % 4);
                    if (t < T && n < m_N)
                        __builtin_nontemporal_store(sxv[i][r] * (yp[i][jb][r] * (1.0f / (float)(1 << SHIFT))),
                                                    &m_y[(size_t)t * m_N + n]);
                }
        }
    } else {
        // Branch-free stores: buffer stores whose resource spans exactly this
        // workgroup's valid rows drop every out-of-range element in hardware
        // (columns past n get an offset past the end).  With a branch per
        // element the compiler would wait for all earlier stores before each.
        // Each store writes 32 consecutive columns of two token rows, with the
        // non-temporal hint: the output is written once and never read here,
        // and should not displace the activation and weight tiles other
        // workgroups re-read from L2 (measured: 4% faster int4 launches, 13%
        // on the binary model's output-bound pass).
        const int rows_here = min(BM, T - m0);
        const __amdgpu_buffer_rsrc_t ry =
            __builtin_amdgcn_make_buffer_rsrc(m_y + (size_t)m0 * m_N, 0, rows_here * m_N * 4, 0x00020000);
        const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
            m_acc ? (void*)(m_acc + (size_t)m0 * m_N) : (void*)m_y, 0, (ACC && m_acc) ? rows_here * m_N * 4 : 0,
            0x00020000);
        // column byte offsets; a column past n gets 2^30, beyond any resource
        // size here (rows * n * 4 <= 256 * 2^20 * 4)
        int col[WNB];
        #pragma unroll
        for (int jb = 0; jb < WNB; ++jb) {
            const int n = n0 + wn * (32 * WNB) + jb * 32 + j;
            col[jb] = n < m_N ? 4 * n : (1 << 30);
        }
        const int row_bytes = 4 * m_N;
        #pragma unroll
        for (int i = 0; i < WMB; ++i) {
            #pragma unroll
            for (int jb = 0; jb < WNB; ++jb) {
                #pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int tl = wm * (32 * WMB) + i * 32 + 8 * (r / 4) + 4 * h + (r % 4);   // row within the tile
                    const int off = tl * row_bytes + col[jb];
                    const int32_t v = C[i][jb][r] >> SHIFT;
                    const float yv = (float)v * (sxv[i][r] * swv[jb]);
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(yv), ry, off, 0, kStoreNT);
                    if constexpr (ACC) __builtin_amdgcn_raw_buffer_store_b32((uint32_t)v, ra, off, 0, kStoreNT);
                }
            }
        }
    }
}

template <int FMT, int WPL, int TILE>
void gemm_mfma_launch_tile(const GemmFastArgs& ga, bool group, bool acc, hipStream_t st) {
    const dim3 grid((unsigned)ga.wg_start[ga.n_mats]), block(64 * GemmShape<FMT, WPL, TILE>::NW);
    if (group) {                                             // group mode runs the small tile only
        if constexpr (TILE == 0) {
            if (acc) gemm_mfma_kernel<FMT, WPL, TILE, true, true><<<grid, block, 0, st>>>(ga);
            else gemm_mfma_kernel<FMT, WPL, TILE, true, false><<<grid, block, 0, st>>>(ga);
        }
    } else {
        if (acc) gemm_mfma_kernel<FMT, WPL, TILE, false, true><<<grid, block, 0, st>>>(ga);
        else gemm_mfma_kernel<FMT, WPL, TILE, false, false><<<grid, block, 0, st>>>(ga);
    }
}

// Tile choice: the least work on the busiest CU over all the launch's tiles,
// rounds of tiles per CU times the tile's area, weighted by how close each
// tile shape runs to the matrix cores' rate (the 256 x 256 tile best: two
// wavefronts per SIMD and the most MFMA work per staged byte).  Group mode
// runs the 128 x 128 tile only.
template <int FMT, int WPL>
void gemm_mfma_launch(GemmFastArgs ga, bool group, bool acc, hipStream_t st) {
    using Big = GemmShape<FMT, WPL, 1>;
    using Mid = GemmShape<FMT, WPL, 2>;
    using Small = GemmShape<FMT, WPL, 0>;
    const long cus = device_cu_count();
    auto tiles_of = [&](int bm, int bn) {
        long tiles = 0;
        for (int i = 0; i < ga.n_mats; ++i) tiles += (long)((ga.T + bm - 1) / bm) * ((ga.m[i].N + bn - 1) / bn);
        return tiles;
    };
    auto cost = [&](int bm, int bn, double eff) {
        return (double)((tiles_of(bm, bn) + cus - 1) / cus) * bm * bn / eff;
    };
    auto place = [&](int bm, int bn) {                       // token blocks, row blocks, first workgroups
        ga.mb = (ga.T + bm - 1) / bm;
        int wgs = 0;
        for (int i = 0; i < ga.n_mats; ++i) {
            ga.m[i].nb = (ga.m[i].N + bn - 1) / bn;
            ga.wg_start[i] = wgs;
            wgs += ga.mb * ga.m[i].nb;
        }
        ga.wg_start[ga.n_mats] = wgs;
        for (int i = ga.n_mats + 1; i <= kGemmMaxMats; ++i) ga.wg_start[i] = 0x7fffffff;
    };
    const double c_big = Big::FITS && !group ? cost(Big::BM, Big::BN, 1.0) : 1e300;
    const double c_mid = Mid::FITS && !group ? cost(Mid::BM, Mid::BN, 0.9) : 1e300;
    const double c_small = cost(Small::BM, Small::BN, 0.8);
    if (c_big <= c_mid && c_big <= c_small) {
        place(Big::BM, Big::BN);
        if constexpr (Big::FITS) gemm_mfma_launch_tile<FMT, WPL, 1>(ga, false, acc, st);
    } else if (c_mid <= c_small) {
        place(Mid::BM, Mid::BN);
        if constexpr (Mid::FITS) gemm_mfma_launch_tile<FMT, WPL, 2>(ga, false, acc, st);
    } else {
        place(Small::BM, Small::BN);
        gemm_mfma_launch_tile<FMT, WPL, 0>(ga, group, acc, st);
    }
}

bool gemm_mfma_supported(const LinearArgs& a) {
    // (n bound: the epilogue's 32-bit buffer offsets span 256 rows of y)
    return a.k % 16 == 0 && (uintptr_t)a.q % 16 == 0 && (uintptr_t)a.packed % 16 == 0 && a.n <= (1 << 20);
}

// `count` products of equal fmt, scale mode, group, k and t, every one
// gemm_mfma_supported: as few launches as kGemmMaxMats allows, of near-equal
// size (a short last launch would run mostly as a tail).
hipError_t launch_gemm_mfma_group(const LinearArgs* mats, int count, hipStream_t stream) {
    const int launches = (count + kGemmMaxMats - 1) / kGemmMaxMats;
    for (int li = 0, b = 0; li < launches; ++li) {
        const int e = (int)((int64_t)count * (li + 1) / launches);
        const int n = e - b;
        const LinearArgs& a = mats[b];
        GemmFastArgs ga{};
        ga.T = a.t; ga.K = a.k;
        ga.n_steps = a.n_steps;
        const bool group = a.scale == LOWBIT_SCALE_GROUP;
        ga.group = group ? a.group : 0;
        ga.G = group ? a.n_groups : 1;
        ga.scale_per_row = a.scale == LOWBIT_SCALE_ROW;
        ga.n_mats = n;
        bool acc = false;
        for (int i = 0; i < n; ++i) {
            const LinearArgs& c = mats[b + i];
            GemmMat& m = ga.m[i];
            m.packed = c.packed; m.scales = c.scales; m.q = c.q; m.sx = c.sx; m.y = c.y; m.acc = c.acc;
            m.N = c.n;
            m.n_tiles = (c.n + 15) / 16;
            acc = acc || c.acc != nullptr;
        }
        switch (a.fmt) {
            case FMT_TERNARY:
                if (a.wpl == 4) gemm_mfma_launch<FMT_TERNARY, 4>(ga, group, acc, stream);
                else if (a.wpl == 2) gemm_mfma_launch<FMT_TERNARY, 2>(ga, group, acc, stream);
                else gemm_mfma_launch<FMT_TERNARY, 1>(ga, group, acc, stream);
                break;
            case FMT_INT4:
                if (a.wpl == 4) gemm_mfma_launch<FMT_INT4, 4>(ga, group, acc, stream);
                else gemm_mfma_launch<FMT_INT4, 2>(ga, group, acc, stream);
                break;
            default:
                if (a.wpl == 4) gemm_mfma_launch<FMT_BINARY, 4>(ga, group, acc, stream);
                else if (a.wpl == 2) gemm_mfma_launch<FMT_BINARY, 2>(ga, group, acc, stream);
                else gemm_mfma_launch<FMT_BINARY, 1>(ga, group, acc, stream);
                break;
        }
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        b = e;
    }
    return hipSuccess;
}

hipError_t launch_gemm_mfma(const LinearArgs& a, hipStream_t stream) { return launch_gemm_mfma_group(&a, 1, stream); }

}  // namespace lowbit
