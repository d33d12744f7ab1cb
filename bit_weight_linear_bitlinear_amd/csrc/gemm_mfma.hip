// gemm_mfma.hip - prefill-shaped low-bit product on the gfx950 matrix cores,
// the streaming path (k a multiple of 16, activation codes 16-byte aligned).
//
// What it computes (M8.8 "Native Binary and Ternary Transformers", 0x02D,
// 0x09C): acc[t, n] = sum_k q[t, k] * code[n, k] exactly in int32 (per scale
// group in group mode), then the fp32 rescale.  Prefill is a dense contraction
// (0x09B), so the work is v_mfma_i32_16x16x64_i8 with the packed codes decoded
// in registers right before each MFMA.
//
// Tiling.  A 256-thread workgroup owns a 128-token x 128-row output tile; its
// four wavefronts are a 2 x 2 grid of 64 x 64 sub-tiles (4 x 4 MFMA blocks).
// k advances one packed-layout k-step (SK codes) at a time.  Each step's
// operands are copied global -> LDS by the memory unit itself (16-byte
// direct-to-LDS loads: no registers, no LDS write instructions), NS steps in
// flight:
//  - activations: 1 KB LDS pieces, one per (64-k chunk, 16-token block), laid
//    out exactly as an MFMA A operand (lane l: token l % 16, bytes 16 (l / 16)
//    .. of the chunk; binary chunks follow the quarter / half order of a
//    128-code block), so every operand read is one contiguous, conflict-free
//    1 KB ds_read_b128;
//  - weights: the packed (16-row tile, k-step) blocks, copied as they are - the
//    packed layout already is the per-lane B operand order.
// The compiler does not track the LDS side of these loads, so the pipeline
// waits with explicit vmcnt counts (every load of a step is unconditional)
// followed by a workgroup barrier.  Tokens past t and rows past n read clamped
// (valid) addresses; their results are never stored.  Binary activations past
// k are zeroed in registers (binary padding codes decode as +1; ternary and
// int4 padding codes are 0).
//
// Workgroups are numbered so that each XCD (workgroup i runs on XCD i % 8)
// owns a contiguous run of output tiles, token-block-major: the weight matrix
// and a few activation blocks stay in that XCD's L2.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace lowbit {

struct GemmFastArgs {
    const uint8_t* packed;
    const float* scales;
    const int8_t* q;
    const float* sx;
    float* y;
    int32_t* acc;
    int T, N, K;
    int n_steps;        // packed-layout k-steps
    int n_tiles;        // ceil(N / 16)
    int group;          // group mode: columns per group
    int G;              // group mode: groups per row
    int scale_per_row;
    int mb, nb;         // token blocks, row blocks (of 128)
};

// Workgroup tile configurations.  TILE 0: 2 x 2 wavefronts of 64 tokens x 64
// rows (4 x 4 MFMA blocks), a 128 x 128 tile, two workgroups per CU.
// TILE 1: 2 x 4 wavefronts of 128 tokens x 64 rows (8 x 4 blocks), a 256 x 256
// tile - twice the MFMA work per staged byte - with eight wavefronts, i.e. two
// per SIMD (one wavefront alone cannot issue i8 MFMAs back to back).
template <int TILE> struct TileCfg;
template <> struct TileCfg<0> {
    static constexpr int WAVES_M = 2, WAVES_N = 2, WMB = 4, WNB = 4, BUDGET = 73728;
};
template <> struct TileCfg<1> {
    static constexpr int WAVES_M = 2, WAVES_N = 4, WMB = 8, WNB = 4, BUDGET = 163840;
};

template <int FMT, int WPL, int TILE> struct GemmShape {
    using TC = TileCfg<TILE>;
    static constexpr int WAVES_M = TC::WAVES_M, WAVES_N = TC::WAVES_N, WMB = TC::WMB, WNB = TC::WNB;
    static constexpr int NW = WAVES_M * WAVES_N;             // wavefronts per workgroup
    static constexpr int CPW = Fmt<FMT>::kCodesPerWord;
    static constexpr int SK = 4 * WPL * CPW;                // k per packed-layout step
    static constexpr int KC = SK / 64;                       // 64-k MFMA chunks per step
    static constexpr int BM = 16 * WMB * WAVES_M, BN = 16 * WNB * WAVES_N;
    static constexpr int TBLK = BM / 16, NTILE = BN / 16;    // 16-token blocks, 16-row tiles
    static constexpr int A_BYTES = BM * SK;
    static constexpr int B_BYTES = NTILE * 256 * WPL;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int NS = 3 * STAGE <= TC::BUDGET ? 3 : 2;   // steps in flight
    static constexpr int A_PIECES = A_BYTES / 1024;          // 1 KB direct loads per step
    static constexpr int B_PIECES = B_BYTES / 1024;
    static constexpr bool FITS = NS * STAGE <= 163840;
};

// one 1 KB direct-to-LDS copy: lane l's 16 bytes land at lds + 16 * l
__device__ __forceinline__ void dma16(const void* src, void* lds) {
    __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    // the direct loads write LDS behind the compiler's back: wait explicitly,
    // and keep every LDS access on its side of the wait
    if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if constexpr (N == 1) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
    else if constexpr (N == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
    else if constexpr (N == 3) asm volatile("s_waitcnt vmcnt(3)" ::: "memory");
    else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else if constexpr (N == 5) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
    else if constexpr (N == 6) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else if constexpr (N == 9) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
    else if constexpr (N == 10) asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
    else if constexpr (N == 12) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
    else if constexpr (N == 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else if constexpr (N == 17) asm volatile("s_waitcnt vmcnt(17)" ::: "memory");
    else if constexpr (N == 18) asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
    else if constexpr (N == 20) asm volatile("s_waitcnt vmcnt(20)" ::: "memory");
    else if constexpr (N == 34) asm volatile("s_waitcnt vmcnt(34)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // any other count: wait for everything
}

template <int FMT, int WPL, int TILE, bool GROUP, bool ACC>
__global__ __launch_bounds__(TILE == 0 ? 256 : 512) void gemm_mfma_kernel(const GemmFastArgs a) {
    using S = GemmShape<FMT, WPL, TILE>;
    constexpr int SK = S::SK, KC = S::KC, NS = S::NS, STAGE = S::STAGE, A_BYTES = S::A_BYTES;
    constexpr int BM = S::BM, BN = S::BN, TBLK = S::TBLK, NW = S::NW;
    constexpr int WMB = S::WMB, WNB = S::WNB;
    constexpr int SHIFT = Fmt<FMT>::kShift;
    // direct loads per wave per step: the fewest any wave issues (waits are
    // then exact or conservative for every wave)
    constexpr int LA = S::A_PIECES / NW;
    constexpr int LB = S::B_PIECES / NW;                     // 0: waves 0 .. B_PIECES-1 issue one
    constexpr int L = LA + LB;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[NS * STAGE];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, g = lane >> 4, rl = lane & 15;
    const int wm = wave / S::WAVES_N, wn = wave % S::WAVES_N;

    // XCD-aware tile order: XCD x runs a contiguous run of tiles
    const int total = a.mb * a.nb;
    const int xcd = (int)blockIdx.x % 8, j = (int)blockIdx.x / 8;
    const int logical = xcd * (total / 8) + min(xcd, total % 8) + j;
    const int tb_m = logical / a.nb, tb_n = logical % a.nb;
    const int m0 = tb_m * BM, n0 = tb_n * BN;
    const int K = a.K, T = a.T;

    // ---- per-lane source addresses of this workgroup's direct loads
    // activation pieces: piece kc * TBLK + tb holds 64-k chunk kc of token
    // block tb; wave w issues the token blocks w, w + NW, ... of every chunk,
    // lane (g, tok) reading 16 bytes of its row
    constexpr int TBW = TBLK / NW;                           // token blocks per wave
    const int8_t* arow[TBW];
    #pragma unroll
    for (int ii = 0; ii < TBW; ++ii)
        arow[ii] = a.q + (size_t)min(m0 + (wave + NW * ii) * 16 + rl, T - 1) * K;
    auto a_off = [&](int kc) -> int {                        // k offset of chunk kc within a step
        if constexpr (FMT == FMT_BINARY) return (kc / 2) * 128 + 32 * g + 16 * (kc % 2);
        else return kc * 64 + 16 * g;
    };
    // weight piece p: 16-byte chunk c = 64 p + lane of the stage's row tiles
    constexpr int LBW = LB > 0 ? LB : 1;
    const uint8_t* b_src[LBW];
    #pragma unroll
    for (int i = 0; i < LBW; ++i) {
        const int p = LB > 0 ? wave + NW * i : wave;
        const int c = 64 * p + lane;
        const int tt = c / (16 * WPL), cc = c % (16 * WPL);
        const int tile = min(tb_n * S::NTILE + tt, a.n_tiles - 1);
        b_src[i] = a.packed + (size_t)tile * a.n_steps * (256 * WPL) + cc * 16;
    }

    // The direct loads of one step, numbered 0 .. NDMA-1 for this wave:
    // activation pieces first (chunk kc, token block ii), then weight pieces.
    constexpr int NDMA = LA + (LB > 0 ? LB : 1);
    auto issue_one = [&](int s, int d) {
        uint8_t* st = smem + (s % NS) * STAGE;
        if (d < LA) {
            const int kc = d / TBW, ii = d % TBW;
            const int k = s * SK + a_off(kc);
            dma16(arow[ii] + (k < K ? k : 0), st + (kc * TBLK + wave + NW * ii) * 1024);
        } else if constexpr (LB > 0) {
            const int i = d - LA;
            dma16(b_src[i] + (size_t)s * (256 * WPL), st + A_BYTES + (wave + NW * i) * 1024);
        } else {
            if (wave < S::B_PIECES) dma16(b_src[0] + (size_t)s * (256 * WPL), st + A_BYTES + wave * 1024);
        }
    };
    auto issue = [&](int s) {                                // all direct loads of step s
        #pragma unroll
        for (int d = 0; d < NDMA; ++d) issue_one(s, d);
    };

    i32x4 C[WMB][WNB];
    #pragma unroll
    for (int i = 0; i < WMB; ++i)
        #pragma unroll
        for (int jj = 0; jj < WNB; ++jj) C[i][jj] = i32x4{0, 0, 0, 0};
    float yp[GROUP ? WMB : 1][GROUP ? WNB : 1][4];
    if constexpr (GROUP) {
        #pragma unroll
        for (int i = 0; i < WMB; ++i)
            #pragma unroll
            for (int jj = 0; jj < WNB; ++jj)
                #pragma unroll
                for (int r = 0; r < 4; ++r) yp[i][jj][r] = 0.0f;
    }

    // group mode: the k-chunks ending at kend close a group
    auto close_groups = [&](int kend) {
        const int gi = (min(kend, K) - 1) / a.group;
        #pragma unroll
        for (int jj = 0; jj < WNB; ++jj) {
            const int n = n0 + wn * (16 * WNB) + jj * 16 + rl;
            const int nc = min(n, a.N - 1);
            const float sg = a.scales[((size_t)(nc >> 4) * a.G + gi) * 16 + (nc & 15)];
            #pragma unroll
            for (int i = 0; i < WMB; ++i) {
                #pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int32_t v = C[i][jj][r] >> SHIFT;
                    yp[i][jj][r] = yp[i][jj][r] + sg * (float)v;
                    if constexpr (ACC) {
                        const int t = m0 + wm * (16 * WMB) + i * 16 + 4 * g + r;
                        if (a.acc && t < T && n < a.N) a.acc[((size_t)t * a.N + n) * a.G + gi] = v;
                    }
                }
                C[i][jj] = i32x4{0, 0, 0, 0};
            }
        }
    };

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
        // spread over this step's MFMA groups, one after each group: issued
        // all at once, every wave would stall behind the others' requests.
        const int sf = s + NS - 1;

        const uint8_t* st = smem + (s % NS) * STAGE;
        const uint8_t* bs = st + A_BYTES;
        uint32_t bw[WNB][WPL];                               // this lane's packed words of the step
        #pragma unroll
        for (int jj = 0; jj < WNB; ++jj) {
            const uint8_t* p = bs + (wn * WNB + jj) * (256 * WPL) + lane * (4 * WPL);
            if constexpr (WPL == 4) {
                const u32x4 v = *reinterpret_cast<const u32x4*>(p);
                bw[jj][0] = v[0]; bw[jj][1] = v[1]; bw[jj][2] = v[2]; bw[jj][3] = v[3];
            } else if constexpr (WPL == 2) {
                const u32x2 v = *reinterpret_cast<const u32x2*>(p);
                bw[jj][0] = v[0]; bw[jj][1] = v[1];
            } else {
                bw[jj][0] = *reinterpret_cast<const uint32_t*>(p);
            }
        }
        const bool tail = (s + 1) * SK > K;                  // uniform: the step holds padding k
        #pragma unroll
        for (int kc = 0; kc < KC; kc += (FMT == FMT_BINARY ? 2 : 1)) {
            i32x4 Aop[WMB][FMT == FMT_BINARY ? 2 : 1];
            #pragma unroll
            for (int i = 0; i < WMB; ++i) {
                const uint8_t* ap = st + (kc * TBLK + wm * WMB + i) * 1024 + lane * 16;
                Aop[i][0] = *reinterpret_cast<const i32x4*>(ap);
                if constexpr (FMT == FMT_BINARY) {
                    i32x4 lo = Aop[i][0];
                    i32x4 hi = *reinterpret_cast<const i32x4*>(ap + TBLK * 1024);
                    if (tail) {
                        const int k0 = s * SK + (kc / 2) * 128 + 32 * g;
                        if (k0 >= K) lo = i32x4{0, 0, 0, 0};
                        if (k0 + 16 >= K) hi = i32x4{0, 0, 0, 0};
                    }
                    const uint32_t X[8] = {(uint32_t)lo[0], (uint32_t)lo[1], (uint32_t)lo[2], (uint32_t)lo[3],
                                           (uint32_t)hi[0], (uint32_t)hi[1], (uint32_t)hi[2], (uint32_t)hi[3]};
                    perm_binary_a(X, Aop[i][0], Aop[i][1]);
                }
            }
            #pragma unroll
            for (int jj = 0; jj < WNB; ++jj) {
                if constexpr (FMT == FMT_TERNARY) {
                    const i32x4 B = decode_ternary(bw[jj][kc]);
                    #pragma unroll
                    for (int i = 0; i < WMB; ++i) C[i][jj] = mfma16(Aop[i][0], B, C[i][jj]);
                } else if constexpr (FMT == FMT_INT4) {
                    const i32x4 B = decode_int4(bw[jj][2 * kc], bw[jj][2 * kc + 1]);
                    #pragma unroll
                    for (int i = 0; i < WMB; ++i) C[i][jj] = mfma16(Aop[i][0], B, C[i][jj]);
                } else {
                    i32x4 b0, b1;
                    decode_binary(bw[jj][kc / 2], b0, b1);
                    #pragma unroll
                    for (int i = 0; i < WMB; ++i) {
                        C[i][jj] = mfma16(Aop[i][0], b0, C[i][jj]);
                        C[i][jj] = mfma16(Aop[i][1], b1, C[i][jj]);
                    }
                }
            }
            #pragma unroll
            for (int jj = 0; jj < WNB; ++jj) {               // this chunk's share of the next loads
                const int d = (FMT == FMT_BINARY ? kc / 2 : kc) * WNB + jj;
                if constexpr (FETCH) {
                    if (d < NDMA) {
                        issue_one(sf, d);
                        __builtin_amdgcn_sched_barrier(0);     // keep it after this group
                    }
                }
            }
            if constexpr (GROUP) {
                const int kw = FMT == FMT_BINARY ? 128 : 64;
                const int kbeg = s * SK + (FMT == FMT_BINARY ? kc / 2 * 128 : kc * 64);
                const int kend = kbeg + kw;
                if (kbeg < K && (kend % a.group == 0 || kend >= K)) close_groups(kend);   // uniform
            }
        }
        constexpr int SLOTS = (FMT == FMT_BINARY ? KC / 2 : KC) * WNB;
        #pragma unroll
        for (int d = SLOTS; d < NDMA; ++d)                   // loads beyond the MFMA groups
            if constexpr (FETCH) issue_one(sf, d);
    };
    int s = 0;
    for (; s + NS - 1 < n_steps; ++s) k_step(s, std::true_type{});
    for (; s < n_steps; ++s) k_step(s, std::false_type{});

    // ---- epilogue (every scale is loaded before the first store: the
    // compiler cannot tell y from sx and would otherwise wait per element)
    float sxv[WMB][4], swv[WNB];
    #pragma unroll
    for (int i = 0; i < WMB; ++i)
        #pragma unroll
        for (int r = 0; r < 4; ++r) sxv[i][r] = a.sx[min(m0 + wm * (16 * WMB) + i * 16 + 4 * g + r, T - 1)];
    #pragma unroll
    for (int jj = 0; jj < WNB; ++jj) {
        const int nc = min(n0 + wn * (16 * WNB) + jj * 16 + rl, a.N - 1);
        swv[jj] = GROUP ? 0.0f : a.scales[a.scale_per_row ? nc : 0];
    }
    if constexpr (GROUP) {
        #pragma unroll
        for (int jj = 0; jj < WNB; ++jj) {
            const int n = n0 + wn * (16 * WNB) + jj * 16 + rl;
            #pragma unroll
            for (int i = 0; i < WMB; ++i)
                #pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = m0 + wm * (16 * WMB) + i * 16 + 4 * g + r;
                    if (t < T && n < a.N) a.y[(size_t)t * a.N + n] = sxv[i][r] * yp[i][jj][r];
                }
        }
    } else {
        // Branch-free stores: buffer stores whose resource spans exactly this
        // workgroup's valid rows drop every out-of-range element in hardware
        // (columns past n get an offset past the end).  With a branch per
        // element the compiler would wait for all earlier stores before each.
        const int rows_here = min(BM, T - m0);
        const __amdgpu_buffer_rsrc_t ry =
            __builtin_amdgcn_make_buffer_rsrc(a.y + (size_t)m0 * a.N, 0, rows_here * a.N * 4, 0x00020000);
        const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
            a.acc ? (void*)(a.acc + (size_t)m0 * a.N) : (void*)a.y, 0, (ACC && a.acc) ? rows_here * a.N * 4 : 0,
            0x00020000);
        // column byte offsets; a column past n gets 2^30, beyond any resource
        // size here (rows * n * 4 <= 256 * 2^20 * 4)
        int col[WNB];
        #pragma unroll
        for (int jj = 0; jj < WNB; ++jj) {
            const int n = n0 + wn * (16 * WNB) + jj * 16 + rl;
            col[jj] = n < a.N ? 4 * n : (1 << 30);
        }
        const int row_bytes = 4 * a.N;
        if (ACC || (a.N & 3) != 0) {
            // one element per store (and the integer products when asked for)
            #pragma unroll
            for (int jj = 0; jj < WNB; ++jj) {
                #pragma unroll
                for (int i = 0; i < WMB; ++i) {
                    #pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int tl = wm * (16 * WMB) + i * 16 + 4 * g + r;      // row within the tile
                        const int off = tl * row_bytes + col[jj];
                        const int32_t v = C[i][jj][r] >> SHIFT;
                        const float yv = (float)v * (sxv[i][r] * swv[jj]);
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(yv), ry, off, 0, 0);
                        if constexpr (ACC) __builtin_amdgcn_raw_buffer_store_b32((uint32_t)v, ra, off, 0, 0);
                    }
                }
            }
        } else {
            // Through LDS, one 16-token block row at a time: the MFMA layout
            // gives each lane 4 rows x 1 column per block, i.e. 64-byte row
            // pieces; re-read row-major, every store is 16 bytes per lane and
            // covers whole 64 * WB-byte row segments.
            constexpr int WC = 16 * WNB;                     // columns of the wave's tile
            constexpr int LD = WC + 4;                       // LDS row stride in floats (16-byte aligned)
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();                    // every wave is done with the pipeline buffers
            asm volatile("" ::: "memory");
            float* ws = reinterpret_cast<float*>(smem) + wave * (16 * LD);
            #pragma unroll
            for (int i = 0; i < WMB; ++i) {
                #pragma unroll
                for (int jj = 0; jj < WNB; ++jj)
                    #pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int32_t v = C[i][jj][r] >> SHIFT;
                        ws[(4 * g + r) * LD + jj * 16 + rl] = (float)v * (sxv[i][r] * swv[jj]);
                    }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // (the wave's own region only)
                #pragma unroll
                for (int it = 0; it < 16 * WC / 4 / 64; ++it) {
                    const int c = it * 64 + lane;             // 16-byte chunk of the block row
                    const int rr = c / (WC / 4), c4 = c % (WC / 4);
                    const u32x4 v = *reinterpret_cast<const u32x4*>(ws + rr * LD + 4 * c4);
                    const int n = n0 + wn * WC + 4 * c4;
                    const int tl = wm * (16 * WMB) + i * 16 + rr;
                    const int off = tl * row_bytes + (n < a.N ? 4 * n : (1 << 30));
                    __builtin_amdgcn_raw_buffer_store_b128(v, ry, off, 0, 0);
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // reads done before the next block row
            }
        }
    }
}

template <int FMT, int WPL, int TILE>
void gemm_mfma_launch_tile(const GemmFastArgs& ga, bool group, bool acc, hipStream_t st) {
    const dim3 grid((unsigned)(ga.mb * ga.nb)), block(64 * GemmShape<FMT, WPL, TILE>::NW);
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

// Tile choice: the 256 x 256 tile whenever it still gives most CUs a
// workgroup; else 128 x 128 (two workgroups per CU).
template <int FMT, int WPL>
void gemm_mfma_launch(GemmFastArgs ga, bool group, bool acc, hipStream_t st) {
    using Big = GemmShape<FMT, WPL, 1>;
    using Small = GemmShape<FMT, WPL, 0>;
    const int big_tiles = ((ga.T + Big::BM - 1) / Big::BM) * ((ga.N + Big::BN - 1) / Big::BN);
    if (Big::FITS && !group && big_tiles >= 192) {
        ga.mb = (ga.T + Big::BM - 1) / Big::BM;
        ga.nb = (ga.N + Big::BN - 1) / Big::BN;
        if constexpr (Big::FITS) gemm_mfma_launch_tile<FMT, WPL, 1>(ga, false, acc, st);
    } else {
        ga.mb = (ga.T + Small::BM - 1) / Small::BM;
        ga.nb = (ga.N + Small::BN - 1) / Small::BN;
        gemm_mfma_launch_tile<FMT, WPL, 0>(ga, group, acc, st);
    }
}

bool gemm_mfma_supported(const LinearArgs& a) {
    // (n bound: the epilogue's 32-bit buffer offsets span 256 rows of y)
    return a.k % 16 == 0 && (uintptr_t)a.q % 16 == 0 && (uintptr_t)a.packed % 16 == 0 && a.n <= (1 << 20);
}

hipError_t launch_gemm_mfma(const LinearArgs& a, hipStream_t stream) {
    GemmFastArgs ga;
    ga.packed = a.packed; ga.scales = a.scales; ga.q = a.q; ga.sx = a.sx; ga.y = a.y; ga.acc = a.acc;
    ga.T = a.t; ga.N = a.n; ga.K = a.k;
    ga.n_steps = a.n_steps;
    ga.n_tiles = (a.n + 15) / 16;
    const bool group = a.scale == LOWBIT_SCALE_GROUP;
    ga.group = group ? a.group : 0;
    ga.G = group ? a.n_groups : 1;
    ga.scale_per_row = a.scale == LOWBIT_SCALE_ROW;
    const bool acc = a.acc != nullptr;
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
    return hipGetLastError();
}

}  // namespace lowbit
