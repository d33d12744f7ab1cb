// gemv_kernel.hpp - decode-shaped low-bit product: t <= 16 tokens per launch,
// one or many weight matrices of equal k per launch.
//
// What it computes (M8.8 "Native Binary and Ternary Transformers", 0x02D,
// 0x05D, 0x09C):  acc[t, n] = sum_k q[t, k] * code[n, k] exactly in int32,
// then y = fp32 rescale (tensor/row scales) or a sum of per-group rescaled
// partials (group scales).
//
// Why this shape: decode streams each packed weight byte once (decode has a
// small token dimension and re-reads large weight matrices every token,
// 0x09B), so the kernel is HBM-bound and the work per packed byte must stay
// small.  Per 16 codes it spends 7 VALU ops (shift + mask decode) and hands
// the multiply-accumulate to one quarter of an i8 MFMA; the token dimension
// (<= 16) rides in the MFMA's M side, so t = 1 and t = 16 stream the same
// weight bytes.
//
// Mapping.  A 16-row tile of W is one MFMA column block: lane l holds weight
// row (l % 16) and lane group (l / 16) holds a quarter of every block, which
// is exactly how the packed layout orders a (tile, k-step) - so a wavefront
// reads one k-step of its tile as ONE contiguous 256 * wpl-byte block, one
// 4 * wpl-byte load per lane (1 KB per wavefront for wpl = 4), with the
// non-temporal hint (the stream is read once and must not evict the reused
// activation and scale lines).  Each wavefront keeps the loads of the next D
// k-steps in flight (a register ring, refilled right after each step is
// consumed).  The activation codes (the
// MFMA A operand: tokens x k) are staged once per workgroup in LDS, zero
// padded to whole k-steps, and read from there; binary activations are staged
// already permuted to the packbits code order.  When t * k is too large for
// LDS they ride in the register ring instead, read from L2.
//
// A workgroup is WV wavefronts (4, or 16 sharing a large LDS stage) on
// WV / ksplit consecutive tiles of ONE matrix;
// `ksplit` wavefronts share a tile's k-range and add their partials in LDS in
// a fixed order.  Group scales are applied per scale unit (a whole number of
// MFMA blocks inside one group): at a group's last unit the int32 partial is
// converted and accumulated in fp32 with the group's scale.
#pragma once

#include <climits>
#include <type_traits>

#include "device_common.hpp"
#include "gemv.hpp"
#include "lowbit.h"

namespace lowbit {


template <int FMT, int WPL> struct GemvShape {
    static constexpr int kKB = FMT == FMT_BINARY ? 128 : 64;    // k per block (one MFMA k-extent per quarter)
    static constexpr int kWB = FMT == FMT_INT4 ? 2 : 1;         // words per lane per block
    static constexpr int kNB = WPL / kWB;                        // blocks per k-step
    static constexpr int kSK = 4 * WPL * Fmt<FMT>::kCodesPerWord;  // k per k-step
    static constexpr int kMPB = FMT == FMT_BINARY ? 2 : 1;      // MFMAs per block
    static constexpr int kStepBytes = 256 * WPL;                 // bytes of one (tile, k-step)
};

// 16 activation bytes q[k0 .. k0 + 16) of one token row, zero past K
// (vec_only: the caller knows vec holds, and the partial-load code is left out).
__device__ __forceinline__ i32x4 load_q16(const int8_t* qrow, int k0, int K, bool vec, bool vec_only = false) {
    i32x4 v = {0, 0, 0, 0};
    if (k0 < K) {
        if (vec_only || vec) {
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

// The codes of four consecutive activations v (scale factor r), packed
// little first; the elements from `valid` on are past K and give 0.
__device__ __forceinline__ uint32_t quant_word(const float4 v, float r, int valid) {
    const float e[4] = {v.x, v.y, v.z, v.w};
    uint32_t w = 0;
    #pragma unroll
    for (int i = 0; i < 4; ++i)
        if (i < valid) w |= (uint32_t)(uint8_t)quant1(e[i], r) << (8 * i);
    return w;
}

// Sixteen-wavefront workgroups are asked for 8 waves per SIMD (64 VGPRs), so
// that two of them share a CU: at the compiler's own choice the ternary and
// int4 kernels take 65-70 registers and one workgroup per CU, which leaves a
// 360-workgroup launch two rounds deep.  The binary kernels (two MFMAs per
// block), ternary with four scale units per k-step, several units per group
// with four token registers, and the kernels that also write the integer
// products would spill at 64.
constexpr int gemv_min_waves(int fmt, int nr, int sps, bool upg1, int wv, bool acc) {
    const bool spills = fmt == FMT_BINARY || acc || (fmt == FMT_TERNARY && sps == 4) || (sps > 0 && !upg1 && nr == 4);
    return wv == 16 && !spills ? 8 : 1;
}

// NR: C registers per lane holding live tokens.  MFMA output row i = 4 g + r
// (lane group g, register r).  With NR = 1 (t <= 4) row i carries token
// g + 4 r, so the four tokens sit in register 0 of the four lane groups and a
// group epilogue converts one register per lane, not four; with NR = 4 row i
// carries token i (the 16 A rows of one LDS read then start on distinct
// banks).
// SPS: group mode: scale units per k-step; 0 = tensor/row scales.
// UPG1: group mode: every scale unit is a whole group.
// LDSA: activations staged in LDS.  ACC: also write the integer products
// (kept out of the streaming instantiations: optional stores inside the
// k-loop make the compiler's wait counting conservative).
// WV: wavefronts per workgroup (4; 16 only for LDSA without FUSE).
// PRE (with FUSE, one load round): what the prologue quantises.  PRE_NONE: x.
// PRE_NORM: h = RMSNorm(x + r; g) (r nullable), the residual sum and h
// written out by the launch's first workgroup (a decoder block's residual add
// and the norm before its next projection).  PRE_SWIGLU: a = SiLU(x) * up
// (the gated FFN between gate/up and down), a written out likewise.
// FUSE (with LDSA, one token): the stage is filled from fp32 x by the
// per-token absmax quantiser itself (M8.8 0x02C, 0x05C: m = max|x|,
// r = 127 / m, codes clip(rint(x r)), s_x = m / 127), every workgroup for its
// own stage; the matrix's first workgroup also writes the codes and scale out.
// FRW (with FUSE): words of x per thread per load round of the prologue
// quantiser.
template <int FMT, int WPL, int NR, int SPS, bool UPG1, bool LDSA, bool ACC, bool FUSE, int WV, int PRE, int FRW = 3>
__global__ __launch_bounds__(64 * WV) __attribute__((amdgpu_waves_per_eu(gemv_min_waves(FMT, NR, SPS, UPG1, WV, ACC)))) void gemv_kernel(const GemvParams p) {
    using S = GemvShape<FMT, WPL>;
    constexpr int D = kGemvD;
    constexpr int NB = S::kNB, KB = S::kKB, SK = S::kSK, MPB = S::kMPB;
    constexpr int STEP = S::kStepBytes;
    constexpr bool GROUP = SPS > 0;
    constexpr int NU = GROUP ? SPS : 1;                      // scale loads per k-step
    constexpr int BPU = GROUP ? NB / SPS : NB;               // blocks per scale unit
    constexpr int NA = LDSA ? 1 : NB * MPB;                  // ring-held activation operands
    constexpr int SHIFT = Fmt<FMT>::kShift;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    static_assert(!FUSE || LDSA, "the fused quantiser fills the LDS stage");
    static_assert(WV == 4 || (WV == 16 && LDSA && !FUSE), "16-wavefront workgroups share an LDS stage");
    static_assert(PRE == PRE_NONE || FUSE, "the input transforms run in the fused prologue");
    constexpr int NT = 64 * WV;                              // threads per workgroup
    __shared__ float fz_m[4];                                // fused: per-wave max |x|
    __shared__ int fz_bad[4];                                // fused: per-wave non-finite flag
    __shared__ float fz_ss[4];                               // PRE_NORM: per-wave sum of squares

    // the wavefront index is uniform; saying so keeps every value derived
    // from it (tile, part, k-range) in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;                                 // lane group
    const int rl = lane & 15;                                // weight row in the tile / token of A

    // matrix of this workgroup: a binary search of the ascending workgroup
    // starts (log2 n_mats dependent scalar loads; a scan of the whole table
    // cost more than it saved once a launch holds a hundred matrices)
    int mi = 0, hi = p.n_mats - 1;
    while (mi < hi) {
        const int mid = (mi + hi + 1) >> 1;
        if ((int)blockIdx.x >= p.wg_start[mid]) mi = mid;
        else hi = mid - 1;
    }
    const GemvMat& M = p.m[mi];
    const int part = wave & (p.ksplit - 1);
    const int tile_raw = ((int)blockIdx.x - p.wg_start[mi]) * p.tiles_per_wg + (wave >> p.ksplit_log);
    const bool live = tile_raw < M.n_tiles;                  // uniform
    const int tile = live ? tile_raw : M.n_tiles - 1;
    const int s0 = part * p.part_len;
    const int s_cnt = live ? min(p.n_steps - s0, p.part_len) : 0;
    const int s_loop = (s_cnt + D - 1) / D * D;
    const int K = p.K, T = p.T;
    // token of A row rl (rows of t >= T are never stored), and of output
    // register r of lane group g
    const int tok = min(NR == 1 ? (rl >> 2) + 4 * (rl & 3) : rl, T - 1);
    auto out_token = [](int g, int r) { return NR == 1 ? g + 4 * r : 4 * g + r; };

    const int row = tile * 16 + rl;

    // (a fused launch issues its ring unconditionally; a wave without steps
    // then reads its tile's first step, never consumed)
    // Buffer resources over the tile's packed steps and its group scales: the
    // ring's loads then take a per-lane constant offset plus a uniform one
    // (scalar arithmetic), where flat addresses cost 64-bit vector adds per
    // load.
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(M.packed) + (size_t)tile * p.n_steps * STEP, 0, p.n_steps * STEP, 0x00020000);
    const int w_voff = lane * (4 * WPL);
    const int w_s0 = FUSE && s_cnt <= 0 ? 0 : s0;           // first step of the part
    __amdgpu_buffer_rsrc_t rs = rw;                          // group mode: [G][16 rows] scales of the tile
    if constexpr (GROUP)
        rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(M.scales) + (size_t)tile * p.G * 16, 0,
                                               p.G * 64, 0x00020000);
    const int s_voff = rl * 4;
    const int8_t* qrow = M.q + (size_t)tok * K;                            // global activations

    uint32_t wv[D][WPL];
    float sg[D][NU];
    i32x4 av[D][NA];

    // Scale units run in order on both sides of the ring, so the group of a
    // unit is tracked with running counters (a part always starts at a group
    // boundary): lu/lg for the loads, cu/cg for the compute.
    const int unit0 = s0 * NU;
    const int g0 = UPG1 ? unit0 : (p.upg_shift >= 0 ? unit0 >> p.upg_shift : unit0 / p.upg);
    int lu = 0, lg = g0;                                     // load side: unit within group, group
    auto load_slot = [&](int u, int j) {
        // Unconditional loads (a dead step past the part re-reads its last
        // step, never consumed): the compiler's wait counting then keeps all
        // D steps in flight.
        const int jj = j < s_cnt ? j : max(s_cnt - 1, 0);
        load_words_stream_buf<WPL>(rw, w_voff, (w_s0 + jj) * STEP, wv[u]);   // each weight byte is read once
        if constexpr (GROUP) {
            #pragma unroll
            for (int v = 0; v < NU; ++v) {
                sg[u][v] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, s_voff, min(lg, p.G - 1) * 64, 0));
                if constexpr (UPG1) {
                    ++lg;
                } else {
                    lu = lu + 1 == p.upg ? 0 : lu + 1;
                    lg = lu == 0 ? lg + 1 : lg;
                }
            }
        }
        if constexpr (!LDSA) {
            #pragma unroll
            for (int b = 0; b < NB; ++b)
                #pragma unroll
                for (int m = 0; m < MPB; ++m) {
                    const int k0 = (s0 + jj) * SK + b * KB + g * (KB / 4) + 16 * m;
                    if (p.q_vec) av[u][b * MPB + m] = *reinterpret_cast<const i32x4*>(qrow + (k0 < K ? k0 : 0));
                    else av[u][b * MPB + m] = load_q16(qrow, k0, K, false);
                }
        }
    };

    // fused: the first round of x is issued ahead of the weight
    // ring, so the quantiser's reduction waits for x alone (the loads are
    // counted in order) and runs while the ring's HBM loads are in flight
    constexpr int FR = FRW;                                  // words (4 k) per thread per round
    const int nword = (K + 3) >> 2;                          // words holding real k
    const int tid = threadIdx.x;
    float4 xv[FR];
    auto load_round = [&](const float* xr, int base) {      // fused launches have k % 4 == 0, x 16-byte aligned
        #pragma unroll
        for (int j = 0; j < FR; ++j)
            xv[j] = reinterpret_cast<const float4*>(xr)[min(base + tid + 256 * j, nword - 1)];
    };
    if constexpr (FUSE) {
        load_round(M.x, 0);
        __builtin_amdgcn_sched_barrier(0);                   // keep these loads ahead of the ring's
    }

    // Stage steps [step0, step0 + nsteps) of every token row into LDS (row t
    // at t * stride): the (token, chunk) space in batches of SB chunks per
    // thread, every load of a batch issued before its stores, so that a
    // thread waits for one L2 round trip per batch, not one per token row.
    // A thread's chunks are NT apart; their (token, chunk) pairs advance
    // incrementally (one division per phase, not one per chunk).
    constexpr int SB = 4;
    constexpr int CB = FMT == FMT_BINARY ? 32 : 16;          // codes per chunk
    auto stage_issue = [&](auto vec_only, auto nb, int step0, int nsteps, int base, int& t, int& cc, i32x4* lo,
                           i32x4* hi, int* tb, int* cb) __attribute__((always_inline)) {
        constexpr bool VEC_ONLY = decltype(vec_only)::value;   // every q row 16-byte aligned, k % 16 == 0
        constexpr int NBAT = decltype(nb)::value;              // chunks per thread in this batch
        const int per_row = nsteps * SK / CB, total = T * per_row;
        const int k0 = step0 * SK;
        const int dt = NT / per_row, dcc = NT - dt * per_row;
        #pragma unroll
        for (int b = 0; b < NBAT; ++b) {
            tb[b] = t; cb[b] = cc;
            cc += dcc; t += dt;
            if (cc >= per_row) { cc -= per_row; ++t; }
            if (base + b * NT < total) {
                const int8_t* qr = M.q + (size_t)tb[b] * K;
                lo[b] = load_q16(qr, k0 + CB * cb[b], K, VEC_ONLY || p.q_vec, VEC_ONLY);
                if constexpr (FMT == FMT_BINARY)
                    hi[b] = load_q16(qr, k0 + CB * cb[b] + 16, K, VEC_ONLY || p.q_vec, VEC_ONLY);
            }
        }
    };
    auto stage_store = [&](auto nb, int nsteps, int base, const i32x4* lo, const i32x4* hi, const int* tb,
                           const int* cb) __attribute__((always_inline)) {
        constexpr int NBAT = decltype(nb)::value;
        const int total = T * (nsteps * SK / CB);
        #pragma unroll
        for (int b = 0; b < NBAT; ++b) {
            if (base + b * NT < total) {
                uint8_t* dst = smem + (size_t)tb[b] * p.stride + CB * cb[b];
                if constexpr (FMT == FMT_BINARY) {
                    // 32-code chunks permuted to the order decode_binary yields
                    const uint32_t X[8] = {(uint32_t)lo[b][0], (uint32_t)lo[b][1], (uint32_t)lo[b][2],
                                           (uint32_t)lo[b][3], (uint32_t)hi[b][0], (uint32_t)hi[b][1],
                                           (uint32_t)hi[b][2], (uint32_t)hi[b][3]};
                    i32x4 a0, a1;
                    perm_binary_a(X, a0, a1);
                    *reinterpret_cast<i32x4*>(dst) = a0;
                    *reinterpret_cast<i32x4*>(dst + 16) = a1;
                } else {
                    *reinterpret_cast<i32x4*>(dst) = lo[b];
                }
            }
        }
    };
    // the batches from chunk base0 (a thread's first chunk is threadIdx.x)
    auto stage_phase = [&](auto vec_only, int step0, int nsteps, int base0) __attribute__((always_inline)) {
        const int per_row = nsteps * SK / CB, total = T * per_row;
        int t = base0 / per_row, cc = base0 - t * per_row;
        for (int base = base0; base < total; base += NT * SB) {
            i32x4 lo[SB], hi[SB];
            int tb[SB], cb[SB];
            stage_issue(vec_only, std::integral_constant<int, SB>{}, step0, nsteps, base, t, cc, lo, hi, tb, cb);
            stage_store(std::integral_constant<int, SB>{}, nsteps, base, lo, hi, tb, cb);
        }
    };
    // A 16-wavefront stage (several tokens): its first two chunks per thread
    // are loaded ahead of the weight ring, so that their wait (counted in
    // order) is for the L2 loads alone and the stage fills while the ring's
    // first HBM loads are in flight.  (Four-wavefront workgroups stage little
    // and are short of registers at that point.)
    constexpr bool EARLY = LDSA && !FUSE && WV == 16;
    constexpr int SBE = 2;
    const int nsteps0 = min(p.ph_steps, p.n_steps);
    i32x4 e_lo[SBE], e_hi[SBE];
    int e_tb[SBE], e_cb[SBE];
    if constexpr (EARLY) {
        const int per_row0 = nsteps0 * SK / CB;
        int t = (int)threadIdx.x / per_row0, cc = (int)threadIdx.x - t * per_row0;
        stage_issue(std::false_type{}, std::integral_constant<int, SBE>{}, 0, nsteps0, threadIdx.x, t, cc, e_lo, e_hi,
                    e_tb, e_cb);
    }

    // ---- ring prologue, the epilogue operands, then the activation stage
    if (FUSE || s_cnt > 0) {
        #pragma unroll
        for (int u = 0; u < D; ++u) load_slot(u, u);
    }
    if constexpr (FUSE) {
        // ... and the quantiser's use of x after them: an empty asm that
        // takes the values (and orders memory) pins that point
        #pragma unroll
        for (int j = 0; j < FR; ++j)
            asm volatile("" : "+v"(xv[j].x), "+v"(xv[j].y), "+v"(xv[j].z), "+v"(xv[j].w) :: "memory");
    }
    float sw = 0.0f;
    if constexpr (!GROUP) sw = M.scales[p.scale_per_row ? min(row, M.n - 1) : 0];
    float sxv[NR];                                           // token scales (loaded after the k-loop)
    const int8_t* lds_a = reinterpret_cast<const int8_t*>(smem) + (size_t)tok * p.stride + g * (KB / 4);

    if constexpr (FUSE) {
        // fp32 x -> int8 codes in the stage (one token).  Thread tid owns the
        // words (4 consecutive k) tid + 256 j and issues their loads in rounds
        // of FR before using any of them, so a round costs one memory round
        // trip; the loads are unconditional at clamped addresses (an element
        // read twice changes neither max |x| nor finiteness).  Pass 1 reduces
        // max |x| (wavefront shuffles, then LDS over the 4 wavefronts); pass 2
        // quantises, from pass 1's registers when the row fits one round,
        // else re-reading the row (L1/L2).  The first round sits outside every
        // loop so that its wait counts the ring's loads as younger (a loop
        // header would merge that away).
        const bool writer = (int)blockIdx.x == p.wg_start[mi];
        const int npad = (p.n_steps * SK) >> 2;              // words of the stage row
        const bool one_round = nword <= 256 * FR;
        if constexpr (PRE != PRE_NONE) {
            // the transform of the (single) load round, in place in xv;
            // words past nword are clamped duplicates and never counted
            const bool first = blockIdx.x == 0;
            float4 yv[FR], gv[FR];
            #pragma unroll
            for (int j = 0; j < FR; ++j) {
                const int idx = min(tid + 256 * j, nword - 1);
                if constexpr (PRE == PRE_NORM) {
                    yv[j] = p.pre_r ? reinterpret_cast<const float4*>(p.pre_r)[idx] : make_float4(0.f, 0.f, 0.f, 0.f);
                    gv[j] = reinterpret_cast<const float4*>(p.pre_g)[idx];
                } else {
                    yv[j] = reinterpret_cast<const float4*>(p.pre_r)[idx];
                }
            }
            if constexpr (PRE == PRE_NORM) {
                float ss = 0.0f;
                #pragma unroll
                for (int j = 0; j < FR; ++j) {
                    if (p.pre_r) {
                        xv[j].x = xv[j].x + yv[j].x; xv[j].y = xv[j].y + yv[j].y;
                        xv[j].z = xv[j].z + yv[j].z; xv[j].w = xv[j].w + yv[j].w;
                    }
                    if (tid + 256 * j < nword)
                        ss += xv[j].x * xv[j].x + xv[j].y * xv[j].y + xv[j].z * xv[j].z + xv[j].w * xv[j].w;
                }
                #pragma unroll
                for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
                if (lane == 0) fz_ss[wave] = ss;
                __syncthreads();
                ss = (fz_ss[0] + fz_ss[1]) + (fz_ss[2] + fz_ss[3]);
                const float rr = 1.0f / sqrtf(ss / (float)K + p.pre_eps);
                #pragma unroll
                for (int j = 0; j < FR; ++j) {
                    const int w = tid + 256 * j;
                    if (first && w < nword) reinterpret_cast<float4*>(p.pre_xo)[w] = xv[j];
                    xv[j].x = xv[j].x * rr * gv[j].x; xv[j].y = xv[j].y * rr * gv[j].y;
                    xv[j].z = xv[j].z * rr * gv[j].z; xv[j].w = xv[j].w * rr * gv[j].w;
                    if (first && p.pre_ho && w < nword) reinterpret_cast<float4*>(p.pre_ho)[w] = xv[j];
                }
            } else {
                #pragma unroll
                for (int j = 0; j < FR; ++j) {
                    const float z[4] = {xv[j].x, xv[j].y, xv[j].z, xv[j].w};
                    const float u[4] = {yv[j].x, yv[j].y, yv[j].z, yv[j].w};
                    float a[4];
                    #pragma unroll
                    for (int e = 0; e < 4; ++e) a[e] = z[e] / (1.0f + expf(-z[e])) * u[e];
                    xv[j] = make_float4(a[0], a[1], a[2], a[3]);
                    const int w = tid + 256 * j;
                    if (first && p.pre_ho && w < nword) reinterpret_cast<float4*>(p.pre_ho)[w] = xv[j];
                }
            }
        }
        float m = 0.0f;
        int bad = 0;
        auto reduce_round = [&]() {
            #pragma unroll
            for (int j = 0; j < FR; ++j) {
                const float4 v = xv[j];
                bad |= !(isfinite(v.x) && isfinite(v.y) && isfinite(v.z) && isfinite(v.w));
                const float a0 = fabsf(v.x), a1 = fabsf(v.y), a2 = fabsf(v.z), a3 = fabsf(v.w);
                m = a0 > m ? a0 : m; m = a1 > m ? a1 : m; m = a2 > m ? a2 : m; m = a3 > m ? a3 : m;
            }
        };
        reduce_round();                                      // round 0: already in flight
        #pragma unroll 1
        for (int base = 256 * FR; base < nword; base += 256 * FR) {
            load_round(M.x, base);
            reduce_round();
        }
        m = wave_max(m);
        bad = wave_or(bad);
        if (lane == 0) { fz_m[wave] = m; fz_bad[wave] = bad; }
        __syncthreads();
        m = fz_m[0];
        bad = fz_bad[0];
        #pragma unroll
        for (int w = 1; w < 4; ++w) {
            m = fz_m[w] > m ? fz_m[w] : m;
            bad |= fz_bad[w];
        }
        float r = 0.0f;
        int flag = 0;
        if (bad) {
            flag = LOWBIT_ACT_NONFINITE;
        } else if (m > 0.0f) {
            r = 127.0f / m;
            if (!isfinite(r)) flag = LOWBIT_ACT_OVERFLOW;
        }
        const float st = flag ? __builtin_nanf("") : m / 127.0f;
        if (writer && threadIdx.x == 0) {
            const_cast<float*>(M.sx)[0] = st;
            if (flag && p.status) atomicOr(p.status, flag);
        }
        int8_t* qo = const_cast<int8_t*>(M.q);
        #pragma unroll 1
        for (int base = 0; base < npad; base += 256 * FR) {
            if (!(one_round && base == 0)) load_round(M.x, base);
            #pragma unroll
            for (int j = 0; j < FR; ++j) {
                const int w = base + tid + 256 * j;
                if (w >= npad) continue;
                const int valid = K - 4 * w;                 // codes of this word that exist
                const uint32_t X = flag || valid <= 0 ? 0u : quant_word(xv[j], r, valid);
                if constexpr (FMT == FMT_BINARY) {
                    // word w of a 32-code chunk holds k = 8b + 4a + e (a = w & 1,
                    // b = (w & 7) >> 1); decode_binary wants it in operand a,
                    // register e, byte b
                    uint8_t* o = smem + 32 * (w >> 3) + 16 * (w & 1) + ((w & 7) >> 1);
                    #pragma unroll
                    for (int e = 0; e < 4; ++e) o[4 * e] = (uint8_t)(X >> (8 * e));
                } else {
                    *reinterpret_cast<uint32_t*>(smem + 4 * w) = X;
                }
                if (writer && valid > 0) {                   // natural-order codes to q (k % 4 == 0)
                    if (p.q_word) {
                        *reinterpret_cast<uint32_t*>(qo + 4 * w) = X;
                    } else {
                        #pragma unroll
                        for (int e = 0; e < 4; ++e) qo[4 * w + e] = (int8_t)(X >> (8 * e));
                    }
                }
            }
        }
        __syncthreads();
        #pragma unroll
        for (int r = 0; r < NR; ++r) sxv[r] = st;
    } else if constexpr (LDSA) {
        if constexpr (EARLY) {
            stage_store(std::integral_constant<int, SBE>{}, nsteps0, threadIdx.x, e_lo, e_hi, e_tb, e_cb);
            stage_phase(std::false_type{}, 0, nsteps0, threadIdx.x + NT * SBE);
        } else {
            stage_phase(std::false_type{}, 0, nsteps0, threadIdx.x);
        }
        __syncthreads();
    }

    i32x4 C = {0, 0, 0, 0};                                  // tensor/row mode: the whole product
    float yp[NR];                                            // group mode: rescaled partial sums
    #pragma unroll
    for (int r = 0; r < NR; ++r) yp[r] = 0.0f;

    const int n_units = (K + SK / NU - 1) / (SK / NU);       // scale units holding real k
    int cu = 0, cg = g0, cunit = unit0;                      // compute side: unit in group, group, unit
    i32x4 Cg = {0, 0, 0, 0};                                 // group partial (groups of several units)

    // LDS phases (16-wavefront workgroups whose whole activation row set
    // would not leave room for two workgroups per CU): the stage holds
    // ph_steps k-steps at a time.  At a phase's first step every wavefront of
    // the workgroup meets at a barrier, the next steps are staged over the
    // old ones, and a second barrier publishes them; the weight ring runs on
    // across the change.  Wavefronts run every step in the same order (one
    // part per tile), so each meets the same barriers.
    int a_off = 0;                                           // A of step s at lds_a + s * SK - a_off
    int ph_next = p.ph_steps;                                // first step of the next phase
    auto next_phase = [&]() __attribute__((always_inline)) {
        __syncthreads();
        stage_phase(std::true_type{}, ph_next, min(p.ph_steps, p.n_steps - ph_next), threadIdx.x);   // phases need q_vec
        __syncthreads();
        a_off = ph_next * SK;
        ph_next += p.ph_steps;
    };

    // MFMAs of block b of slot u into C
    auto block_mfma = [&](int u, int s, int b, i32x4 C, bool fresh) -> i32x4 {
        const i32x4 zero = {0, 0, 0, 0};
        i32x4 A[MPB];
        if constexpr (LDSA) {
            #pragma unroll
            for (int m = 0; m < MPB; ++m) A[m] = *reinterpret_cast<const i32x4*>(lds_a + (s * SK - a_off) + b * KB + 16 * m);
        } else if constexpr (FMT == FMT_BINARY) {
            // binary padding codes decode as +1: activations past K must be zero
            const int k0 = s * SK + b * KB + g * (KB / 4);
            i32x4 lo = av[u][2 * b], hi = av[u][2 * b + 1];
            if (k0 >= K) lo = zero;
            if (k0 + 16 >= K) hi = zero;
            const uint32_t X[8] = {(uint32_t)lo[0], (uint32_t)lo[1], (uint32_t)lo[2], (uint32_t)lo[3],
                                   (uint32_t)hi[0], (uint32_t)hi[1], (uint32_t)hi[2], (uint32_t)hi[3]};
            perm_binary_a(X, A[0], A[1]);
        } else {
            A[0] = av[u][b];                                 // padding codes are 0: any A is fine
        }
        if constexpr (FMT == FMT_TERNARY) {
            C = mfma16(A[0], decode_ternary(wv[u][b]), fresh ? zero : C);
        } else if constexpr (FMT == FMT_INT4) {
            C = mfma16(A[0], decode_int4(wv[u][2 * b], wv[u][2 * b + 1]), fresh ? zero : C);
        } else {
            i32x4 b0, b1;
            decode_binary(wv[u][b], b0, b1);
            C = mfma16(A[0], b0, fresh ? zero : C);
            C = mfma16(A[1], b1, C);
        }
        return C;
    };
    // a group's integer partial is complete: rescale into yp (and record it).
    // Cx holds 2^SHIFT times the partial, and yp is kept 2^SHIFT times too:
    // converting Cx itself gives exactly 2^SHIFT (float)partial, and scaling
    // by a power of two commutes with fp32 rounding, so the products and sums
    // are the unshifted ones times 2^SHIFT, bit for bit (one shift fewer per
    // register per group; the epilogue scales by 2^-SHIFT).
    auto close_group = [&](const i32x4& Cx, float sc, int gi) {
        #pragma unroll
        for (int r = 0; r < NR; ++r) {
            yp[r] = yp[r] + sc * (float)Cx[r];
            if constexpr (ACC) {
                const int t = out_token(g, r);
                if (M.acc && live && t < T && row < M.n) M.acc[((size_t)t * M.n + row) * p.G + gi] = Cx[r] >> SHIFT;
            }
        }
    };

    auto compute_slot = [&](int u, int j) {
        if (j >= s_cnt) return;                              // dead step (uniform)
        const int s = s0 + j;
        if constexpr (!GROUP) {
            #pragma unroll
            for (int b = 0; b < NB; ++b) C = block_mfma(u, s, b, C, false);
        } else {
            #pragma unroll
            for (int v = 0; v < NU; ++v) {
                i32x4 Cu = {0, 0, 0, 0};                     // this unit's partial: a fresh chain
                #pragma unroll
                for (int bb = 0; bb < BPU; ++bb) Cu = block_mfma(u, s, v * BPU + bb, Cu, bb == 0);
                const bool real = cunit < n_units;           // (uniform) units past k hold only padding
                if constexpr (UPG1) {
                    // padding units add exact zeros (and never record a partial)
                    if constexpr (ACC) { if (real) close_group(Cu, sg[u][v], cg); }
                    else close_group(Cu, sg[u][v], cg);
                    ++cg;
                } else {
                    #pragma unroll
                    for (int r = 0; r < NR; ++r) Cg[r] += Cu[r];
                    const bool last = cu + 1 == p.upg || cunit + 1 == n_units;
                    if (real && last) {                      // uniform
                        close_group(Cg, sg[u][v], cg);
                        #pragma unroll
                        for (int r = 0; r < NR; ++r) Cg[r] = 0;
                    }
                    cu = cu + 1 == p.upg ? 0 : cu + 1;
                    cg = cu == 0 ? cg + 1 : cg;
                }
                ++cunit;
            }
        }
    };

    // steady state: consume a step, refill its slot D steps ahead; then the
    // last D steps without refills
    int j = 0;
    for (; j + D < s_loop; j += D) {
        if constexpr (LDSA && !FUSE) {
            if (j == ph_next) next_phase();                  // (uniform; phases are whole rounds of D steps)
        }
        #pragma unroll
        for (int u = 0; u < D; ++u) {
            compute_slot(u, j + u);
            load_slot(u, j + u + D);
        }
    }
    if (s_loop > 0) {
        if constexpr (LDSA && !FUSE) {
            if (j == ph_next) next_phase();
        }
        #pragma unroll
        for (int u = 0; u < D; ++u) compute_slot(u, j + u);
    }
    if constexpr (LDSA && !FUSE) {
        // a wave without a tile still takes its part in every phase change
        if (s_cnt <= 0)
            while (ph_next < p.n_steps) next_phase();
    }

    // ---- combine k-split partials (fixed order), rescale, store
    if constexpr (!FUSE) {
        #pragma unroll
        for (int r = 0; r < NR; ++r) sxv[r] = M.sx[min(out_token(g, r), T - 1)];
    }
    int32_t ai[NR];
    #pragma unroll
    for (int r = 0; r < NR; ++r) ai[r] = C[r] >> SHIFT;
    if (p.ksplit > 1) {
        int32_t* red = reinterpret_cast<int32_t*>(smem + p.lds_a_bytes);   // [WV waves][NR][64], after A
        #pragma unroll
        for (int r = 0; r < NR; ++r)
            red[(wave * NR + r) * 64 + lane] = GROUP ? __float_as_int(yp[r]) : ai[r];
        __syncthreads();
        if (part == 0) {
            for (int q = 1; q < p.ksplit; ++q) {
                #pragma unroll
                for (int r = 0; r < NR; ++r) {
                    const int32_t o = red[((wave + q) * NR + r) * 64 + lane];
                    if constexpr (GROUP) yp[r] = yp[r] + __int_as_float(o);
                    else ai[r] += o;
                }
            }
        }
    }
    // Several tokens: y with the non-temporal hint.  The output stream is
    // small beside the weights, but its writes reach HBM in the middle of the
    // read stream and cost far more than their bytes (t = 4, the 4B-class
    // pass: 17 MB of y took 24 us of a 142 us launch; non-temporal stores
    // saved a third of that).  One token keeps y cached for its consumer.
    if (part == 0 && live && row < M.n) {
        const __amdgpu_buffer_rsrc_t ry =
            __builtin_amdgcn_make_buffer_rsrc(M.y, 0, (int)min((int64_t)T * M.n * 4, (int64_t)INT_MAX), 0x00020000);
        #pragma unroll
        for (int r = 0; r < NR; ++r) {
            const int t = out_token(g, r);
            if (t < T) {
                float v;
                if constexpr (GROUP) v = sxv[r] * (yp[r] * (1.0f / (float)(1 << SHIFT)));
                else v = (float)ai[r] * (sxv[r] * sw);
                const int off = (t * M.n + row) * 4;
                if (T > 1) __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), ry, off, 0, 2);   // nt
                else __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), ry, off, 0, 0);
                if constexpr (ACC && !GROUP) {
                    if (M.acc) M.acc[(size_t)t * M.n + row] = ai[r];
                }
            }
        }
    }
}

template <int FMT, int WPL, int NR, int SPS, bool UPG1>
void gemv_launch_lds(const GemvParams& p, const GemvCfg& c, hipStream_t st) {
    const dim3 grid((unsigned)c.grid), block(64 * c.waves);
    if (c.lds_a) {
        if constexpr (NR == 1) {   // fused launches have one token
            if (c.fuse) {
                if (c.pre == PRE_NORM)
                    gemv_kernel<FMT, WPL, 1, SPS, UPG1, true, false, true, 4, PRE_NORM><<<grid, block, c.lds_bytes, st>>>(p);
                else if (c.pre == PRE_SWIGLU)
                    gemv_kernel<FMT, WPL, 1, SPS, UPG1, true, false, true, 4, PRE_SWIGLU><<<grid, block, c.lds_bytes, st>>>(p);
                else if (p.K > 256 * 3 * 4 && p.K <= 256 * 10 * 4)
                    // a row of 3073 .. 10240 elements in one load round (86
                    // VGPRs; these one-token launches are latency-bound, not
                    // occupancy-bound): the max and the codes then wait for one
                    // memory round trip, not one per 3072 elements in each of
                    // the two passes (k = 9728: prologue 6.0 -> 4.8 us)
                    gemv_kernel<FMT, WPL, 1, SPS, UPG1, true, false, true, 4, PRE_NONE, 10><<<grid, block, c.lds_bytes, st>>>(p);
                else
                    gemv_kernel<FMT, WPL, 1, SPS, UPG1, true, false, true, 4, PRE_NONE><<<grid, block, c.lds_bytes, st>>>(p);
                return;
            }
        }
        if (c.waves == 16) {       // a large stage shared by 16 wavefronts (several tokens)
            if (c.acc) gemv_kernel<FMT, WPL, NR, SPS, UPG1, true, true, false, 16, PRE_NONE><<<grid, block, c.lds_bytes, st>>>(p);
            else gemv_kernel<FMT, WPL, NR, SPS, UPG1, true, false, false, 16, PRE_NONE><<<grid, block, c.lds_bytes, st>>>(p);
            return;
        }
        if (c.acc) gemv_kernel<FMT, WPL, NR, SPS, UPG1, true, true, false, 4, PRE_NONE><<<grid, block, c.lds_bytes, st>>>(p);
        else gemv_kernel<FMT, WPL, NR, SPS, UPG1, true, false, false, 4, PRE_NONE><<<grid, block, c.lds_bytes, st>>>(p);
    } else {
        // activations from L2: the fallback for stages too large for LDS, always 4 token registers
        if (c.acc) gemv_kernel<FMT, WPL, 4, SPS, UPG1, false, true, false, 4, PRE_NONE><<<grid, block, c.lds_bytes, st>>>(p);
        else gemv_kernel<FMT, WPL, 4, SPS, UPG1, false, false, false, 4, PRE_NONE><<<grid, block, c.lds_bytes, st>>>(p);
    }
}

template <int FMT, int WPL>
void gemv_launch_wpl(const GemvParams& p, const GemvCfg& c, hipStream_t st) {
    constexpr int NB = GemvShape<FMT, WPL>::kNB;
    auto by_nr = [&](auto sps_tag) {
        constexpr int SPS = decltype(sps_tag)::value;
        if constexpr (SPS == 0) {
            if (c.nr == 1 && c.lds_a) gemv_launch_lds<FMT, WPL, 1, 0, false>(p, c, st);
            else gemv_launch_lds<FMT, WPL, 4, 0, false>(p, c, st);
        } else if (p.upg == 1) {
            if (c.nr == 1 && c.lds_a) gemv_launch_lds<FMT, WPL, 1, SPS, true>(p, c, st);
            else gemv_launch_lds<FMT, WPL, 4, SPS, true>(p, c, st);
        } else {
            if (c.nr == 1 && c.lds_a) gemv_launch_lds<FMT, WPL, 1, SPS, false>(p, c, st);
            else gemv_launch_lds<FMT, WPL, 4, SPS, false>(p, c, st);
        }
    };
    switch (c.sps) {
        case 0: by_nr(std::integral_constant<int, 0>{}); break;
        case 1: by_nr(std::integral_constant<int, 1>{}); break;
        case 2: if constexpr (NB >= 2) by_nr(std::integral_constant<int, 2>{}); break;
        default: if constexpr (NB >= 4) by_nr(std::integral_constant<int, 4>{}); break;
    }
}

}  // namespace lowbit
