// gemv.hip - host-side dispatch of the decode GEMV (the kernel itself is in
// gemv_kernel.hpp, instantiated per format in gemv_{ternary,int4,binary}.hip).
#include <algorithm>
#include <climits>

#include "device_common.hpp"
#include "gemv.hpp"
#include "kernels.hpp"

namespace lowbit {

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

namespace {

int log2_exact(int v) {   // log2 of a power of two, else -1
    if (v <= 0 || (v & (v - 1)) != 0) return -1;
    int l = 0;
    while ((1 << l) < v) ++l;
    return l;
}

}  // namespace

// One launch over `count` matrices that share fmt, scale mode, group, k and
// the token count t <= 16.  Workgroups run over the matrices in order.
hipError_t launch_gemv_group(const LinearArgs* mats, int count, hipStream_t stream) {
    const LinearArgs& a = mats[0];
    const bool group = a.scale == LOWBIT_SCALE_GROUP;
    const int SK = a.step_k, n_steps = a.n_steps;
    const int nb = a.fmt == FMT_INT4 ? a.wpl / 2 : a.wpl;   // MFMA blocks per k-step

    GemvParams gp{};
    GemvCfg cfg{};
    gp.n_mats = count;
    gp.K = a.k;
    gp.T = a.t;
    gp.n_steps = n_steps;
    gp.G = group ? a.n_groups : 1;
    gp.scale_per_row = a.scale == LOWBIT_SCALE_ROW;
    gp.upg = 1;
    gp.upg_shift = 0;
    cfg.wpl = a.wpl;
    cfg.sps = 0;
    if (group) {
        // scale units: the fewest per k-step that each lie inside one group
        int sps = nb;
        for (int s = 1; s <= nb; s *= 2)
            if (a.group % (SK / s) == 0) { sps = s; break; }
        cfg.sps = sps;
        gp.upg = a.group / (SK / sps);
        gp.upg_shift = log2_exact(gp.upg);
    }
    // LDS row stride: whole k-steps plus 32 bytes, which puts the 16 token
    // rows' 16-byte operand reads (one row per lane, lane groups 16 bytes
    // apart) on distinct banks; a 16-byte pad measured 2-way conflicts on
    // every read
    constexpr int kPad = 32;
    gp.stride = n_steps * SK + kPad;
    gp.ph_steps = n_steps;
    int64_t stage = (int64_t)a.t * gp.stride;                // LDS bytes of the staged activations
    const bool small_stage = stage <= kGemvLdsA;
    cfg.nr = a.t <= 4 ? 1 : 4;                                // live token registers per lane

    // The quantiser runs in the product kernel's prologue for one token (every
    // workgroup redoes the row; for a single token that is cheaper than a
    // launch), with the LDS stage and whole 16-byte x words (k % 4 == 0, every
    // x 16-byte aligned).  Otherwise the quantiser kernel produces the codes
    // first, into the given q / sx (one launch for all the matrices).
    const bool fused_in = a.x != nullptr;
    bool x_vec = a.k % 4 == 0;
    for (int i = 0; fused_in && i < count; ++i) x_vec = x_vec && (uintptr_t)mats[i].x % 16 == 0;
    cfg.fuse = fused_in && small_stage && x_vec && a.t == 1;
    // an input transform needs the fused prologue with one load round (k <= 3072),
    // 16-byte aligned operands, and one x shared by every matrix of the launch
    cfg.pre = a.pre;
    if (a.pre != 0) {
        bool ok = cfg.fuse && a.k <= 3 * 256 * 4 && (uintptr_t)a.pre_r % 16 == 0 && (uintptr_t)a.pre_g % 16 == 0 &&
                  (uintptr_t)a.pre_xo % 16 == 0 && (uintptr_t)a.pre_ho % 16 == 0 &&
                  (a.pre == 1 ? (a.pre_g != nullptr && a.pre_xo != nullptr) : a.pre_r != nullptr);
        for (int i = 1; i < count; ++i) ok = ok && mats[i].x == a.x;
        if (!ok) return hipErrorInvalidValue;
    }
    gp.pre_r = a.pre_r; gp.pre_g = a.pre_g; gp.pre_eps = a.pre_eps; gp.pre_xo = a.pre_xo; gp.pre_ho = a.pre_ho;
    if (fused_in && !cfg.fuse) {                             // every matrix's input in one launch
        const float* xs[kGemvMaxMats];
        int8_t* qs[kGemvMaxMats];
        float* sxs[kGemvMaxMats];
        for (int i = 0; i < count; ++i) {
            xs[i] = mats[i].x;
            qs[i] = const_cast<int8_t*>(mats[i].q);
            sxs[i] = const_cast<float*>(mats[i].sx);
        }
        hipError_t e = launch_act_quant_group(xs, qs, sxs, count, a.t, a.k, a.status, stream);
        if (e != hipSuccess) return e;
    }
    gp.status = cfg.fuse ? a.status : nullptr;
    bool q_word = a.k % 4 == 0;

    bool q_vec = a.k % 16 == 0;
    int tiles = 0;
    bool any_acc = false;
    for (int i = 0; i < count; ++i) {
        const LinearArgs& b = mats[i];
        gp.m[i].packed = b.packed; gp.m[i].scales = b.scales; gp.m[i].q = b.q; gp.m[i].sx = b.sx;
        gp.m[i].y = b.y; gp.m[i].acc = b.acc;
        gp.m[i].x = cfg.fuse ? b.x : nullptr;
        q_word = q_word && (uintptr_t)b.q % 4 == 0;
        gp.m[i].n = b.n;
        gp.m[i].n_tiles = (b.n + 15) / 16;
        tiles += gp.m[i].n_tiles;
        q_vec = q_vec && ((uintptr_t)b.q % 16 == 0);
        any_acc = any_acc || b.acc != nullptr;
    }
    gp.q_vec = q_vec;
    gp.q_word = q_word;
    cfg.acc = any_acc && !cfg.fuse;

    // k-split: enough wavefronts to fill the chip; in group mode every part
    // holds whole groups
    const int cus = device_cu_count();
    int spg = 1;                                             // k-steps per group (0: groups straddle steps)
    if (group) spg = a.group % SK == 0 ? a.group / SK : (SK % a.group == 0 ? 1 : 0);
    int ksplit = 1;
    if (spg > 0) {
        if (tiles < 4 * cus && n_steps >= 4) ksplit = 2;
        if (tiles < 2 * cus && n_steps >= 8) ksplit = 4;
        // several tokens: more parts while the launch holds fewer wavefronts
        // than two rounds of the CUs' resident ones (32 each), unless the
        // stage is one that needs LDS phases (those take whole k-ranges).
        // (With one token each part's workgroup restages the row for one
        // tile, and a fused launch would quantise it once more per part.)
        const bool phased_stage = stage + (int64_t)16 * 4 * 64 * 4 > kGemvLdsHalf;
        while (a.t > 1 && !cfg.fuse && !phased_stage && ksplit < 4 && (int64_t)tiles * ksplit < 2LL * cus * 32 &&
               n_steps >= 4 * ksplit)
            ksplit *= 2;
    }
    int part_len = n_steps;
    for (; ksplit > 1; ksplit /= 2) {
        part_len = (n_steps + ksplit - 1) / ksplit;
        part_len = (part_len + spg - 1) / spg * spg;
        if ((ksplit - 1) * part_len < n_steps) break;       // every part has a step
    }
    if (ksplit == 1) part_len = n_steps;
    gp.ksplit = ksplit;
    gp.ksplit_log = ksplit == 4 ? 2 : (ksplit == 2 ? 1 : 0);
    gp.part_len = part_len;

    // Where the activations live.  Several tokens make the LDS stage large
    // (t * k bytes): above kGemvLdsWide four-wavefront workgroups would leave
    // the CU short of wavefronts streaming weights, so 16-wavefront workgroups
    // share one stage.  Two of them fit a CU while the stage takes at most
    // half the LDS; a larger one is staged in phases of k-steps that do
    // (without a k-split; with one, the whole stage may take the whole LDS).
    // Otherwise the activations ride in the register ring from L2.
    const int64_t red16 = ksplit > 1 ? (int64_t)16 * cfg.nr * 64 * 4 : 0;
    cfg.waves = 4;
    cfg.lds_a = small_stage;
    if (!cfg.fuse && a.t > 1 && stage > kGemvLdsWide) {
        if (stage + red16 <= kGemvLdsHalf) {
            cfg.lds_a = true;
            cfg.waves = 16;
        } else if (ksplit == 1 && q_vec) {
            // phases of whole ring rounds (kGemvD steps), as few as fit
            int ph = n_steps;
            for (int parts = 2; (int64_t)a.t * (ph * SK + kPad) > kGemvLdsHalf; ++parts)
                ph = ((n_steps + parts - 1) / parts + kGemvD - 1) / kGemvD * kGemvD;
            gp.ph_steps = ph;
            gp.stride = ph * SK + kPad;
            stage = (int64_t)a.t * gp.stride;
            cfg.lds_a = true;
            cfg.waves = 16;
        } else if (stage + red16 <= kGemvLdsMax) {
            cfg.lds_a = true;
            cfg.waves = 16;
        }
    }
    if (!cfg.lds_a) cfg.nr = 4;                              // the L2 fallback keeps four token registers
    gp.lds_a_bytes = cfg.lds_a ? (int)stage : 0;
    gp.tiles_per_wg = cfg.waves / ksplit;

    int wgs = 0;
    for (int i = 0; i < count; ++i) {
        gp.wg_start[i] = wgs;
        wgs += (gp.m[i].n_tiles + gp.tiles_per_wg - 1) / gp.tiles_per_wg;
    }
    for (int i = count; i <= kGemvMaxMats; ++i) gp.wg_start[i] = 0x7fffffff;   // never reached
    cfg.grid = wgs;
    cfg.lds_bytes = (size_t)gp.lds_a_bytes + (ksplit > 1 ? (size_t)cfg.waves * cfg.nr * 64 * 4 : 0);

    switch (a.fmt) {
        case FMT_TERNARY: return gemv_launch_ternary(gp, cfg, stream);
        case FMT_INT4: return gemv_launch_int4(gp, cfg, stream);
        default: return gemv_launch_binary(gp, cfg, stream);
    }
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
        c.x = a.x ? a.x + (size_t)t0 * a.k : nullptr;
        hipError_t e = launch_gemv_group(&c, 1, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace lowbit
