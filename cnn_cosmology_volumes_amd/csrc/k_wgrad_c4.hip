// Backward-weight of the 3^3 stride-1 pad-1 convolution for the 4-channel
// first layer on bf16 MFMA (the separate backward-weight operator of
// CosmoFlow, Sec. III-C): from the conv-output gradient (wgrad_c4_kernel),
// or with the pool backward fused into the staging (wgrad_c4_ws_kernel).
#include "cf_internal.h"
#include "wgrad_common.h"

#include <type_traits>

namespace cf {

namespace {

// --------------------------------------------------------- Cin == 4 layer
// dW[tap][ci][co] for 4 input channels and 32 output channels.  Same
// channel-major LDS tiles as above; the N dimension packs 4 (kd,kh) pairs x
// 4 input channels per 16-column fragment (3 fragments cover the 9 pairs),
// and kw is applied by the register shift, so one X read serves 3 taps.
// Every wave accumulates the whole 32 x 108 result over its own k-steps of
// each box; the waves are summed through LDS at the end in a fixed order.
constexpr int C4_VB = C4_TD * C4_TH * C4_TW;               // 256 voxels per box
constexpr int C4_NOCT = C4_VB / 8;                         // 32 octets
constexpr int C4_HH = C4_TH + 2;
constexpr int C4_NR = (C4_TD + 2) * C4_HH;                 // 36 halo rows
// X tile [ci][halo row][w]: 64-byte rows and a 2336-byte channel plane.  The
// operand read pairs 4 channels with 4 (kd,kh) rows per 16 lanes; of the
// plane/row pitches that keep 16-byte alignment, this pair gave the fewest
// LDS bank conflicts for that pattern when measured on gfx950 (about 7 clk
// per 16-byte wave read against 12 with 48-byte rows and 1760-byte planes).
constexpr int C4_XW = 32;
constexpr int C4_XPL = C4_NR * C4_XW + 16;                 // per-channel plane: 2336 B
constexpr int C4_DROW = C4_VB + 16;                        // dYT row: 544 B (odd multiple of 32)
constexpr int C4_NT = 256;
constexpr int C4_NDB = C4_NOCT * 4;                        // dY blocks: 32 octets x 4 groups of 8 co
constexpr int C4_NXB = C4_NR * 3;                          // X blocks: rows x {0-7, 8-15, 16-17}
constexpr int C4_NACC = 2 * 3 * 3;                         // co frags x pair frags x kw
constexpr int C4_NPV = (C4_TD / 2) * (C4_TH / 2) * (C4_TW / 2);   // 32 pooled voxels per box

template <int CO>
__global__ __launch_bounds__(C4_NT, 2)
void wgrad_c4_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ dY, float* __restrict__ part, int N,
                     int D, int H, int W, int bD, int bH, int bW, int64_t nbox, int boxes_per_split)
{
    // CO output channels: 32, or 16, where the dY staging tasks of channel
    // groups 4..7 are empty and one output-channel fragment is live
    static_assert(CO == 32 || CO == 16, "output channels");
    constexpr int NCF = CO / 16;                           // output-channel fragments
    __shared__ __attribute__((aligned(16))) uint16_t xt[2][4 * C4_XPL];
    __shared__ __attribute__((aligned(16))) uint16_t dt[2][32 * C4_DROW];
    __shared__ __attribute__((aligned(16))) float red[64 * C4_NACC * 4];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const int split = blockIdx.x;
    const int64_t plane = (int64_t)H * W;

    // Staging.  dY: 256 tasks of 8 voxels (one w-octet) x 4 channels, one
    // per thread, so every lane of every wave shares the dY work and no wave
    // diverges on it.  X: 108 tasks (halo row x {w 0-7, 8-15, 16-17}) on
    // threads 128-235.
    static_assert(C4_NOCT * 8 == C4_NT && C4_NXB <= 128, "task layout");
    const int oct = tid % C4_NOCT, cg = tid / C4_NOCT;       // dY: octet, 4-channel group
    const int xtask = tid - 128;
    const bool is_x = xtask >= 0 && xtask < C4_NXB;
    const int row = xtask / 3, slot = xtask % 3;
    const int nvl = slot == 2 ? 2 : 8;
    const int td_o = oct / (C4_TH * 2), th_o = (oct / 2) % C4_TH, w0_o = (oct & 1) * 8;

    // Staging registers, two sets (the box loop is unrolled by two, so each
    // box's loads are issued two compute phases before they are stored):
    // ud: dY 8 voxels x 4 co; ux: X 8 voxels x 4 ci.
    //
    // Every wave issues the same buffer loads for every box, whatever its
    // role and wherever the box lies: a lane with nothing to fetch (no role,
    // a voxel outside the volume, a box past the end of the split) gets an
    // offset beyond the resource and reads zeros without a memory access.
    // With no load under a branch, the number of loads in flight is the same
    // on every path, so the compiler waits only for the set being stored and
    // leaves the other set in flight (a conditional load makes it wait for
    // all of them).  Offsets are 32-bit, relative to the box's first plane.
    uint2 ud_[2][8];
    uint2 ux_[2][8];
    constexpr uint32_t OOB = 0x80000000u;
    // offset or OOB, held in a register so the choice stays a select (the
    // compiler would otherwise turn it into a branch around the load)
    auto pick = [](bool ok, uint32_t off) {
        uint32_t r = ok ? off : OOB;
        asm volatile("" : "+v"(r));
        return r;
    };
    const int hd_x = row / C4_HH, hh_x = row % C4_HH;

    auto load_box = [&](const BoxPos& bp, bool valid, auto set) {
        constexpr int S = decltype(set)::value;
        uint2 (&ud)[8] = ud_[S];
        uint2 (&ux)[8] = ux_[S];
        const uint32_t lim = valid ? OOB : 0u;
        const int gd0 = bp.bd * C4_TD;
        {
        const auto rd = buf_rsrc(dY + ((int64_t)bp.n * D + gd0) * plane * CO, lim);
        const int gh = bp.bh * C4_TH + th_o, gw0 = bp.bw * C4_TW + w0_o;
        const bool rok = (gd0 + td_o < D) & (gh < H) & (cg < CO / 4);
        const uint32_t rbase = ((uint32_t)td_o * (uint32_t)H + (uint32_t)gh) * (uint32_t)W + (uint32_t)gw0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t off = pick(rok & (gw0 + j < W), (rbase + j) * (CO * 2) + cg * 8);
            ud[j] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rd, off, 0, 0));
        }
        }
        // X halo planes gd0-1 .. gd0+4, addressed from the first one inside the volume
        const int xd0 = gd0 > 0 ? gd0 - 1 : 0;
        const auto rx = buf_rsrc(X + ((int64_t)bp.n * D + xd0) * plane * 4, lim);
        const int gd = gd0 + hd_x - 1, gh = bp.bh * C4_TH + hh_x - 1;
        const bool rok = is_x & ((unsigned)gd < (unsigned)D) & ((unsigned)gh < (unsigned)H);
        const int gwb = bp.bw * C4_TW + 8 * slot - 1;
        const uint32_t rbase = ((uint32_t)(gd - xd0) * (uint32_t)H + (uint32_t)gh) * (uint32_t)W + (uint32_t)gwb;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t off = pick(rok & (j < nvl) & ((unsigned)(gwb + j) < (unsigned)W), (rbase + j) * 8u);
            ux[j] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rx, off, 0, 0));
        }
    };

    // 8 voxels x 4 channels (uint2 per voxel) -> 4 channel rows of 8 voxels
    auto transpose8x4 = [](const uint2 (&v)[8], uint4 (&t)[4]) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
            uint32_t d[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t wl = (c >> 1) ? v[2 * k].y : v[2 * k].x;
                const uint32_t wh = (c >> 1) ? v[2 * k + 1].y : v[2 * k + 1].x;
                d[k] = __builtin_amdgcn_perm(wh, wl, sel);
            }
            t[c] = make_uint4(d[0], d[1], d[2], d[3]);
        }
    };

    auto store_box = [&](int buf, auto set) {
        constexpr int S = decltype(set)::value;
        uint2 (&ud)[8] = ud_[S];
        uint2 (&ux)[8] = ux_[S];
        // Every lane takes delivery of the whole set here, whatever its role,
        // so the loads are complete on every path before their registers are
        // reused (a use only under a role branch leaves them pending on the
        // other paths, and the next write to those registers waits for all
        // loads in flight).
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            asm volatile("" ::"v"(ud[j].x), "v"(ud[j].y));
            asm volatile("" ::"v"(ux[j].x), "v"(ux[j].y));
        }
        {
            uint4 t[4];
            transpose8x4(ud, t);
            // (CO = 16: groups 4..7 loaded zeros and fill rows 16..31, unread)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                *reinterpret_cast<uint4*>(&dt[buf][(cg * 4 + c) * C4_DROW + oct * 8]) = t[c];
        }
        if (is_x) {
            uint4 tx[4];
            transpose8x4(ux, tx);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                uint16_t* dst = &xt[buf][c * C4_XPL + row * C4_XW + slot * 8];
                if (slot < 2) *reinterpret_cast<uint4*>(dst) = tx[c];
                else *reinterpret_cast<uint32_t*>(dst) = tx[c].x;
            }
        }
    };

    f32x4 acc[NCF][3][3];          // [co frag][pair frag][kw]
#pragma unroll
    for (int i = 0; i < NCF; ++i)
#pragma unroll
        for (int f = 0; f < 3; ++f)
#pragma unroll
            for (int kw = 0; kw < 3; ++kw) acc[i][f][kw] = f32x4{0.f, 0.f, 0.f, 0.f};

    // (kd,kh) pair of this lane's column in each pair fragment (pairs >= 9 read pair 0, result discarded)
    int pkd[3], pkh[3];
#pragma unroll
    for (int f = 0; f < 3; ++f) {
        const int pr = 4 * f + (l16 >> 2);
        pkd[f] = pr < 9 ? pr / 3 : 0;
        pkh[f] = pr < 9 ? pr % 3 : 0;
    }
    const int ci = l16 & 3;

    const int64_t b_begin = (int64_t)split * boxes_per_split;
    const int64_t b_end = min(b_begin + boxes_per_split, nbox);
    using Set0 = std::integral_constant<int, 0>;
    using Set1 = std::integral_constant<int, 1>;
    auto compute_box = [&](int buf) {
        const uint16_t* xb = xt[buf];
        const uint16_t* db = dt[buf];
#pragma unroll
        for (int ss = 0; ss < 2; ++ss) {
            const int s = wave + 4 * ss;                       // k-step of this wave
            const int o = 4 * s + lg;                          // octet of this lane group
            const int td = o / (C4_TH * 2), th = (o / 2) % C4_TH, w0 = (o & 1) * 8;
            bf16x8 a[NCF];
#pragma unroll
            for (int i = 0; i < NCF; ++i)
                a[i] = *reinterpret_cast<const bf16x8*>(db + (16 * i + l16) * C4_DROW + o * 8);
#pragma unroll
            for (int f = 0; f < 3; ++f) {
                const int r = (td + pkd[f]) * C4_HH + th + pkh[f];
                const uint16_t* xp = xb + ci * C4_XPL + r * C4_XW + w0;
                uint4 q = *reinterpret_cast<const uint4*>(xp);
                uint32_t e = reinterpret_cast<const uint4*>(xp)[1].x;
                // opaque to the optimizer: it would otherwise re-read the kw = 2
                // operand (bytes 4..19, unaligned) from LDS as two more reads
                asm volatile("" : "+v"(q.x), "+v"(q.y), "+v"(q.z), "+v"(q.w), "+v"(e));
                const uint4 s1 = make_uint4(__builtin_amdgcn_alignbit(q.y, q.x, 16), __builtin_amdgcn_alignbit(q.z, q.y, 16),
                                            __builtin_amdgcn_alignbit(q.w, q.z, 16), __builtin_amdgcn_alignbit(e, q.w, 16));
                const bf16x8 b0 = __builtin_bit_cast(bf16x8, q);
                const bf16x8 b1 = __builtin_bit_cast(bf16x8, s1);
                const bf16x8 b2 = __builtin_bit_cast(bf16x8, make_uint4(q.y, q.z, q.w, e));
#pragma unroll
                for (int i = 0; i < NCF; ++i) {
                    acc[i][f][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b0, acc[i][f][0], 0, 0, 0);
                    acc[i][f][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b1, acc[i][f][1], 0, 0, 0);
                    acc[i][f][2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b2, acc[i][f][2], 0, 0, 0);
                }
            }
        }
    };
    // The loop handles two boxes per iteration and leaves only at its end:
    // an exit between the halves would be a path on which the set loaded
    // for the next box is never consumed, and the compiler would then drain
    // every load at the top of each iteration.  With an odd number of boxes
    // the last half computes a box past the end, which was loaded as zeros
    // and adds exactly zero.
    BoxPos bp = box_uniform(box_decode(b_begin, bD, bH, bW));
    load_box(bp, true, Set0{});
    store_box(0, Set0{});
    lds_barrier();
    bp = box_uniform(box_next(bp, bD, bH, bW));
    load_box(bp, b_begin + 1 < b_end, Set1{});
    int buf = 0;
    for (int64_t box = b_begin; box < b_end; box += 2) {
        // box is in LDS buffer buf, box + 1 in register set 1; set 0 is free
        bp = box_uniform(box_next(bp, bD, bH, bW));
        load_box(bp, box + 2 < b_end, Set0{});
        compute_box(buf);
        store_box(buf ^ 1, Set1{});
        lds_barrier();
        buf ^= 1;
        // box + 1 is in LDS, box + 2 in register set 0; set 1 is free
        bp = box_uniform(box_next(bp, bD, bH, bW));
        load_box(bp, box + 3 < b_end, Set1{});
        compute_box(buf);
        store_box(buf ^ 1, Set0{});
        lds_barrier();
        buf ^= 1;
    }

    // Sum the four waves' accumulators in the order ((w0 + w3) + w2) + w1.
    for (int w = 3; w >= 1; --w) {
        __syncthreads();
        if (wave == w) {
#pragma unroll
            for (int i = 0; i < NCF; ++i)
#pragma unroll
                for (int f = 0; f < 3; ++f)
#pragma unroll
                    for (int kw = 0; kw < 3; ++kw)
                        *reinterpret_cast<f32x4*>(&red[(((i * 3 + f) * 3 + kw) * 64 + lane) * 4]) = acc[i][f][kw];
        }
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int i = 0; i < NCF; ++i)
#pragma unroll
                for (int f = 0; f < 3; ++f)
#pragma unroll
                    for (int kw = 0; kw < 3; ++kw)
                        acc[i][f][kw] += *reinterpret_cast<const f32x4*>(&red[(((i * 3 + f) * 3 + kw) * 64 + lane) * 4]);
        }
    }
    if (wave == 0) {
        float* out = part + (int64_t)split * (27 * 4 * CO);
#pragma unroll
        for (int f = 0; f < 3; ++f) {
            const int pr = 4 * f + (l16 >> 2);
            if (pr >= 9) continue;
#pragma unroll
            for (int kw = 0; kw < 3; ++kw) {
                const int t = pr * 3 + kw;
#pragma unroll
                for (int i = 0; i < NCF; ++i) {
                    const int co = 16 * i + 4 * lg;
                    const f32x4 r = acc[i][f][kw];
                    *reinterpret_cast<float4*>(out + (t * 4 + ci) * CO + co) = make_float4(r[0], r[1], r[2], r[3]);
                }
            }
        }
    }
}

// Wave-specialized form of the fused kernel (32 output channels).  Waves 0-3
// compute exactly as wgrad_c4_kernel<true, 32> does; waves 4-7 hold no
// accumulators and only stage, one box ahead: while the compute waves walk
// box k, they load box k + 1's X halo and box k + 2's pooled gradient,
// pooled values and indices, rebuild box k + 1's dY from the gated pooled
// gradient and indices staged one phase earlier, then store the X halo and
// the new pooled tiles.  The pooled tiles are double-buffered like the
// operand tiles, so a phase needs one workgroup barrier, for all eight waves.
constexpr int C4W_NT = 512, C4W_NCT = 256;                 // threads; compute threads (waves 0-3)

__global__ __launch_bounds__(C4W_NT, 4)
void wgrad_c4_ws_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ dP,
                        const uint16_t* __restrict__ Pv, const uint8_t* __restrict__ pidx, float slope,
                        float* __restrict__ part, int N, int D, int H, int W, int bD, int bH, int bW, int64_t nbox,
                        int boxes_per_split)
{
    constexpr int CO = 32, NCF = 2;
    constexpr int GT_S = C4_NPV + 2;
    __shared__ __attribute__((aligned(16))) uint16_t xt[2][4 * C4_XPL];
    __shared__ __attribute__((aligned(16))) uint16_t dt[2][32 * C4_DROW];
    __shared__ __attribute__((aligned(16))) float red[64 * C4_NACC * 4];
    __shared__ __attribute__((aligned(16))) uint16_t gtile[2][8 * GT_S * 4];
    __shared__ __attribute__((aligned(16))) uint32_t itile[2][8 * C4_NPV];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wu = __builtin_amdgcn_readfirstlane(wave);
    const int l16 = lane & 15, lg = lane >> 4;
    const int split = blockIdx.x;
    const int64_t plane = (int64_t)H * W;
    const int Dp = D / 2, Hp = H / 2, Wp = W / 2;
    const int64_t b_begin = (int64_t)split * boxes_per_split;
    const int64_t b_end = min(b_begin + boxes_per_split, nbox);
    const int nb = (int)(b_end - b_begin);
    // an even number of phases: with an odd number of boxes the last phase
    // computes a box past the end, staged as zeros, which adds exactly zero
    const int nph = (nb + 1) & ~1;

    f32x4 acc[NCF][3][3];          // [co frag][pair frag][kw] (compute waves)
#pragma unroll
    for (int i = 0; i < NCF; ++i)
#pragma unroll
        for (int f = 0; f < 3; ++f)
#pragma unroll
            for (int kw = 0; kw < 3; ++kw) acc[i][f][kw] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (wu >= C4W_NCT / 64) {
        // ------------------------------------------------------- staging waves
        // Task layout of wgrad_c4_kernel with thread index p: dY rebuild task
        // p (octet, 4-channel group); X task p - 128 on p = 128..235; pooled
        // dP and P (one pooled voxel x 8 channels) on p < 128, indices (16)
        // on p = 128..191.
        const int p = tid - C4W_NCT;
        const int oct = p % C4_NOCT, cg = p / C4_NOCT;
        const int xtask = p - 128;
        const bool is_x = xtask >= 0 && xtask < C4_NXB;
        const int row = xtask / 3, slot = xtask % 3;
        const int nvl = slot == 2 ? 2 : 8;
        const int td_o = oct / (C4_TH * 2), th_o = (oct / 2) % C4_TH, w0_o = (oct & 1) * 8;
        const bool is_pg = p < 128;
        const bool is_pi = p >= 128 && p < 192;
        const int pv = is_pg ? p >> 2 : (p - 128) >> 1;
        const int pc = is_pg ? (p & 3) * 8 : ((p - 128) & 1) * 16;
        const int hd_x = row / C4_HH, hh_x = row % C4_HH;
        const int pw_ = wu - C4W_NCT / 64;                    // staging wave 0..3
        constexpr uint32_t OOB = 0x80000000u;
        auto pick = [](bool ok, uint32_t off) {
            uint32_t r = ok ? off : OOB;
            asm volatile("" : "+v"(r));
            return r;
        };
        // two register sets of loads in flight (set s is consumed and
        // refilled in the phases of its parity); a box past the end of the
        // split gets an empty resource, so its loads read zeros
        uint4 upd_[2], upp_[2];
        uint2 ux_[2][8];
        auto load_pooled = [&](const BoxPos& bp, bool valid, auto set) {
            constexpr int S = decltype(set)::value;
            const uint32_t lim = valid ? OOB : 0u;
            // staging waves 0-1: dP and P; wave 2: window indices; wave 3: nothing
            const int pd0 = bp.bd * (C4_TD / 2);
            const int64_t pe = ((int64_t)bp.n * Dp + pd0) * ((int64_t)Hp * Wp) * CO;
            const auto r1 = pw_ == 2 ? buf_rsrc(pidx + pe, lim) : buf_rsrc(dP + pe, lim);
            const auto r2 = buf_rsrc(Pv + pe, lim);
            const int pd = pd0 + pv / 16, ph = bp.bh * (C4_TH / 2) + (pv / 8) % 2, pw = bp.bw * (C4_TW / 2) + pv % 8;
            const bool pok = (is_pg | is_pi) & (pd < Dp) & (ph < Hp) & (pw < Wp);
            const uint32_t e = ((uint32_t)(pd - pd0) * (uint32_t)Hp + (uint32_t)ph) * (uint32_t)Wp * CO +
                               (uint32_t)pw * CO + (uint32_t)pc;
            upd_[S] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r1, pick(pok, is_pg ? 2 * e : e), 0, 0));
            upp_[S] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r2, pick(pok & is_pg, 2 * e), 0, 0));
        };
        auto load_x = [&](const BoxPos& bp, bool valid, auto set) {
            constexpr int S = decltype(set)::value;
            const uint32_t lim = valid ? OOB : 0u;
            const int gd0 = bp.bd * C4_TD;
            const int xd0 = gd0 > 0 ? gd0 - 1 : 0;
            const auto rx = buf_rsrc(X + ((int64_t)bp.n * D + xd0) * plane * 4, lim);
            const int gd = gd0 + hd_x - 1, gh = bp.bh * C4_TH + hh_x - 1;
            const bool rok = is_x & ((unsigned)gd < (unsigned)D) & ((unsigned)gh < (unsigned)H);
            const int gwb = bp.bw * C4_TW + 8 * slot - 1;
            const uint32_t rbase = ((uint32_t)(gd - xd0) * (uint32_t)H + (uint32_t)gh) * (uint32_t)W + (uint32_t)gwb;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t off = pick(rok & (j < nvl) & ((unsigned)(gwb + j) < (unsigned)W), (rbase + j) * 8u);
                ux_[S][j] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rx, off, 0, 0));
            }
        };
        // gated pooled gradient dP * (P > 0 ? 1 : slope), rounded to bf16, and the indices
        auto store_pooled = [&](int g, auto set) {
            constexpr int S = decltype(set)::value;
            const uint4& upd = upd_[S];
            const uint4& upp = upp_[S];
            // every lane takes delivery of the set, whatever its role, so the
            // loads are complete on every path before the registers are reused
            asm volatile("" ::"v"(upd.x), "v"(upd.y), "v"(upd.z), "v"(upd.w), "v"(upp.x), "v"(upp.y), "v"(upp.z), "v"(upp.w));
            if (is_pg) {
                const uint32_t gd4[4] = {upd.x, upd.y, upd.z, upd.w};
                const uint32_t pv4[4] = {upp.x, upp.y, upp.z, upp.w};
                uint32_t gg[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    float gl = __uint_as_float(gd4[m] << 16), gh_ = __uint_as_float(gd4[m] & 0xffff0000u);
                    const float pl = __uint_as_float(pv4[m] << 16), ph = __uint_as_float(pv4[m] & 0xffff0000u);
                    gl = pl > 0.f ? gl : slope * gl;
                    gh_ = ph > 0.f ? gh_ : slope * gh_;
                    gg[m] = pack_bf16x2(gl, gh_);
                }
                *reinterpret_cast<uint2*>(&gtile[g][((pc / 4) * GT_S + pv) * 4]) = make_uint2(gg[0], gg[1]);
                *reinterpret_cast<uint2*>(&gtile[g][((pc / 4 + 1) * GT_S + pv) * 4]) = make_uint2(gg[2], gg[3]);
            } else if (is_pi) {
                itile[g][(pc / 4) * C4_NPV + pv] = upd.x;
                itile[g][(pc / 4 + 1) * C4_NPV + pv] = upd.y;
                itile[g][(pc / 4 + 2) * C4_NPV + pv] = upd.z;
                itile[g][(pc / 4 + 3) * C4_NPV + pv] = upd.w;
            }
        };
        auto store_x = [&](int buf, auto set) {
            constexpr int S = decltype(set)::value;
            uint2 (&ux)[8] = ux_[S];
#pragma unroll
            for (int j = 0; j < 8; ++j) asm volatile("" ::"v"(ux[j].x), "v"(ux[j].y));
            if (!is_x) return;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
                uint32_t d[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t wl = (c >> 1) ? ux[2 * k].y : ux[2 * k].x;
                    const uint32_t wh = (c >> 1) ? ux[2 * k + 1].y : ux[2 * k + 1].x;
                    d[k] = __builtin_amdgcn_perm(wh, wl, sel);
                }
                uint16_t* dst = &xt[buf][c * C4_XPL + row * C4_XW + slot * 8];
                if (slot < 2) *reinterpret_cast<uint4*>(dst) = make_uint4(d[0], d[1], d[2], d[3]);
                else *reinterpret_cast<uint32_t*>(dst) = d[0];
            }
        };
        // This thread's 8 voxels x 4 channels of dY, exactly as the pool
        // backward makes them: the gated gradient dP * (P > 0 ? 1 : slope),
        // rounded to bf16, at the voxel the window index names, zero
        // elsewhere.  Byte lookups (v_perm) instead of per-channel compares:
        // x has byte c = idx_c ^ pos, which is 0 where the window maximum is
        // the even-w voxel of this thread's pair and 1 where it is the odd one
        // (pos is even); a lookup turns those bytes into 0xff masks for all
        // four channels at once, the masks are widened to the 16-bit lanes of
        // the gradient pairs, and a permute assembles each output word (even
        // voxel in the low half, odd voxel in the high half).
        auto rebuild = [&](int g, int buf) {
            const uint32_t pos_ab = (uint32_t)((td_o & 1) * 4 + (th_o & 1) * 2);
            const int pv0 = ((td_o >> 1) * 2 + (th_o >> 1)) * 8 + w0_o / 2;
            const uint4 g01 = *reinterpret_cast<const uint4*>(&gtile[g][(cg * GT_S + pv0) * 4]);
            const uint4 g23 = *reinterpret_cast<const uint4*>(&gtile[g][(cg * GT_S + pv0 + 2) * 4]);
            const uint4 i4 = *reinterpret_cast<const uint4*>(&itile[g][cg * C4_NPV + pv0]);
            const uint2 gq[4] = {make_uint2(g01.x, g01.y), make_uint2(g01.z, g01.w), make_uint2(g23.x, g23.y),
                                 make_uint2(g23.z, g23.w)};
            const uint32_t iq[4] = {i4.x, i4.y, i4.z, i4.w};
            const uint32_t posrep = pos_ab * 0x01010101u;
            uint32_t wd[4][4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t x = iq[k] ^ posrep;
                const uint32_t lom = __builtin_amdgcn_perm(0u, 0x000000ffu, x);
                const uint32_t him = __builtin_amdgcn_perm(0u, 0x0000ff00u, x);
                const uint32_t a01 = gq[k].x & __builtin_amdgcn_perm(lom, lom, 0x01010000u);
                const uint32_t b01 = gq[k].x & __builtin_amdgcn_perm(him, him, 0x01010000u);
                const uint32_t a23 = gq[k].y & __builtin_amdgcn_perm(lom, lom, 0x03030202u);
                const uint32_t b23 = gq[k].y & __builtin_amdgcn_perm(him, him, 0x03030202u);
                wd[k][0] = __builtin_amdgcn_perm(b01, a01, 0x05040100u);
                wd[k][1] = __builtin_amdgcn_perm(b01, a01, 0x07060302u);
                wd[k][2] = __builtin_amdgcn_perm(b23, a23, 0x05040100u);
                wd[k][3] = __builtin_amdgcn_perm(b23, a23, 0x07060302u);
            }
#pragma unroll
            for (int c = 0; c < 4; ++c)
                *reinterpret_cast<uint4*>(&dt[buf][(cg * 4 + c) * C4_DROW + oct * 8]) =
                    make_uint4(wd[0][c], wd[1][c], wd[2][c], wd[3][c]);
        };

        // Phase k (the compute waves on box k): store box k + 1's X halo and
        // box k + 2's pooled tiles from register set k & 1 (loaded two phases
        // earlier), rebuild box k + 1's dY, then refill set k & 1 with the
        // loads of box k + 3's X halo and box k + 4's pooled tiles.  The loads
        // are the same on every path (boxes past the end read zeros), so the
        // compiler waits only for the set being stored.
        using Set0 = std::integral_constant<int, 0>;
        using Set1 = std::integral_constant<int, 1>;
        BoxPos bx = box_uniform(box_decode(b_begin, bD, bH, bW));      // next X box to load
        load_x(bx, true, Set0{});
        BoxPos bq = bx;                                                  // next pooled box to load
        load_pooled(bq, true, Set1{});
        store_x(0, Set0{});
        store_pooled(0, Set1{});
        bq = box_uniform(box_next(bq, bD, bH, bW));
        load_pooled(bq, nb > 1, Set1{});
        store_pooled(1, Set1{});
        // sets: 0 = {X 1, pooled 2}, 1 = {X 2, pooled 3}
        bx = box_uniform(box_next(bx, bD, bH, bW));
        load_x(bx, nb > 1, Set0{});
        bq = box_uniform(box_next(bq, bD, bH, bW));
        load_pooled(bq, nb > 2, Set0{});
        bx = box_uniform(box_next(bx, bD, bH, bW));
        load_x(bx, nb > 2, Set1{});
        bq = box_uniform(box_next(bq, bD, bH, bW));
        load_pooled(bq, nb > 3, Set1{});
        lds_barrier();
        rebuild(0, 0);
        lds_barrier();
        auto phase = [&](int k, auto set) {
            constexpr int S = decltype(set)::value;
            const int b1 = (k + 1) & 1;
            store_x(b1, set);
            rebuild(b1, b1);
            store_pooled(k & 1, set);
            bx = box_uniform(box_next(bx, bD, bH, bW));
            load_x(bx, k + 3 < nb, set);
            bq = box_uniform(box_next(bq, bD, bH, bW));
            load_pooled(bq, k + 4 < nb, set);
            (void)S;
            lds_barrier();
        };
        for (int k = 0; k < nph; k += 2) {
            phase(k, Set0{});
            phase(k + 1, Set1{});
        }
    } else {
        // ------------------------------------------------------- compute waves
        int pkd[3], pkh[3];
#pragma unroll
        for (int f = 0; f < 3; ++f) {
            const int pr = 4 * f + (l16 >> 2);
            pkd[f] = pr < 9 ? pr / 3 : 0;
            pkh[f] = pr < 9 ? pr % 3 : 0;
        }
        const int ci = l16 & 3;
        lds_barrier();
        lds_barrier();
        for (int k = 0; k < nph; ++k) {
            const int buf = k & 1;
            const uint16_t* xb = xt[buf];
            const uint16_t* db = dt[buf];
#pragma unroll
            for (int ss = 0; ss < 2; ++ss) {
                const int s = wave + 4 * ss;                       // k-step of this wave
                const int o = 4 * s + lg;                          // octet of this lane group
                const int td = o / (C4_TH * 2), th = (o / 2) % C4_TH, w0 = (o & 1) * 8;
                bf16x8 a[NCF];
#pragma unroll
                for (int i = 0; i < NCF; ++i)
                    a[i] = *reinterpret_cast<const bf16x8*>(db + (16 * i + l16) * C4_DROW + o * 8);
#pragma unroll
                for (int f = 0; f < 3; ++f) {
                    const int r = (td + pkd[f]) * C4_HH + th + pkh[f];
                    const uint16_t* xp = xb + ci * C4_XPL + r * C4_XW + w0;
                    uint4 q = *reinterpret_cast<const uint4*>(xp);
                    uint32_t e = reinterpret_cast<const uint4*>(xp)[1].x;
                    asm volatile("" : "+v"(q.x), "+v"(q.y), "+v"(q.z), "+v"(q.w), "+v"(e));
                    const uint4 s1 = make_uint4(__builtin_amdgcn_alignbit(q.y, q.x, 16), __builtin_amdgcn_alignbit(q.z, q.y, 16),
                                                __builtin_amdgcn_alignbit(q.w, q.z, 16), __builtin_amdgcn_alignbit(e, q.w, 16));
                    const bf16x8 b0 = __builtin_bit_cast(bf16x8, q);
                    const bf16x8 b1 = __builtin_bit_cast(bf16x8, s1);
                    const bf16x8 b2 = __builtin_bit_cast(bf16x8, make_uint4(q.y, q.z, q.w, e));
#pragma unroll
                    for (int i = 0; i < NCF; ++i) {
                        acc[i][f][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b0, acc[i][f][0], 0, 0, 0);
                        acc[i][f][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b1, acc[i][f][1], 0, 0, 0);
                        acc[i][f][2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b2, acc[i][f][2], 0, 0, 0);
                    }
                }
            }
            lds_barrier();
        }
    }

    // Sum the four compute waves' accumulators in the order ((w0 + w3) + w2) + w1
    // (every wave passes these barriers; the staging waves have nothing to add).
    for (int w = 3; w >= 1; --w) {
        __syncthreads();
        if (wu == w) {
#pragma unroll
            for (int i = 0; i < NCF; ++i)
#pragma unroll
                for (int f = 0; f < 3; ++f)
#pragma unroll
                    for (int kw = 0; kw < 3; ++kw)
                        *reinterpret_cast<f32x4*>(&red[(((i * 3 + f) * 3 + kw) * 64 + lane) * 4]) = acc[i][f][kw];
        }
        __syncthreads();
        if (wu == 0) {
#pragma unroll
            for (int i = 0; i < NCF; ++i)
#pragma unroll
                for (int f = 0; f < 3; ++f)
#pragma unroll
                    for (int kw = 0; kw < 3; ++kw)
                        acc[i][f][kw] += *reinterpret_cast<const f32x4*>(&red[(((i * 3 + f) * 3 + kw) * 64 + lane) * 4]);
        }
    }
    if (wu == 0) {
        const int ci = l16 & 3;
        float* out = part + (int64_t)split * (27 * 4 * CO);
#pragma unroll
        for (int f = 0; f < 3; ++f) {
            const int pr = 4 * f + (l16 >> 2);
            if (pr >= 9) continue;
#pragma unroll
            for (int kw = 0; kw < 3; ++kw) {
                const int t = pr * 3 + kw;
#pragma unroll
                for (int i = 0; i < NCF; ++i) {
                    const int co = 16 * i + 4 * lg;
                    const f32x4 r = acc[i][f][kw];
                    *reinterpret_cast<float4*>(out + (t * 4 + ci) * CO + co) = make_float4(r[0], r[1], r[2], r[3]);
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_wgrad_c4_partials(const WgradPlan& p, const uint16_t* X, const uint16_t* dY, const uint16_t* dP,
                                    const uint16_t* P, const uint8_t* idx, float slope, float* part, const cf_dims& x,
                                    int cout, hipStream_t s)
{
    const int bD = (int)((x.d + C4_TD - 1) / C4_TD), bH = (int)((x.h + C4_TH - 1) / C4_TH),
              bW = (int)((x.w + C4_TW - 1) / C4_TW);
    const int64_t nbox = x.n * bD * bH * bW;
    if (dP) {
        if (cout != 32) return hipErrorInvalidValue;
        hipLaunchKernelGGL(wgrad_c4_ws_kernel, dim3((unsigned)p.splits), dim3(C4W_NT), 0, s, X, dP, P, idx, slope, part,
                           (int)x.n, (int)x.d, (int)x.h, (int)x.w, bD, bH, bW, nbox, (int)p.vox_per_split);
    } else if (cout == 32) {
        hipLaunchKernelGGL((wgrad_c4_kernel<32>), dim3((unsigned)p.splits), dim3(C4_NT), 0, s, X, dY, part, (int)x.n,
                           (int)x.d, (int)x.h, (int)x.w, bD, bH, bW, nbox, (int)p.vox_per_split);
    } else if (cout == 16) {
        hipLaunchKernelGGL((wgrad_c4_kernel<16>), dim3((unsigned)p.splits), dim3(C4_NT), 0, s, X, dY, part, (int)x.n,
                           (int)x.d, (int)x.h, (int)x.w, bD, bH, bW, nbox, (int)p.vox_per_split);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_wgrad_c4_pool(const WgradPlan& p, const uint16_t* X, const uint16_t* dP, const uint16_t* P,
                                const uint8_t* idx, float slope, float* part, float* dW, const cf_dims& x,
                                hipStream_t s)
{
    hipError_t e = launch_wgrad_c4_partials(p, X, nullptr, dP, P, idx, slope, part, x, 32, s);
    if (e != hipSuccess) return e;
    return launch_wgrad_reduce(part, dW, (int64_t)27 * 4 * 32, p.splits, s);
}

}  // namespace cf
