// Backward-weight of the 3^3 stride-1 pad-1 convolution on bf16 MFMA.
//
//   dW[tap][ci][co] = sum over voxels v of X[v + off(tap)][ci] * dY[v][co]
//
// (the separate backward-weight operator of CosmoFlow, Sec. III-C; the
// convolution itself is the "same"-padded stride-1 one of Oyama et al.,
// Sec. IV / Table I).  This is a GEMM whose reduction runs over voxels, while
// NDHWC stores channels contiguously: every MFMA operand needs 8 consecutive
// voxels of one channel per lane, so the staging transposes the voxel box
// into channel-major LDS tiles (below).  The X halo is staged once per voxel
// box and reused by all 27 taps.
//
// Orientation: C[co][ci] += dY^T[co][k] * Xshift[k][ci] (16x16x32 MFMA), so
// a lane's accumulator holds 4 consecutive co of one ci -> one 16-byte store
// into the [tap][ci][co] result.  The voxel reduction is split into fixed
// ranges (one per block), written as fp32 partials and summed in a fixed
// order by wgrad_reduce: the result is deterministic.
#include "cf_internal.h"
#include "wgrad_common.h"

#include <type_traits>

namespace cf {

namespace {

// ---------------------------------------------------------------- general
// MFMA operands need 8 consecutive voxels of one channel per lane.  While a
// voxel box is staged, every thread transposes 8x8 blocks (8 voxels along w
// x 8 channels) in registers and stores them channel-major in LDS, so the
// MFMA operands are single aligned 16-byte LDS reads:
//   dYT[co][k]                      k = box voxel, 8 consecutive along w
//   XT[ci][halo row (d,h)][w]       halo w 0..15; the halo w 16-17 of every
//                                   row follow the rows of the channel
//                                   plane, one bf16 pair per row
// A k-step of 32 voxels is 4 lane groups x 8 voxels along w.  For tap
// (kd,kh,kw) the X operand of an octet starting at halo w0 is XT[..][w0+kw
// .. w0+kw+7]: the lane reads the octet and the next two halo values once
// and forms the three kw-shifted operands by register selection (kw = 0, 2)
// and a 16-bit funnel shift (kw = 1).
// Block: BO output channels x 32 input channels.  A wave owns two 16-wide
// output-channel fragments, one 16-wide input-channel fragment and one kd,
// i.e. 2 x 9 accumulator tiles.  A lane group walks the two w-octets of one
// halo row together, so the first octet's kw-shift word is the second
// octet's first word and only the second needs a separate 4-byte read: per
// 36 MFMAs a wave issues 4 dY reads and 9 X reads.  LDS instruction issue,
// not bytes, is what limits these loops on gfx950 (a 4-byte and a 16-byte
// per-lane read cost about the same), so reads per MFMA is the figure that
// matters.  Box: 4 x 4 x 16 voxels (halo 6 x 6 x 18); the wave-specialized
// kernel also has a 4 x 8 x 8 box for narrow volumes.  The next box is
// loaded into registers while the current one is computed.
constexpr int GW_TD = 4, GW_TH = 4, GW_TW = 16;
constexpr int GW_VB = GW_TD * GW_TH * GW_TW;                 // 256 voxels per box
constexpr int GW_NOCT = GW_VB / 8;                          // 32 w-octets
constexpr int GW_HH = GW_TH + 2;
constexpr int GW_NR = (GW_TD + 2) * GW_HH;                  // 36 halo rows
constexpr int GW_XW = 16;                                   // bf16 per XT row: halo w 0-15
constexpr int GW_XE = GW_NR * GW_XW;                        // halo w 16-17 of the rows, one bf16 pair each
constexpr int GW_XPL = GW_XE + 2 * GW_NR + 16;              // per-channel plane: 1328 B (odd multiple of 16)
constexpr int GW_DROW = GW_VB + 16;                         // dYT row: 544 B (odd multiple of 32)
constexpr int GW_NXB = GW_NR * 2 * 4;                       // X blocks of 8 voxels: rows x {w 0-7, 8-15} x 4 ci-groups
constexpr int GW_NXE = GW_NR * 4;                           // X edge blocks (w 16-17): rows x 4 ci-groups


// 8x8 transpose of bf16: in[v] holds 8 channels of voxel v; out[c] holds
// voxel 0..7 of channel c.
__device__ __forceinline__ void transpose8x8(const uint4 (&in)[8], uint4 (&out)[8])
{
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
        uint32_t d[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint4& lo = in[2 * k];
            const uint4& hi = in[2 * k + 1];
            const uint32_t wl = (c >> 1) == 0 ? lo.x : (c >> 1) == 1 ? lo.y : (c >> 1) == 2 ? lo.z : lo.w;
            const uint32_t wh = (c >> 1) == 0 ? hi.x : (c >> 1) == 1 ? hi.y : (c >> 1) == 2 ? hi.z : hi.w;
            d[k] = __builtin_amdgcn_perm(wh, wl, sel);
        }
        out[c] = make_uint4(d[0], d[1], d[2], d[3]);
    }
}

template <int BO>
struct GwCfg {
    static constexpr int NCP = BO / 32;                     // output-channel fragment pairs
    static constexpr int NW = NCP * 2 * 3;                  // waves: co pair x ci fragment x kd
    static constexpr int NT = NW * 64;
    static constexpr int NDB = GW_NOCT * (BO / 8);          // dY blocks of 8 voxels x 8 co
    static constexpr int NB = NDB + GW_NXB;                 // full 8-voxel blocks per box
    static constexpr int KB = (NB + NT - 1) / NT;           // full blocks per thread
    // Waves per SIMD the registers are sized for (the second launch bound):
    // three for the 12-wave block; two for the 6-wave block, whose two
    // staging blocks per thread do not fit in a third of the register file.
    static constexpr int WPE = BO == 64 ? 3 : 2;
    static_assert(GW_NXE <= NT, "one edge block per thread");
};

template <int BO>
__global__ __launch_bounds__(GwCfg<BO>::NT, GwCfg<BO>::WPE)
void wgrad_mfma_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ dY,
                       float* __restrict__ part, int N, int D, int H, int W, int Cin, int Cout,
                       int bD, int bH, int bW, int nco, int nci, int64_t nbox, int boxes_per_split)
{
    using G = GwCfg<BO>;
    // Two buffers of each tile: a box is staged into one while the waves
    // still compute the previous box from the other, so a box costs one
    // barrier (after its staging) instead of two.  Halo w 16-17 of the X
    // rows sit together after the rows of their channel plane (one bf16
    // pair per row), which keeps the rows 16 wide and both buffers within
    // the LDS.
    __shared__ __attribute__((aligned(16))) uint16_t xt[2][32 * GW_XPL];
    __shared__ __attribute__((aligned(16))) uint16_t dt[2][BO * GW_DROW];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const int kd = wave % 3, jf = (wave / 3) % 2, cp = wave / 6;
    // Blocks that share a voxel range (all channel blocks of one split) get
    // consecutive logical ids and therefore the same XCD and L2.
    uint32_t id = xcd_remap(blockIdx.x, gridDim.x);
    const int cob = (int)(id % (uint32_t)nco); id /= (uint32_t)nco;
    const int cib = (int)(id % (uint32_t)nci);
    const int split = (int)(id / (uint32_t)nci);
    const int co0 = cob * BO, ci0 = cib * 32;
    const int64_t plane = (int64_t)H * W;

    // Staging: full blocks t = tid + k * NT (dY blocks first, then X blocks
    // for halo w 0-15); edge blocks (X, halo w 16-17) for tid < GW_NXE.
    // 16 consecutive lanes store 16 consecutive 16-byte columns of the same
    // channel rows.  The dY and X block counts are multiples of 64, so a
    // wave's role (dY, X, edge, none) is uniform and chosen by a scalar
    // branch.  The loads are raw buffer loads at 32-bit byte offsets from
    // the box's first plane (the host keeps six planes below 2^31 bytes); a
    // lane with nothing to fetch (no task, a voxel outside the volume) gets
    // an offset beyond the resource and reads zeros without a memory access,
    // so no load sits under a per-lane branch and each address is one add
    // on a per-row base.
    // The task indices are re-derived from an opaque copy of the thread id
    // in every load and store: kept live across the compute loop they were
    // spilled, and each scratch reload then waited for the whole in-order
    // queue of the next box's prefetch loads.
    static_assert(G::NDB % 64 == 0, "wave-uniform staging roles");
    uint4 u[G::KB][8];
    uint4 ue[2];
    auto opaque_tid = [&]() {
        int t = tid;
        asm volatile("" : "+v"(t));
        return t;
    };
    const int wu = __builtin_amdgcn_readfirstlane(wave);
    constexpr uint32_t OOB = 0x80000000u;
    // offset or OOB, held in a register so the choice stays a select
    auto pick = [](bool ok, uint32_t off) {
        uint32_t r = ok ? off : OOB;
        asm volatile("" : "+v"(r));
        return r;
    };
    const uint32_t ystride = (uint32_t)Cout * 2u, xstride = (uint32_t)Cin * 2u;   // bytes per voxel

    auto load_box = [&](const BoxPos& bp) {
        const int tid_ = opaque_tid();
        const int gd0 = bp.bd * GW_TD, bh0 = bp.bh * GW_TH, bw0 = bp.bw * GW_TW;
        // dY planes gd0 .. gd0 + 3; X halo planes gd0 - 1 .. gd0 + 4 from the
        // first one inside the volume
        const int xd0 = gd0 > 0 ? gd0 - 1 : 0;
        const auto rd = buf_rsrc(dY + ((int64_t)bp.n * D + gd0) * plane * Cout + co0, OOB);
        const auto rx = buf_rsrc(X + ((int64_t)bp.n * D + xd0) * plane * Cin + ci0, OOB);
#pragma unroll
        for (int k = 0; k < G::KB; ++k) {
            const int t = tid_ + k * G::NT;
            const int t0 = wu * 64 + k * G::NT;                 // the wave's first task
            if (t0 < G::NDB) {
                const int oct = t % GW_NOCT, grp = t / GW_NOCT;
                const int td = oct / (GW_TH * 2), th = (oct / 2) % GW_TH, w0 = (oct & 1) * 8;
                const int gh = bh0 + th, gwb = bw0 + w0;
                const bool rok = (gd0 + td < D) & (gh < H);
                const uint32_t rb = (((uint32_t)td * (uint32_t)H + (uint32_t)gh) * (uint32_t)W + (uint32_t)gwb) * ystride +
                                    (uint32_t)grp * 16u;
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    u[k][j] = __builtin_bit_cast(
                        uint4, __builtin_amdgcn_raw_buffer_load_b128(rd, pick(rok & (gwb + j < W), rb + j * ystride), 0, 0));
            } else if (t0 < G::NB) {
                const int x = t - G::NDB;
                const int grp = x / (GW_NR * 2), rem = x % (GW_NR * 2);
                const int row = rem / 2, slot = rem % 2;
                const int hd = row / GW_HH, hh = row % GW_HH;
                const int gd = gd0 + hd - 1, gh = bh0 + hh - 1, gwb = bw0 + 8 * slot - 1;
                const bool rok = (t < G::NB) & ((unsigned)gd < (unsigned)D) & ((unsigned)gh < (unsigned)H);
                const uint32_t rb =
                    (((uint32_t)(gd - xd0) * (uint32_t)H + (uint32_t)gh) * (uint32_t)W + (uint32_t)gwb) * xstride +
                    (uint32_t)grp * 16u;
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    u[k][j] = __builtin_bit_cast(
                        uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                   rx, pick(rok & ((unsigned)(gwb + j) < (unsigned)W), rb + j * xstride), 0, 0));
            }
            // (a wave past the last task loads nothing; store_box skips it)
        }
        if (wu * 64 < GW_NXE) {
            const int erow = tid_ % GW_NR, egrp = tid_ / GW_NR;
            const int hd = erow / GW_HH, hh = erow % GW_HH;
            const int gd = gd0 + hd - 1, gh = bh0 + hh - 1, gw = bw0 + 15;   // halo w = 16 + j
            const bool rok = (tid_ < GW_NXE) & ((unsigned)gd < (unsigned)D) & ((unsigned)gh < (unsigned)H);
            const uint32_t rb =
                (((uint32_t)(gd - xd0) * (uint32_t)H + (uint32_t)gh) * (uint32_t)W + (uint32_t)gw) * xstride +
                (uint32_t)egrp * 16u;
#pragma unroll
            for (int j = 0; j < 2; ++j)
                ue[j] = __builtin_bit_cast(
                    uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, pick(rok & (gw + j < W), rb + j * xstride), 0, 0));
        }
    };
    auto store_box = [&](int buf) {
        const int tid_ = opaque_tid();
#pragma unroll
        for (int k = 0; k < G::KB; ++k) {
            const int t = tid_ + k * G::NT;
            const int t0 = wu * 64 + k * G::NT;
            if (t0 >= G::NB) continue;
            uint4 tr[8];
            transpose8x8(u[k], tr);
            if (t0 < G::NDB) {
                const int oct = t % GW_NOCT, grp = t / GW_NOCT;
                // octet slot (w half, box row): the 4 lane groups of a k-step then
                // read adjacent 16-byte slots, which the LDS serves without conflict
                const int slot = (oct & 1) * (GW_NOCT / 2) + (oct >> 1);
#pragma unroll
                for (int c = 0; c < 8; ++c)
                    *reinterpret_cast<uint4*>(&dt[buf][(grp * 8 + c) * GW_DROW + slot * 8]) = tr[c];
            } else if (t < G::NB) {
                const int x = t - G::NDB;
                const int grp = x / (GW_NR * 2), rem = x % (GW_NR * 2);
                const int row = rem / 2, slot = rem % 2;
#pragma unroll
                for (int c = 0; c < 8; ++c)
                    *reinterpret_cast<uint4*>(&xt[buf][(grp * 8 + c) * GW_XPL + row * GW_XW + slot * 8]) = tr[c];
            }
        }
        if (wu * 64 < GW_NXE && tid_ < GW_NXE) {
            const int erow = tid_ % GW_NR, egrp = tid_ / GW_NR;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
                const int h = c >> 1;
                const uint32_t w0v = h == 0 ? ue[0].x : h == 1 ? ue[0].y : h == 2 ? ue[0].z : ue[0].w;
                const uint32_t w1v = h == 0 ? ue[1].x : h == 1 ? ue[1].y : h == 2 ? ue[1].z : ue[1].w;
                *reinterpret_cast<uint32_t*>(&xt[buf][(egrp * 8 + c) * GW_XPL + GW_XE + 2 * erow]) =
                    __builtin_amdgcn_perm(w1v, w0v, sel);
            }
        }
    };

    f32x4 acc[2][3][3];      // [co fragment][kh][kw]
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int kh = 0; kh < 3; ++kh)
#pragma unroll
            for (int kw = 0; kw < 3; ++kw) acc[c][kh][kw] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int64_t b_begin = (int64_t)split * boxes_per_split;
    const int64_t b_end = min(b_begin + boxes_per_split, nbox);
    BoxPos bp = box_uniform(box_decode(b_begin, bD, bH, bW));
    load_box(bp);
    store_box(0);
    __syncthreads();
    // lane bases in buffer 0; the buffer offset is wave-uniform (scalar)
    const uint16_t* drow0 = dt[0] + (32 * cp + l16) * GW_DROW;
    const uint16_t* xpl0 = xt[0] + (16 * jf + l16) * GW_XPL + kd * GW_HH * GW_XW;
    int buf = 0;
    for (int64_t box = b_begin; box < b_end; ++box) {
        const int sb = __builtin_amdgcn_readfirstlane(buf);
        const uint16_t* drow = drow0 + sb * (BO * GW_DROW);
        const uint16_t* xpl = xpl0 + sb * (32 * GW_XPL);
        const bool more = box + 1 < b_end;
        if (more) {
            bp = box_uniform(box_next(bp, bD, bH, bW));
            load_box(bp);                      // in flight during this box's MFMAs
        }
#pragma unroll 1
        for (int s2 = 0; s2 < GW_TD; ++s2) {
            // lane group lg takes box row (td, th) = (s2, lg), both w-octets
            const int row = s2 * GW_TH + lg;
            bf16x8 a[2][2];                                 // [co fragment][octet]
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    a[c][h] = *reinterpret_cast<const bf16x8*>(drow + c * 16 * GW_DROW + (h * (GW_NOCT / 2) + row) * 8);
            const uint16_t* xr = xpl + (s2 * GW_HH + lg) * GW_XW;
            // this lane's edge pairs: row (kd + s2) * GW_HH + lg + kh of its plane
            const uint32_t* er = reinterpret_cast<const uint32_t*>(xpl - kd * GW_HH * GW_XW + GW_XE) +
                                 (kd + s2) * GW_HH + lg;
#pragma unroll
            for (int kh = 0; kh < 3; ++kh) {
                const uint16_t* xp = xr + kh * GW_XW;
                uint4 q0 = *reinterpret_cast<const uint4*>(xp);
                uint4 q1 = *reinterpret_cast<const uint4*>(xp + 8);
                uint32_t e1 = er[kh];                                              // halo w 16-17
                // opaque to the optimizer, which would otherwise re-read the
                // kw = 2 operands (unaligned) from LDS as extra 4-byte reads
                asm volatile("" : "+v"(q0.x), "+v"(q0.y), "+v"(q0.z), "+v"(q0.w), "+v"(q1.x), "+v"(q1.y),
                             "+v"(q1.z), "+v"(q1.w), "+v"(e1));
                const uint32_t e0 = q1.x;                                          // halo w 8-9
                bf16x8 b[2][3];                                                    // [octet][kw]
                b[0][0] = __builtin_bit_cast(bf16x8, q0);
                b[0][1] = __builtin_bit_cast(bf16x8, make_uint4(__builtin_amdgcn_alignbit(q0.y, q0.x, 16),
                                                                __builtin_amdgcn_alignbit(q0.z, q0.y, 16),
                                                                __builtin_amdgcn_alignbit(q0.w, q0.z, 16),
                                                                __builtin_amdgcn_alignbit(e0, q0.w, 16)));
                b[0][2] = __builtin_bit_cast(bf16x8, make_uint4(q0.y, q0.z, q0.w, e0));
                b[1][0] = __builtin_bit_cast(bf16x8, q1);
                b[1][1] = __builtin_bit_cast(bf16x8, make_uint4(__builtin_amdgcn_alignbit(q1.y, q1.x, 16),
                                                                __builtin_amdgcn_alignbit(q1.z, q1.y, 16),
                                                                __builtin_amdgcn_alignbit(q1.w, q1.z, 16),
                                                                __builtin_amdgcn_alignbit(e1, q1.w, 16)));
                b[1][2] = __builtin_bit_cast(bf16x8, make_uint4(q1.y, q1.z, q1.w, e1));
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int kw = 0; kw < 3; ++kw)
#pragma unroll
                        for (int c = 0; c < 2; ++c)
                            acc[c][kh][kw] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[c][h], b[h][kw], acc[c][kh][kw], 0, 0, 0);
            }
        }
        // the next box goes into the other buffer (read last in the box
        // before this one, behind the barrier that ended it)
        if (more) {
            store_box(buf ^ 1);
            __syncthreads();
            buf ^= 1;
        }
    }

    // partial[split][tap][ci][co]; lane holds co rows 4 lg..4 lg+3 of column ci
    const int64_t dwsize = (int64_t)27 * Cin * Cout;
    const int ci = ci0 + 16 * jf + l16;
    float* out = part + split * dwsize + (int64_t)ci * Cout + co0 + 32 * cp + 4 * lg;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int kh = 0; kh < 3; ++kh)
#pragma unroll
            for (int kw = 0; kw < 3; ++kw) {
                const int tap = (kd * 3 + kh) * 3 + kw;
                const f32x4 r = acc[c][kh][kw];
                *reinterpret_cast<float4*>(out + (int64_t)tap * Cin * Cout + 16 * c) = make_float4(r[0], r[1], r[2], r[3]);
            }
}


// Wave-specialized form of the 64-output-channel kernel.  Waves 0-11 compute
// exactly as wgrad_mfma_kernel<64> does; waves 12-15 hold no accumulators
// and only stage: while the compute waves walk box k from one LDS buffer,
// they load box k + 1 from global memory, transpose it and store it into the
// other buffer.  One barrier per box for all 16 waves, as before, but the
// staging's loads, permutes and stores now run beside the MFMA work instead
// of between boxes.
//
// Two box shapes of 256 voxels: 4 x 4 x 16 (TW = 16), and 4 x 8 x 8 for
// volumes at most 8 voxels wide (TW = 8), where half of a 16-wide box would
// lie outside the volume and its matrix work would be spent on zeros.  With
// TW = 16 a staging thread p (0-255) owns dY block p, X block p and either
// X block 256 + p (p < 32) or edge block p - 32 (p < 176): three sets of
// eight 16-byte loads, all issued before the first store.  With TW = 8 a
// halo row holds one 8-voxel block and one edge pair, and thread p owns dY
// block p, X block p and edge block p (p < 240).
constexpr int WS_NCW = 12, WS_NPW = 4, WS_NT = (WS_NCW + WS_NPW) * 64, WS_NPT = WS_NPW * 64;

template <int TW_>
struct WsGeom {
    static constexpr int TW = TW_, TD = 4, TH = 256 / (TD * TW);
    static constexpr int OPR = TW / 8;                      // w-octets per box row
    static constexpr int VB = TD * TH * TW, NOCT = VB / 8;
    static constexpr int HH = TH + 2, NR = (TD + 2) * HH;   // halo rows
    static constexpr int XW = TW;                           // bf16 per XT row: halo w 0 .. TW-1
    static constexpr int XE = NR * XW;                      // halo w TW, TW+1 of the rows, one bf16 pair each
    static constexpr int XPL = XE + 2 * NR + 16;            // per-channel plane (an odd multiple of 16 bytes)
    static constexpr int DROW = VB + 16;                    // dYT row: 544 bytes
    static constexpr int NXB = NR * OPR * 4;                // X blocks of 8 voxels: rows x octets x 4 ci-groups
    static constexpr int NXE = NR * 4;                      // X edge blocks: rows x 4 ci-groups
    static constexpr int NXC = NXB > WS_NPT ? NXB - WS_NPT : 0;   // X blocks staged as a thread's third task
    static_assert(VB == 256 && (TW == 8 || TW == 16), "box shape");
    static_assert(((XPL * 2 / 16) & 1) == 1, "plane stride: odd multiple of 16 bytes");
    static_assert(NOCT * 8 == WS_NPT && NXB - NXC <= WS_NPT && NXC + NXE <= WS_NPT, "staging task layout");
};
static_assert(GwCfg<64>::NW == WS_NCW && WsGeom<16>::NR == GW_NR && WsGeom<16>::XPL == GW_XPL &&
                  WsGeom<16>::NXB == GW_NXB && WsGeom<16>::NXE == GW_NXE && WsGeom<16>::DROW == GW_DROW,
              "the 16-wide box is the shared-kernel box");

// Transposes 8 voxels x 8 channels (in[v] = channels of voxel v) and stores
// channel row c (8 voxels) at dst + c * stride, one row at a time, so only
// four registers of transposed data are live at once.
__device__ __forceinline__ void transpose_store8x8(const uint4 (&in)[8], uint16_t* dst, int stride)
{
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
        uint32_t d[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint4& lo = in[2 * k];
            const uint4& hi = in[2 * k + 1];
            const uint32_t wl = (c >> 1) == 0 ? lo.x : (c >> 1) == 1 ? lo.y : (c >> 1) == 2 ? lo.z : lo.w;
            const uint32_t wh = (c >> 1) == 0 ? hi.x : (c >> 1) == 1 ? hi.y : (c >> 1) == 2 ? hi.z : hi.w;
            d[k] = __builtin_amdgcn_perm(wh, wl, sel);
        }
        *reinterpret_cast<uint4*>(dst + c * stride) = make_uint4(d[0], d[1], d[2], d[3]);
    }
}

template <int TW>
__global__ __launch_bounds__(WS_NT)
void wgrad_ws_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ dY, float* __restrict__ part,
                     int N, int D, int H, int W, int Cin, int Cout, int bD, int bH, int bW, int nco, int nci,
                     int64_t nbox, int boxes_per_split)
{
    constexpr int BO = 64;
    using G = WsGeom<TW>;
    __shared__ __attribute__((aligned(16))) uint16_t xt[2][32 * G::XPL];
    __shared__ __attribute__((aligned(16))) uint16_t dt[2][BO * G::DROW];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wu = __builtin_amdgcn_readfirstlane(wave);
    const int l16 = lane & 15, lg = lane >> 4;
    uint32_t id = xcd_remap(blockIdx.x, gridDim.x);
    const int cob = (int)(id % (uint32_t)nco); id /= (uint32_t)nco;
    const int cib = (int)(id % (uint32_t)nci);
    const int split = (int)(id / (uint32_t)nci);
    const int co0 = cob * BO, ci0 = cib * 32;
    const int64_t plane = (int64_t)H * W;
    const int64_t b_begin = (int64_t)split * boxes_per_split;
    const int64_t b_end = min(b_begin + boxes_per_split, nbox);

    // ------------------------------------------------------------ staging
    constexpr uint32_t OOB = 0x80000000u;
    auto pick = [](bool ok, uint32_t off) {
        uint32_t r = ok ? off : OOB;
        asm volatile("" : "+v"(r));
        return r;
    };
    const uint32_t ystride = (uint32_t)Cout * 2u, xstride = (uint32_t)Cin * 2u;
    // Staging-thread constants (box-independent parts of the offsets), set
    // once before the box loop.  A box adds one scalar per tensor and voxel
    // j of a task j * voxel bytes, so a load costs an add, a compare and a
    // select.  (The same j * voxel bytes passed as the instruction's scalar
    // offset instead gave wrong staged values in testing, so the whole
    // offset stays in the per-lane operand.)
    // A: dY block p (octet, 8-channel group): byte offset from the box's
    // first plane kA + (bh0 * W + bw0) * ystride + j * ystride.
    // B: X block p; C: X block 256 + p (p < 32) or edge block p - 32: byte
    // offset from the halo's first in-volume plane
    // kX + ((e0 * H + bh0) * W + bw0) * xstride + j * xstride, with e0 = 1
    // unless the box starts at depth 0; kX may be negative, the sum is not
    // for a voxel inside the volume.
    struct XTask { int hd, hh, wb; int32_t k; bool live; };
    auto xtask = [&](int x) {
        const int grp = x / (G::NR * G::OPR), rem = x % (G::NR * G::OPR);
        const int row = rem / G::OPR, slot = rem % G::OPR;
        XTask t;
        t.hd = row / G::HH; t.hh = row % G::HH; t.wb = 8 * slot - 1;
        t.k = (((t.hd - 1) * H + (t.hh - 1)) * W + t.wb) * (int32_t)xstride + grp * 16;
        t.live = x < G::NXB;
        return t;
    };
    auto etask = [&](int e) {
        const int erow = e % G::NR, egrp = e / G::NR;
        XTask t;
        t.hd = erow / G::HH; t.hh = erow % G::HH; t.wb = TW - 1;      // halo w = TW + j
        t.k = (((t.hd - 1) * H + (t.hh - 1)) * W + t.wb) * (int32_t)xstride + egrp * 16;
        t.live = e < G::NXE;
        return t;
    };
    // voxel j of a row that starts at w = base (>= -1) is inside 0 <= w < W
    auto wok = [&](int base, int j) { return j == 0 ? (unsigned)base < (unsigned)W : base < W - j; };
    struct STasks { int32_t kA; int tdA, thA, w0A; XTask tB, tC; };
    auto stage_tasks = [&](int p) {
        STasks T;
        const int oct = p % G::NOCT, grp = p / G::NOCT;
        T.tdA = oct / (G::TH * G::OPR); T.thA = (oct / G::OPR) % G::TH; T.w0A = (oct & (G::OPR - 1)) * 8;
        T.kA = ((T.tdA * H + T.thA) * W + T.w0A) * (int32_t)ystride + grp * 16;
        T.tB = xtask(p);
        T.tC = p < G::NXC ? xtask(WS_NPT + p) : etask(p - G::NXC);
        return T;
    };
    auto stage = [&](const BoxPos& bp, int buf, const STasks& T) {
        int p = tid - WS_NCW * 64;
        asm volatile("" : "+v"(p));
        const int gd0 = bp.bd * G::TD, bh0 = bp.bh * G::TH, bw0 = bp.bw * TW;
        const int xd0 = gd0 > 0 ? gd0 - 1 : 0;
        const auto rd = buf_rsrc(dY + ((int64_t)bp.n * D + gd0) * plane * Cout + co0, OOB);
        const auto rx = buf_rsrc(X + ((int64_t)bp.n * D + xd0) * plane * Cin + ci0, OOB);
        const int32_t sA = (bh0 * W + bw0) * (int32_t)ystride;
        const int32_t sX = (((gd0 > 0 ? 1 : 0) * H + bh0) * W + bw0) * (int32_t)xstride;
        uint4 ua[8], ub[8], uc[8];
        {
            const bool rok = (gd0 + T.tdA < D) & (bh0 + T.thA < H);
            const uint32_t off = (uint32_t)(T.kA + sA);
            const int base = bw0 + T.w0A;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                ua[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                      rd, pick(rok & wok(base, j), off + j * ystride), 0, 0));
        }
        auto xload = [&](const XTask& t, uint4 (&u)[8], int n) {
            const bool rok = t.live & ((unsigned)(gd0 + t.hd - 1) < (unsigned)D) & ((unsigned)(bh0 + t.hh - 1) < (unsigned)H);
            const uint32_t off = (uint32_t)(t.k + sX);
            const int base = bw0 + t.wb;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (j < n)
                    u[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                         rx, pick(rok & wok(base, j), off + j * xstride), 0, 0));
        };
        xload(T.tB, ub, 8);
        const bool c_edge = p >= G::NXC;
        const int e = p - G::NXC;
        if (!c_edge) {
            xload(T.tC, uc, 8);
        } else {
            xload(T.tC, uc, 2);
        }
        // stores: dY block p, X block p, then block C
        {
            const int oct = p % G::NOCT, grp = p / G::NOCT;
            const int slot = (oct & (G::OPR - 1)) * (G::NOCT / G::OPR) + (oct >> (G::OPR / 2));
            transpose_store8x8(ua, &dt[buf][(grp * 8) * G::DROW + slot * 8], G::DROW);
        }
        auto xstore = [&](int x, const uint4 (&u)[8]) {
            const int grp = x / (G::NR * G::OPR), rem = x % (G::NR * G::OPR);
            const int row = rem / G::OPR, slot = rem % G::OPR;
            transpose_store8x8(u, &xt[buf][(grp * 8) * G::XPL + row * G::XW + slot * 8], G::XPL);
        };
        if (G::NXB >= WS_NPT || p < G::NXB) xstore(p, ub);
        if (!c_edge) {
            xstore(WS_NPT + p, uc);
        } else if (e < G::NXE) {
            const int erow = e % G::NR, egrp = e / G::NR;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
                const int h = c >> 1;
                const uint32_t w0v = h == 0 ? uc[0].x : h == 1 ? uc[0].y : h == 2 ? uc[0].z : uc[0].w;
                const uint32_t w1v = h == 0 ? uc[1].x : h == 1 ? uc[1].y : h == 2 ? uc[1].z : uc[1].w;
                *reinterpret_cast<uint32_t*>(&xt[buf][(egrp * 8 + c) * G::XPL + G::XE + 2 * erow]) =
                    __builtin_amdgcn_perm(w1v, w0v, sel);
            }
        }
    };

    // ------------------------------------------------------------ compute
    const int kd = wave % 3, jf = (wave / 3) % 2, cp = wave / 6;    // meaningful for waves 0-11
    f32x4 acc[2][3][3];      // [co fragment][kh][kw]
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int kh = 0; kh < 3; ++kh)
#pragma unroll
            for (int kw = 0; kw < 3; ++kw) acc[c][kh][kw] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint16_t* drow0 = dt[0] + (32 * cp + l16) * G::DROW;
    const uint16_t* xpl0 = xt[0] + (16 * jf + l16) * G::XPL + kd * G::HH * G::XW;
    // the three kw operands of one 8-voxel halo row segment q (w 0-7 of the
    // row's part) whose next two halo voxels are the low half of e: kw = 1
    // and 2 shift by one and two voxels (MFMA operands need aligned
    // register quads, so kw = 2 is a copy)
    auto shifts = [](const uint4& q, uint32_t e, bf16x8 (&b)[3]) {
        b[0] = __builtin_bit_cast(bf16x8, q);
        b[1] = __builtin_bit_cast(bf16x8, make_uint4(__builtin_amdgcn_alignbit(q.y, q.x, 16),
                                                     __builtin_amdgcn_alignbit(q.z, q.y, 16),
                                                     __builtin_amdgcn_alignbit(q.w, q.z, 16),
                                                     __builtin_amdgcn_alignbit(e, q.w, 16)));
        b[2] = __builtin_bit_cast(bf16x8, make_uint4(q.y, q.z, q.w, e));
    };
    auto compute = [&](int buf) {
        const uint16_t* drow = drow0 + buf * (BO * G::DROW);
        const uint16_t* xpl = xpl0 + buf * (32 * G::XPL);
#pragma unroll 1
        for (int s2 = 0; s2 < G::TD; ++s2) {
            // the 32-voxel reduction step of one MFMA: 4 h rows (one per lane
            // group) x 8 w voxels.  TW = 16: the two w-octets of rows
            // s2 * 4 + lg; TW = 8: rows s2 * 8 + lg and s2 * 8 + 4 + lg.
            bf16x8 a[2][2];                                 // [co fragment][step]
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int slot = TW == 16 ? h * (G::NOCT / 2) + s2 * G::TH + lg : s2 * G::TH + 4 * h + lg;
                    a[c][h] = *reinterpret_cast<const bf16x8*>(drow + c * 16 * G::DROW + slot * 8);
                }
            if constexpr (TW == 16) {
                const uint16_t* xr = xpl + (s2 * G::HH + lg) * G::XW;
                const uint32_t* er = reinterpret_cast<const uint32_t*>(xpl - kd * G::HH * G::XW + G::XE) +
                                     (kd + s2) * G::HH + lg;
#pragma unroll
                for (int kh = 0; kh < 3; ++kh) {
                    const uint16_t* xp = xr + kh * G::XW;
                    uint4 q0 = *reinterpret_cast<const uint4*>(xp);
                    uint4 q1 = *reinterpret_cast<const uint4*>(xp + 8);
                    uint32_t e1 = er[kh];
                    asm volatile("" : "+v"(q0.x), "+v"(q0.y), "+v"(q0.z), "+v"(q0.w), "+v"(q1.x), "+v"(q1.y),
                                 "+v"(q1.z), "+v"(q1.w), "+v"(e1));
                    bf16x8 b[2][3];
                    shifts(q0, q1.x, b[0]);
                    shifts(q1, e1, b[1]);
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int kw = 0; kw < 3; ++kw)
#pragma unroll
                            for (int c = 0; c < 2; ++c)
                                acc[c][kh][kw] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[c][h], b[h][kw], acc[c][kh][kw], 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint16_t* xr = xpl + (s2 * G::HH + 4 * h + lg) * G::XW;
                    const uint32_t* er = reinterpret_cast<const uint32_t*>(xpl - kd * G::HH * G::XW + G::XE) +
                                         (kd + s2) * G::HH + 4 * h + lg;
#pragma unroll
                    for (int kh = 0; kh < 3; ++kh) {
                        uint4 q0 = *reinterpret_cast<const uint4*>(xr + kh * G::XW);
                        uint32_t e0 = er[kh];
                        asm volatile("" : "+v"(q0.x), "+v"(q0.y), "+v"(q0.z), "+v"(q0.w), "+v"(e0));
                        bf16x8 b[3];
                        shifts(q0, e0, b);
#pragma unroll
                        for (int kw = 0; kw < 3; ++kw)
#pragma unroll
                            for (int c = 0; c < 2; ++c)
                                acc[c][kh][kw] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[c][h], b[kw], acc[c][kh][kw], 0, 0, 0);
                    }
                }
            }
        }
    };

    // Box b_begin is staged before the loop; in the iteration of box k the
    // compute waves read buffer (k - b_begin) & 1 while the staging waves
    // fill the other with box k + 1 (last read in the iteration before,
    // behind the barrier that ended it).  The two roles run separate loops
    // (the accumulators are live only in the compute waves' loop), and each
    // passes one barrier before its loop and one per box: the same count,
    // which is what the workgroup barrier needs.
    if (wu >= WS_NCW) {
        const STasks T = stage_tasks(tid - WS_NCW * 64);
        BoxPos bp = box_uniform(box_decode(b_begin, bD, bH, bW));
        stage(bp, 0, T);
        __syncthreads();
        int buf = 0;
        for (int64_t box = b_begin; box < b_end; ++box) {
            if (box + 1 < b_end) {
                bp = box_uniform(box_next(bp, bD, bH, bW));
                stage(bp, buf ^ 1, T);
            }
            __syncthreads();
            buf ^= 1;
        }
        return;
    }
    __syncthreads();
    int buf = 0;
    for (int64_t box = b_begin; box < b_end; ++box) {
        compute(__builtin_amdgcn_readfirstlane(buf));
        __syncthreads();
        buf ^= 1;
    }

    // partial[split][tap][ci][co]; lane holds co rows 4 lg..4 lg+3 of column ci
    const int64_t dwsize = (int64_t)27 * Cin * Cout;
    const int ci = ci0 + 16 * jf + l16;
    float* out = part + split * dwsize + (int64_t)ci * Cout + co0 + 32 * cp + 4 * lg;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int kh = 0; kh < 3; ++kh)
#pragma unroll
            for (int kw = 0; kw < 3; ++kw) {
                const int tap = (kd * 3 + kh) * 3 + kw;
                const f32x4 r = acc[c][kh][kw];
                *reinterpret_cast<float4*>(out + (int64_t)tap * Cin * Cout + 16 * c) = make_float4(r[0], r[1], r[2], r[3]);
            }
}


// dW[e] = sum over splits of part[s][e].  A block owns RD_E consecutive
// elements (4 per thread, 16-byte loads; small blocks, so even a few
// thousand elements spread over all CUs); its 16 split-lanes each sum the
// splits s = lane, lane + 16, ... in increasing order, and the 16 lane sums
// are added in lane order.  The order is fixed, so the result is
// deterministic.  n must be a multiple of 4 (27 * Cin * Cout with Cin a
// multiple of 4).
constexpr int RD_T = 16, RD_E = RD_T * 4, RD_L = 16;   // 256 threads, 64 elements per block

__global__ __launch_bounds__(RD_T * RD_L)
void wgrad_reduce_kernel(const float* __restrict__ part, float* __restrict__ dW, int64_t n, int splits)
{
    __shared__ float4 red[RD_L][RD_T];
    const int el = threadIdx.x % RD_T, sl = threadIdx.x / RD_T;
    const int64_t i = (int64_t)blockIdx.x * RD_E + 4 * el;
    const int64_t n4 = n / 4;
    const float4* p4 = reinterpret_cast<const float4*>(part);
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < n) {
        int k = sl;
        for (; k + 7 * RD_L < splits; k += 8 * RD_L) {
            float4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = p4[(int64_t)(k + u * RD_L) * n4 + i / 4];
#pragma unroll
            for (int u = 0; u < 8; ++u) { s.x += v[u].x; s.y += v[u].y; s.z += v[u].z; s.w += v[u].w; }
        }
        for (; k < splits; k += RD_L) {
            const float4 v = p4[(int64_t)k * n4 + i / 4];
            s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
        }
    }
    red[sl][el] = s;
    __syncthreads();
    if (sl == 0 && i < n) {
        float4 t = red[0][el];
#pragma unroll
        for (int k = 1; k < RD_L; ++k) {
            const float4 v = red[k][el];
            t.x += v.x; t.y += v.y; t.z += v.z; t.w += v.w;
        }
        dW[i] = t.x; dW[i + 1] = t.y; dW[i + 2] = t.z; dW[i + 3] = t.w;
    }
}

// Box width of the Cin % 32 == 0 kernels: the 4 x 8 x 8 box where a 16-wide
// one would be half outside the volume (64-channel output blocks only).
int wgrad_box_w(const cf_dims& x, int cout)
{
    return cout % 64 == 0 && x.w <= 8 ? 8 : 16;
}

}  // namespace

bool wgrad_mfma_fits(const cf_dims& x, int cout)
{
    const int64_t c = x.c > cout ? x.c : cout;
    return 6 * x.h * x.w * c * 2 + 64 < ((int64_t)1 << 31);
}

bool wgrad_c4_fits(const cf_dims& x)
{
    return x.h * x.w <= ((int64_t)1 << 23);
}

WgradPlan plan_wgrad(const cf_dims& x, int cout)
{
    WgradPlan p{};
    const int64_t dw_bytes = (int64_t)27 * x.c * cout * 4;
    if (x.c == 4) {
        p.kind = 1;
        const int64_t nbox = x.n * ((x.d + C4_TD - 1) / C4_TD) * ((x.h + C4_TH - 1) / C4_TH) *
                             ((x.w + C4_TW - 1) / C4_TW);
        int64_t splits = nbox < 512 ? nbox : 512;
        const int64_t per = (nbox + splits - 1) / splits;
        splits = (nbox + per - 1) / per;
        p.splits = (int)splits;
        p.vox_per_split = per;   // boxes per split
    } else {
        p.kind = 0;
        const int bo = cout % 64 == 0 ? 64 : 32;
        const int tw = wgrad_box_w(x, cout), th = 256 / (4 * tw);
        const int64_t nbox = x.n * ((x.d + 3) / 4) * ((x.h + th - 1) / th) * ((x.w + tw - 1) / tw);
        const int64_t outer = (int64_t)(cout / bo) * (x.c / 32);
        // one round of blocks over the 256 CUs (one 12-wave or two 6-wave blocks per CU)
        const int64_t conc = bo == 64 ? 256 : 512;
        int64_t want = (conc + outer - 1) / outer;
        int64_t cap = (int64_t)(64ll << 20) / dw_bytes;   // bound the partial buffer to ~64 MiB
        if (cap < 1) cap = 1;
        if (want > cap) want = cap;
        if (want > nbox) want = nbox;
        if (want < 1) want = 1;
        const int64_t per = (nbox + want - 1) / want;
        p.splits = (int)((nbox + per - 1) / per);
        p.vox_per_split = per;
    }
    p.part_bytes = (size_t)p.splits * (size_t)dw_bytes;
    return p;
}

hipError_t launch_wgrad(const WgradPlan& p, const uint16_t* X, const uint16_t* dY, float* part, float* dW,
                        const cf_dims& x, int cout, hipStream_t s)
{
    if (p.kind == 1) {
        hipError_t e = launch_wgrad_c4_partials(p, X, dY, nullptr, nullptr, nullptr, 0.f, part, x, cout, s);
        if (e != hipSuccess) return e;
    } else {
        const int tw = wgrad_box_w(x, cout), th = 256 / (4 * tw);
        const int bD = (int)((x.d + 3) / 4), bH = (int)((x.h + th - 1) / th), bW = (int)((x.w + tw - 1) / tw);
        const int64_t nbox = x.n * bD * bH * bW;
        const int nci = (int)(x.c / 32);
        if (cout % 64 == 0) {
            const int nco = cout / 64;
            const dim3 grid((unsigned)((int64_t)nco * nci * p.splits));
            if (tw == 8)
                hipLaunchKernelGGL(wgrad_ws_kernel<8>, grid, dim3(WS_NT), 0, s, X, dY, part, (int)x.n, (int)x.d,
                                   (int)x.h, (int)x.w, (int)x.c, cout, bD, bH, bW, nco, nci, nbox,
                                   (int)p.vox_per_split);
            else
                hipLaunchKernelGGL(wgrad_ws_kernel<16>, grid, dim3(WS_NT), 0, s, X, dY, part, (int)x.n, (int)x.d,
                                   (int)x.h, (int)x.w, (int)x.c, cout, bD, bH, bW, nco, nci, nbox,
                                   (int)p.vox_per_split);
        } else {
            const int nco = cout / 32;
            hipLaunchKernelGGL(wgrad_mfma_kernel<32>, dim3((unsigned)((int64_t)nco * nci * p.splits)),
                               dim3(GwCfg<32>::NT), 0, s, X, dY, part, (int)x.n, (int)x.d, (int)x.h, (int)x.w,
                               (int)x.c, cout, bD, bH, bW, nco, nci, nbox, (int)p.vox_per_split);
        }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_wgrad_reduce(part, dW, (int64_t)27 * x.c * cout, p.splits, s);
}

hipError_t launch_wgrad_reduce(const float* part, float* dW, int64_t n, int splits, hipStream_t s)
{
    hipLaunchKernelGGL(wgrad_reduce_kernel, dim3((unsigned)((n + RD_E - 1) / RD_E)), dim3(RD_T * RD_L), 0, s, part, dW,
                       n, splits);
    return hipGetLastError();
}

}  // namespace cf
