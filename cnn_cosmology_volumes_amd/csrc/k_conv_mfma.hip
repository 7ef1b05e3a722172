// Implicit-GEMM 3^3 convolution on gfx950 bf16 MFMA (v_mfma_f32_16x16x32_bf16).
//
// Computes Y[v, co] = sum_{tap, ci} X[v + off(tap), ci] * Wk[tap][co][ci] for a
// stride-1, pad-1 3^3 cross-correlation on NDHWC tensors (the forward
// convolution of Oyama et al., Sec. IV / Table I: "same" padding, stride 1, no
// bias).  With Wk prepared as the tap-flipped, channel-swapped weights the same
// kernel computes the backward-data pass (the adjoint of the forward operator
// for stride 1 and pad 1 is a pad-1 correlation with W[2-kd,2-kh,2-kw]^T).
//
// GEMM view: rows = output channels (MFMA A operand = weights), columns =
// output voxels (MFMA B operand = input halo), K = 27 taps x in-channels.
//  - A block owns a TD x TH x TW output tile of one sample and BM output
//    channels.  For every 32-channel input chunk it stages the
//    (TD+2)(TH+2)(TW+2) halo of the input in LDS once and then walks the 27
//    taps; a tap only shifts the LDS row index, so every B fragment is one
//    aligned 16-byte LDS read at a compile-time offset from one of three
//    per-lane bases.  The LDS voxel stride is 64 bytes (unpadded), and the
//    two 32-byte halves of a voxel are swapped where bit 2 of its halo w is
//    set: 16 lanes read 16 consecutive voxels, and without the swap voxels
//    w and w + 4 fall on the same LDS banks (a measured 2-way conflict on
//    gfx950: 8.7 against 4.4 clocks per 16-byte wave read).  One tile that
//    is at the register limit keeps the plain layout (see SWZ).
//  - A fragments (8 consecutive in-channels of one output channel) are
//    16-byte global loads from the [tap][co][ci] weight copy, which is small
//    and stays L2/L1 resident.
//  - Accumulation is fp32; the epilogue rounds to bf16 (or writes fp32
//    partial sums when the in-channel reduction is split across blocks).
#include "cf_internal.h"

namespace cf {

namespace {

// BM output channels per block split over BM/WM waves; TD*TH*TW voxels per
// block split over VT/WN waves; each wave owns a WM x WN accumulator tile.
// Waves that share a channel slice load the same weight fragments, so a
// narrow WM (32) with a wide WN (128) halves the redundant weight traffic
// against a 64 x 64 wave tile; the halo (B) side is read from LDS.
// LS: bf16 per halo voxel in LDS (32 = 64 bytes, unpadded; 48 adds 32 bytes
// of padding, which speeds the B reads but loses overall).
template <int BM, int WM, int WN, int TD, int TH, int TW, int LS, int WPE_ = 0>
struct Tile {
    static constexpr int NWM = BM / WM;
    static constexpr int VT = TD * TH * TW;
    static constexpr int NWV = VT / WN;
    static constexpr int NW = NWM * NWV;
    static constexpr int NT = NW * 64;
    static constexpr int HD = TD + 2, HH = TH + 2, HW = TW + 2;
    static constexpr int HV = HD * HH * HW;
    static constexpr int MI = WM / 16;
    static constexpr int NJ = WN / 16;
    // waves per SIMD the registers are sized for (the second launch bound)
    static constexpr int MINB = WPE_ ? WPE_ : (NW > 4 ? 1 : 2);
    static constexpr int NE = HV * 4;             // 16-byte halo pieces per chunk
    static constexpr int IT = (NE + NT - 1) / NT; // halo pieces per thread
    static_assert(VT % WN == 0 && (NW == 4 || NW == 8), "tile");
    // halo voxel offset (tap 0) of tile voxel v, in voxels
    __host__ __device__ static constexpr int vox_off(int v) {
        return ((v / (TH * TW)) * HH + (v / TW) % TH) * HW + v % TW;
    }
    // vox_off(w*WN + 16j + l) == vox_off(w*WN + l) + vox_off(16j) for every
    // wave w, fragment j and lane l16
    __host__ __device__ static constexpr bool frag_split() {
        for (int w = 0; w < NWV; ++w)
            for (int j = 0; j < NJ; ++j)
                for (int l = 0; l < 16; ++l)
                    if (vox_off(w * WN + 16 * j + l) != vox_off(w * WN + l) + vox_off(16 * j)) return false;
        return true;
    }
    static_assert(BM % WM == 0 && WM % 16 == 0 && WN % 16 == 0, "frag");
};

// POOL: instead of Y, write the leaky-ReLU + 2^3 max-pooled output P
// ([n][D/2][H/2][W/2][Cout]) and the window indices (first strict maximum
// of the bf16-rounded conv outputs in window order a*4 + b*2 + e, then
// leaky ReLU, exactly as the separate pool kernel computes them).  Needs a
// wave to own two whole depth planes of a 16-wide tile (WN = 2*TH*TW,
// TW = 16), so a window is 4 accumulator fragments of one lane and of its
// neighbour lane, and no split of the channel reduction.
// 16-byte chunk (0..3) of a halo voxel that holds channels 8q..8q+7: the two
// 32-byte halves are swapped where bit 2 of the voxel's halo w is set.
__device__ __forceinline__ int halo_chunk(int q, int hw) { return q ^ (((hw >> 2) & 1) << 1); }

// Pooled epilogue of the 4 x 4 x 16 tiles (BM output channels, NT threads),
// through LDS.  Each wave writes its accumulators, rounded to bf16, into a
// [tile voxel][channel] tile ZS channels wide that reuses the halo's LDS
// (every wave has passed a barrier after its last halo read); after a
// barrier, one thread per (pooled voxel, 8-channel group) reads its 2^3
// window 16 bytes per voxel, takes the first strict maximum in window order
// a*4 + b*2 + e (d, h, w offsets), applies leaky ReLU to it and stores P and
// the index.  These are the separate pool kernel's values.  vox(j) is the
// tile voxel of fragment j in this lane; the lane's channels of fragment i
// are co_wave + 16 i + 4 lg .. + 3 within the block.
template <int BM, int TD, int TH, int TW>
struct PoolTile {
    static constexpr int ZS = BM + 8;       // bf16 per tile voxel (144 bytes for BM = 64)
    static constexpr int SIZE = TD * TH * TW * ZS;
};

template <int BM, int TD, int TH, int TW, int NT, int MI, int NJ, typename Vox>
__device__ __forceinline__ void pool_epilogue_lds(uint16_t* __restrict__ zt, const f32x4 (&acc)[MI][NJ], Vox vox,
                                                  int co_wave, int lg, uint16_t* __restrict__ P,
                                                  uint8_t* __restrict__ pidx, float slope, int n, int D, int H, int W,
                                                  int Cout, int co_block, int d0, int h0, int w0)
{
    constexpr int ZS = PoolTile<BM, TD, TH, TW>::ZS;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int v = vox(j);
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const f32x4 r = acc[i][j];
            *reinterpret_cast<uint2*>(zt + v * ZS + co_wave + 16 * i + 4 * lg) =
                make_uint2(pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]));
        }
    }
    __syncthreads();
    constexpr int PD = TD / 2, PH = TH / 2, PW = TW / 2, NG = BM / 8;
    const int Dp = D >> 1, Hp = H >> 1, Wp = W >> 1;
    // 16-byte P and 8-byte index stores where every group is aligned to them
    const bool wide = Cout % 8 == 0 && (((uintptr_t)P & 15) | ((uintptr_t)pidx & 7)) == 0;
    for (int e = threadIdx.x; e < PD * PH * PW * NG; e += NT) {
        const int g = e % NG, pv = e / NG;
        const int pk = pv % PW, pj = (pv / PW) % PH, pi = pv / (PW * PH);
        const int gpd = (d0 >> 1) + pi, gph = (h0 >> 1) + pj, gpw = (w0 >> 1) + pk;
        const int co = co_block + 8 * g;
        if (gpd >= Dp || gph >= Hp || gpw >= Wp || co >= Cout) continue;
        float best[8];
        uint32_t bi[8];
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int a = p >> 2, b = (p >> 1) & 1, c = p & 1;
            const int v = ((2 * pi + a) * TH + 2 * pj + b) * TW + 2 * pk + c;
            const uint4 u = *reinterpret_cast<const uint4*>(zt + v * ZS + 8 * g);
            const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float z = __uint_as_float((k & 1) ? (w4[k >> 1] & 0xffff0000u) : (w4[k >> 1] << 16));
                if (p == 0 || z > best[k]) { best[k] = z; bi[k] = (uint32_t)p; }
            }
        }
        float out[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) out[k] = best[k] > 0.f ? best[k] : slope * best[k];
        const uint2 plo = make_uint2(pack_bf16x2(out[0], out[1]), pack_bf16x2(out[2], out[3]));
        const uint2 phi = make_uint2(pack_bf16x2(out[4], out[5]), pack_bf16x2(out[6], out[7]));
        const uint32_t ilo = bi[0] | (bi[1] << 8) | (bi[2] << 16) | (bi[3] << 24);
        const uint32_t ihi = bi[4] | (bi[5] << 8) | (bi[6] << 16) | (bi[7] << 24);
        const int64_t o = (((int64_t)n * Dp + gpd) * Hp + gph) * Wp * Cout + (int64_t)gpw * Cout + co;
        if (wide) {
            *reinterpret_cast<uint4*>(P + o) = make_uint4(plo.x, plo.y, phi.x, phi.y);
            *reinterpret_cast<uint2*>(pidx + o) = make_uint2(ilo, ihi);
        } else {
            // Cout % 4 == 0: the group's first four channels, and the next
            // four where they exist
            *reinterpret_cast<uint2*>(P + o) = plo;
            *reinterpret_cast<uint32_t*>(pidx + o) = ilo;
            if (co + 8 <= Cout) {
                *reinterpret_cast<uint2*>(P + o + 4) = phi;
                *reinterpret_cast<uint32_t*>(pidx + o + 4) = ihi;
            }
        }
    }
}

template <int BM, int WM, int WN, int TD, int TH, int TW, int LS, int WPE_ = 0, bool POOL = false>
__global__ __launch_bounds__((Tile<BM, WM, WN, TD, TH, TW, LS, WPE_>::NT), (Tile<BM, WM, WN, TD, TH, TW, LS, WPE_>::MINB))
void conv3d_mfma_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wk,
                        uint16_t* __restrict__ Y, float* __restrict__ part,
                        int N, int D, int H, int W, int Cin, int Cout, int CoutPad,
                        int tD, int tH, int tW, int chunks_per_split, uint8_t* __restrict__ pidx, float slope)
{
    using T = Tile<BM, WM, WN, TD, TH, TW, LS, WPE_>;
    __shared__ __attribute__((aligned(16))) uint16_t halo[T::HV * LS];
    const int lane = threadIdx.x & 63;
    const int wm = (threadIdx.x >> 6) % T::NWM;     // co slice of this wave
    const int wave = (threadIdx.x >> 6) / T::NWM;   // voxel slice of this wave
    const int l16 = lane & 15, lg = lane >> 4;

    uint32_t tile = xcd_remap(blockIdx.x, gridDim.x);
    const int tw_ = tile % tW; tile /= tW;
    const int th_ = tile % tH; tile /= tH;
    const int td_ = tile % tD;
    const int n = tile / tD;
    const int d0 = td_ * TD, h0 = th_ * TH, w0 = tw_ * TW;
    const int co_base = blockIdx.y * BM + wm * WM;
    const int nchunks = Cin >> 5;
    const int c_begin = blockIdx.z * chunks_per_split;
    const int c_end = min(c_begin + chunks_per_split, nchunks);

    // Per-lane LDS offsets (in bf16 units) of the B fragments: the halo
    // offset of a tile voxel splits exactly into a per-lane part (the wave's
    // planes and l16) and a compile-time part per fragment j (checked by
    // T::frag_split), so every fragment of a tap reads from one base
    // register per kw with an immediate offset.  Plus the lane's swizzled
    // 16-byte chunk for each kw (the halo w of a lane's voxel is tw + kw,
    // the same for every j).
    static_assert(T::frag_split(), "fragment offsets must split into lane and fragment parts");
    const int hb0 = T::vox_off(wave * WN + l16) * LS;
    int hb[T::NJ];
#pragma unroll
    for (int j = 0; j < T::NJ; ++j) hb[j] = hb0 + T::vox_off(16 * j) * LS;
    int sw[3];
#pragma unroll
    for (int kw = 0; kw < 3; ++kw) sw[kw] = halo_chunk(lg, (l16 % TW) + kw) * 8;

    f32x4 acc[T::MI][T::NJ];
#pragma unroll
    for (int i = 0; i < T::MI; ++i)
#pragma unroll
        for (int j = 0; j < T::NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int64_t plane = (int64_t)H * W;
    // Halo loads: raw buffer loads at 32-bit byte offsets from the tile's
    // first in-volume depth plane (the host keeps six planes below 2^31
    // bytes), computed once for all channel chunks; a piece outside the
    // volume gets an offset beyond the buffer and reads zeros, so no load
    // sits under a branch.
    constexpr uint32_t OOB = 0x80000000u;
    const int dlo = d0 > 0 ? d0 - 1 : 0;
    const int dhi = min(d0 + TD + 1, D);
    const uint16_t* xbase = X + ((int64_t)n * D + dlo) * plane * Cin;
    const uint32_t xbytes = (uint32_t)((int64_t)(dhi - dlo) * plane * Cin * 2);
    uint32_t hoff[T::IT];
#pragma unroll
    for (int it = 0; it < T::IT; ++it) {
        const int e = threadIdx.x + it * T::NT;
        const int q = e & 3, hv = e >> 2;
        const int hw_ = hv % T::HW, hh_ = (hv / T::HW) % T::HH, hd_ = hv / (T::HW * T::HH);
        const int gd = d0 + hd_ - 1, gh = h0 + hh_ - 1, gw = w0 + hw_ - 1;
        const bool ok = (T::NE % T::NT == 0 || e < T::NE) && (unsigned)gd < (unsigned)D && (unsigned)gh < (unsigned)H &&
                        (unsigned)gw < (unsigned)W;
        uint32_t r = ok ? (((uint32_t)(gd - dlo) * (uint32_t)H + (uint32_t)gh) * (uint32_t)W + (uint32_t)gw) *
                              (uint32_t)(Cin * 2) + (uint32_t)q * 16u
                        : OOB;
        asm volatile("" : "+v"(r));     // a select, not a branch around the load
        hoff[it] = r;
    }
    for (int c = c_begin; c < c_end; ++c) {
        __syncthreads();
        // Stage the input halo of this 32-channel chunk (zero outside the
        // volume).  All of a thread's global loads are issued before any of
        // its LDS stores, so their latencies overlap instead of adding up.
        {
            const auto rx = buf_rsrc(xbase + c * 32, xbytes - (uint32_t)c * 64u);
            uint4 val[T::IT];
#pragma unroll
            for (int it = 0; it < T::IT; ++it)
                val[it] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, hoff[it], 0, 0));
#pragma unroll
            for (int it = 0; it < T::IT; ++it) {
                const int e = threadIdx.x + it * T::NT;
                if (T::NE % T::NT == 0 || e < T::NE)
                    *reinterpret_cast<uint4*>(halo + (e >> 2) * LS + halo_chunk(e & 3, (e >> 2) % T::HW) * 8) = val[it];
            }
        }
        __syncthreads();

        if constexpr (T::MINB >= 3) {
        // Register-lean pipeline for three waves per SIMD: weight (A)
        // fragments come from global memory two taps ahead; a tap's halo (B)
        // fragments are read from LDS at the start of the tap, and the other
        // waves on the SIMD cover their latency.
        const uint16_t* wrow = Wk + ((int64_t)(co_base + l16) * Cin + c * 32 + 8 * lg);
        const int64_t tap_stride = (int64_t)CoutPad * Cin;
        bf16x8 a0[T::MI], a1[T::MI], a2[T::MI], b0[T::NJ];
#pragma unroll
        for (int i = 0; i < T::MI; ++i) {
            a0[i] = *reinterpret_cast<const bf16x8*>(wrow + (int64_t)16 * i * Cin);
            a1[i] = *reinterpret_cast<const bf16x8*>(wrow + tap_stride + (int64_t)16 * i * Cin);
        }
#pragma unroll
        for (int tap = 0; tap < 27; ++tap) {
            if (tap + 2 < 27) {
#pragma unroll
                for (int i = 0; i < T::MI; ++i)
                    a2[i] = *reinterpret_cast<const bf16x8*>(wrow + (tap + 2) * tap_stride + (int64_t)16 * i * Cin);
            }
            const int toff = (((tap / 9) * T::HH + (tap / 3) % 3) * T::HW + tap % 3) * LS;
#pragma unroll
            for (int j = 0; j < T::NJ; ++j) b0[j] = *reinterpret_cast<const bf16x8*>(halo + (hb[j] + sw[tap % 3]) + toff);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < T::NJ; ++j)
#pragma unroll
                for (int i = 0; i < T::MI; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[i], b0[j], acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < T::MI; ++i) { a0[i] = a1[i]; a1[i] = a2[i]; }
        }
        } else {
        // Software pipeline over the 27 taps: weight (A) fragments are
        // loaded from global memory three taps ahead, halo (B) fragments are
        // read from LDS one tap ahead, so neither latency sits in front of
        // the MFMAs of the current tap.
        const uint16_t* wrow = Wk + ((int64_t)(co_base + l16) * Cin + c * 32 + 8 * lg);
        const int64_t tap_stride = (int64_t)CoutPad * Cin;
        bf16x8 a0[T::MI], a1[T::MI], a2[T::MI], a3[T::MI], b0[T::NJ], b1[T::NJ];
#pragma unroll
        for (int i = 0; i < T::MI; ++i) {
            a0[i] = *reinterpret_cast<const bf16x8*>(wrow + (int64_t)16 * i * Cin);
            a1[i] = *reinterpret_cast<const bf16x8*>(wrow + tap_stride + (int64_t)16 * i * Cin);
            a2[i] = *reinterpret_cast<const bf16x8*>(wrow + 2 * tap_stride + (int64_t)16 * i * Cin);
        }
#pragma unroll
        for (int j = 0; j < T::NJ; ++j) b0[j] = *reinterpret_cast<const bf16x8*>(halo + hb[j] + sw[0]);
#pragma unroll
        for (int tap = 0; tap < 27; ++tap) {
            if (tap + 3 < 27) {
#pragma unroll
                for (int i = 0; i < T::MI; ++i)
                    a3[i] = *reinterpret_cast<const bf16x8*>(wrow + (tap + 3) * tap_stride + (int64_t)16 * i * Cin);
            }
            if (tap + 1 < 27) {
                const int tn = tap + 1;
                const int toff = (((tn / 9) * T::HH + (tn / 3) % 3) * T::HW + tn % 3) * LS;
#pragma unroll
                for (int j = 0; j < T::NJ; ++j) b1[j] = *reinterpret_cast<const bf16x8*>(halo + (hb[j] + sw[tn % 3]) + toff);
            }
            // Fence: keep the prefetches above in front of this tap's MFMAs
            // (the scheduler would otherwise sink each load next to its use).
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < T::MI; ++i)
#pragma unroll
                for (int j = 0; j < T::NJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[i], b0[j], acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < T::MI; ++i) { a0[i] = a1[i]; a1[i] = a2[i]; a2[i] = a3[i]; }
#pragma unroll
            for (int j = 0; j < T::NJ; ++j) b0[j] = b1[j];
        }
        }
    }

    if constexpr (POOL) {
        static_assert(TW == 16 && WN == 2 * TH * TW && TD % 2 == 0 && TH % 2 == 0, "pooled epilogue mapping");
        static_assert(PoolTile<BM, TD, TH, TW>::SIZE <= T::HV * LS, "pooled tile fits in the halo's LDS");
        // every wave's last halo reads come before the tile overwrites them
        lds_barrier();
        // fragment j of this wave holds tile voxels (2 * wave + j / TH, j % TH, l16)
        pool_epilogue_lds<BM, TD, TH, TW, T::NT>(
            halo, acc, [&](int j) { return ((2 * wave + j / TH) * TH + j % TH) * TW + l16; }, wm * WM, lg, Y, pidx,
            slope, n, D, H, W, Cout, blockIdx.y * BM, d0, h0, w0);
        return;
    }

    // Epilogue: lane holds 4 consecutive output channels of one voxel per fragment.
    const int64_t nvox = (int64_t)N * D * plane;
#pragma unroll
    for (int j = 0; j < T::NJ; ++j) {
        const int v = wave * WN + 16 * j + l16;
        const int td = v / (TH * TW), th = (v / TW) % TH, tw = v % TW;
        const int gd = d0 + td, gh = h0 + th, gw = w0 + tw;
        if (gd >= D || gh >= H || gw >= W) continue;
        const int64_t gv = ((int64_t)n * D + gd) * plane + (int64_t)gh * W + gw;
#pragma unroll
        for (int i = 0; i < T::MI; ++i) {
            const int co = co_base + 16 * i + 4 * lg;
            if (co >= Cout) continue;
            const f32x4 r = acc[i][j];
            if (part) {
                float* dst = part + ((int64_t)blockIdx.z * nvox + gv) * Cout + co;
                *reinterpret_cast<float4*>(dst) = make_float4(r[0], r[1], r[2], r[3]);
            } else {
                uint2 pk = make_uint2(pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]));
                *reinterpret_cast<uint2*>(Y + gv * Cout + co) = pk;
            }
        }
    }
}

// kd-reuse variant of the same convolution.  The taps are walked as 9 (kh, kw)
// steps with the three kd taps inside each step, and a wave's fragments are
// whole depth columns of its h rows: fragment j covers tile depth j / JH and
// h rows (wave * JH + j % JH) * RPF .. + RPF - 1.  At step (kh, kw) the B
// operand of fragment j under tap kd is then the halo fragment that fragment
// j + JH * kd reads under tap 0, so a step reads (TD + 2) * JH B fragments
// for 3 * NJ fragment-taps (6 for 12 on a 4-deep, one-fragment-per-plane
// wave) instead of one per fragment-tap.  The operand reads per MFMA drop
// by about a third; the sums over the taps are taken in (kh, kw)-major,
// kd-minor order.
// The block's weight tiles of a step's three taps (BM rows x 32 channels
// each, row stride AS bf16) are loaded once into one of two 3-slot LDS groups
// (one group per step, alternating), from registers filled two steps ahead;
// a group is rewritten only after the barrier that ends the step which read
// it.  AS = 40 keeps the 32-channel block at 53.8 KB of LDS (three blocks per
// CU); the 64-channel blocks measured faster with AS = 48.
// POOL as in conv3d_mfma_kernel: a 2^3 window is the fragments (2 pd + a) *
// JH + b of one lane (a = d, b = h offset) and of its w-neighbour lane.
template <int BM, int WM, int WN, int TD, int TH, int TW, int LS, int AS, bool POOL = false>
__global__ __launch_bounds__((Tile<BM, WM, WN, TD, TH, TW, LS>::NT), (Tile<BM, WM, WN, TD, TH, TW, LS>::MINB))
void conv3d_mfma_kdr_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wk,
                            uint16_t* __restrict__ Y, float* __restrict__ part,
                            int N, int D, int H, int W, int Cin, int Cout, int CoutPad,
                            int tD, int tH, int tW, int chunks_per_split, uint8_t* __restrict__ pidx, float slope)
{
    using T = Tile<BM, WM, WN, TD, TH, TW, LS>;
    constexpr int RPF = 16 / TW;            // h rows per fragment
    constexpr int JH = T::NJ / TD;          // fragments per depth plane of a wave
    constexpr int RPW = JH * RPF;           // h rows of a wave
    constexpr int NB = (TD + 2) * JH;       // distinct B fragments per step
    static_assert(TW * RPF == 16 && T::NJ % TD == 0 && T::NWV * RPW == TH, "kd-reuse fragment layout");
    __shared__ __attribute__((aligned(16))) uint16_t halo[T::HV * LS];
    __shared__ __attribute__((aligned(16))) uint16_t aring[6 * BM * AS];
    static_assert(AS >= 32 && AS % 8 == 0, "weight ring");

    const int lane = threadIdx.x & 63;
    const int wm = (threadIdx.x >> 6) % T::NWM;
    const int wave = (threadIdx.x >> 6) / T::NWM;
    const int l16 = lane & 15, lg = lane >> 4;

    uint32_t tile = xcd_remap(blockIdx.x, gridDim.x);
    const int tw_ = tile % tW; tile /= tW;
    const int th_ = tile % tH; tile /= tH;
    const int td_ = tile % tD;
    const int n = tile / tD;
    const int d0 = td_ * TD, h0 = th_ * TH, w0 = tw_ * TW;
    const int co_base = blockIdx.y * BM + wm * WM;
    const int nchunks = Cin >> 5;
    const int c_begin = blockIdx.z * chunks_per_split;
    const int c_end = min(c_begin + chunks_per_split, nchunks);

    // lane part of the halo offset (depth plane 0, h-sub 0, tap 0); the
    // plane, h-sub and tap parts are compile-time immediates
    const int hbl = ((wave * RPW + l16 / TW) * T::HW + l16 % TW) * LS;
    int sw[3];
#pragma unroll
    for (int kw = 0; kw < 3; ++kw) sw[kw] = hbl + halo_chunk(lg, (l16 % TW) + kw) * 8;

    f32x4 acc[T::MI][T::NJ];
#pragma unroll
    for (int i = 0; i < T::MI; ++i)
#pragma unroll
        for (int j = 0; j < T::NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int64_t plane = (int64_t)H * W;
    const int64_t tap_stride = (int64_t)CoutPad * Cin;
    // Ring pieces: a step's three weight tiles are 3 * BM * 4 16-byte pieces,
    // spread over all threads (piece threadIdx.x + k * NT, k < PPT), so that
    // every wave takes a share of the ring stores before each step's barrier.
    constexpr int NPC = 3 * BM * 4, PPT = (NPC + T::NT - 1) / T::NT;
    uint32_t pl[PPT];                            // LDS offset of each piece in a group (bf16 units)
    // Every global load of this kernel is a raw buffer load at a 32-bit byte
    // offset computed once for all channel chunks; a piece outside the volume
    // (or a thread that loads nothing) gets an offset beyond the buffer, which
    // reads zeros.  Halo offsets are relative to the tile's first in-volume
    // depth plane (the host keeps (TD + 2) planes below 2^31 bytes); weight
    // offsets to the block's first row, with the tap in the scalar offset.
    constexpr uint32_t OOB = 0x80000000u;
    auto pick = [](bool ok, uint32_t off) {
        uint32_t r = ok ? off : OOB;
        asm volatile("" : "+v"(r));     // keeps the choice a select, not a branch around the load
        return r;
    };
    const int dlo = d0 > 0 ? d0 - 1 : 0;
    const int dhi = min(d0 + TD + 1, D);
    const uint16_t* xbase = X + ((int64_t)n * D + dlo) * plane * Cin;
    const uint32_t xbytes = (uint32_t)((int64_t)(dhi - dlo) * plane * Cin * 2);
    uint32_t hoff[T::IT];
#pragma unroll
    for (int it = 0; it < T::IT; ++it) {
        const int e = threadIdx.x + it * T::NT;
        const int q = e & 3, hv = e >> 2;
        const int hw_ = hv % T::HW, hh_ = (hv / T::HW) % T::HH, hd_ = hv / (T::HW * T::HH);
        const int gd = d0 + hd_ - 1, gh = h0 + hh_ - 1, gw = w0 + hw_ - 1;
        const bool ok = (T::NE % T::NT == 0 || e < T::NE) && (unsigned)gd < (unsigned)D && (unsigned)gh < (unsigned)H &&
                        (unsigned)gw < (unsigned)W;
        hoff[it] = pick(ok, (((uint32_t)(gd - dlo) * (uint32_t)H + (uint32_t)gh) * (uint32_t)W + (uint32_t)gw) *
                                (uint32_t)(Cin * 2) + (uint32_t)q * 16u);
    }
    const uint32_t wbytes = (uint32_t)(27 * tap_stride * 2);
    const uint16_t* wbase = Wk + (int64_t)blockIdx.y * BM * Cin;
    // global byte offset of each piece: its row and quarter, plus its tap
    // (kd * 9) in the weight copy; the step's tap (kh, kw) goes in the scalar offset
    uint32_t pg[PPT];
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
        const int pc = threadIdx.x + k * T::NT;
        const int kd = pc / (BM * 4), row = (pc >> 2) % BM, q = pc & 3;
        pl[k] = (uint32_t)(kd * BM * AS + row * AS + q * 8);
        pg[k] = pick(pc < NPC, ((uint32_t)row * (uint32_t)Cin + (uint32_t)q * 8u) * 2u +
                                   (uint32_t)(kd * 9) * (uint32_t)(tap_stride * 2));
    }
    auto wload = [&](int c, int k, int step) {
        const auto rw = buf_rsrc(wbase + c * 32, wbytes - (uint32_t)(blockIdx.y * BM * Cin + c * 32) * 2u);
        return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, pg[k], (int)(step * tap_stride * 2), 0));
    };
    auto pvalid = [&](int k) { return T::NT * (k + 1) <= NPC || (int)threadIdx.x + k * T::NT < NPC; };
    // The halo of chunk c + 1 is loaded into registers during chunk c and
    // stored when chunk c is done, so its latency hides behind chunk c's
    // MFMAs; past the last chunk the resource is empty and the loads read
    // zeros, so the loads are the same on every path.  64-channel blocks
    // issue the loads in chunk c's first step.  The 32-channel block, at its
    // register bound for three waves per SIMD, issues them in step 7 of 9:
    // the registers are then held for two steps only (162 VGPRs; held for
    // the whole chunk they cost more than the latency they hid).
    constexpr int PFS = BM == 64 ? 0 : 7;
    uint4 val[T::IT];
    auto hload = [&](int c, bool valid) {
        const auto rx = buf_rsrc(xbase + c * 32, valid ? xbytes - (uint32_t)c * 64u : 0u);
#pragma unroll
        for (int it = 0; it < T::IT; ++it)
            val[it] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rx, hoff[it], 0, 0));
    };
    hload(c_begin, true);
    for (int c = c_begin; c < c_end; ++c) {
        __syncthreads();
        uint4 ra[PPT];
        {
            // weight ring prologue: step 0's tiles go to group 0 with the
            // halo, step 1's are held in registers until step 0 stores them
            uint4 w0v[PPT];
#pragma unroll
            for (int k = 0; k < PPT; ++k) {
                w0v[k] = wload(c, k, 0);
                ra[k] = wload(c, k, 1);
            }
#pragma unroll
            for (int it = 0; it < T::IT; ++it) {
                const int e = threadIdx.x + it * T::NT;
                if (T::NE % T::NT == 0 || e < T::NE)
                    *reinterpret_cast<uint4*>(halo + (e >> 2) * LS + halo_chunk(e & 3, (e >> 2) % T::HW) * 8) = val[it];
            }
#pragma unroll
            for (int k = 0; k < PPT; ++k)
                if (pvalid(k)) *reinterpret_cast<uint4*>(aring + pl[k]) = w0v[k];
        }
        __syncthreads();

        int aoff[T::MI];
#pragma unroll
        for (int i = 0; i < T::MI; ++i) aoff[i] = (wm * WM + 16 * i + l16) * AS + 8 * lg;
        bf16x8 a[3][T::MI], b[NB];
#pragma unroll
        for (int s = 0; s < 9; ++s) {
            const int kh = s / 3, kw = s % 3;
            if (s == PFS) hload(c + 1, c + 1 < c_end);
            // ring loads two steps ahead, then this step's operands
            uint4 rn[PPT];
#pragma unroll
            for (int k = 0; k < PPT; ++k) rn[k] = s + 2 < 9 ? wload(c, k, s + 2) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
            for (int kd = 0; kd < 3; ++kd)
#pragma unroll
                for (int i = 0; i < T::MI; ++i)
                    a[kd][i] = *reinterpret_cast<const bf16x8*>(aring + ((s & 1) * 3 + kd) * BM * AS + aoff[i]);
#pragma unroll
            for (int p = 0; p < TD + 2; ++p)
#pragma unroll
                for (int hs = 0; hs < JH; ++hs)
                    b[p * JH + hs] = *reinterpret_cast<const bf16x8*>(
                        halo + sw[kw] + ((p * T::HH + hs * RPF + kh) * T::HW + kw) * LS);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kd = 0; kd < 3; ++kd)
#pragma unroll
                for (int i = 0; i < T::MI; ++i)
#pragma unroll
                    for (int j = 0; j < T::NJ; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[kd][i], b[j + kd * JH], acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            // the next step's tiles into the other group (last read in the
            // step before this one, behind its barrier)
            if (s + 1 < 9) {
#pragma unroll
                for (int k = 0; k < PPT; ++k)
                    if (pvalid(k)) *reinterpret_cast<uint4*>(aring + ((s + 1) & 1) * 3 * BM * AS + pl[k]) = ra[k];
            }
#pragma unroll
            for (int k = 0; k < PPT; ++k) ra[k] = rn[k];
            if (s + 1 < 9) lds_barrier();
        }
    }

    if constexpr (POOL) {
        static_assert(TW == 16 && JH == 2 && TD % 2 == 0 && RPF == 1, "pooled epilogue mapping");
        static_assert(PoolTile<BM, TD, TH, TW>::SIZE <= T::HV * LS, "pooled tile fits in the halo's LDS");
        lds_barrier();
        // fragment j of this wave holds tile voxels (j / JH, wave * JH + j % JH, l16)
        pool_epilogue_lds<BM, TD, TH, TW, T::NT>(
            halo, acc, [&](int j) { return ((j / JH) * TH + wave * JH + j % JH) * TW + l16; }, wm * WM, lg, Y, pidx,
            slope, n, D, H, W, Cout, blockIdx.y * BM, d0, h0, w0);
        return;
    }

    const int64_t nvox = (int64_t)N * D * plane;
#pragma unroll
    for (int j = 0; j < T::NJ; ++j) {
        const int td = j / JH, th = (wave * JH + j % JH) * RPF + l16 / TW, tw = l16 % TW;
        const int gd = d0 + td, gh = h0 + th, gw = w0 + tw;
        if (gd >= D || gh >= H || gw >= W) continue;
        const int64_t gv = ((int64_t)n * D + gd) * plane + (int64_t)gh * W + gw;
#pragma unroll
        for (int i = 0; i < T::MI; ++i) {
            const int co = co_base + 16 * i + 4 * lg;
            if (co >= Cout) continue;
            const f32x4 r = acc[i][j];
            if (part) {
                float* dst = part + ((int64_t)blockIdx.z * nvox + gv) * Cout + co;
                *reinterpret_cast<float4*>(dst) = make_float4(r[0], r[1], r[2], r[3]);
            } else {
                uint2 pk = make_uint2(pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]));
                *reinterpret_cast<uint2*>(Y + gv * Cout + co) = pk;
            }
        }
    }
}

// Sum the split partials in split order and round to bf16.
__global__ void split_reduce_bf16(const float* __restrict__ part, uint16_t* __restrict__ Y, int64_t n4,
                                  int splits)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        float4 s = reinterpret_cast<const float4*>(part)[i];
        for (int k = 1; k < splits; ++k) {
            const float4 p = reinterpret_cast<const float4*>(part)[(int64_t)k * n4 + i];
            s.x += p.x; s.y += p.y; s.z += p.z; s.w += p.w;
        }
        reinterpret_cast<uint2*>(Y)[i] = make_uint2(pack_bf16x2(s.x, s.y), pack_bf16x2(s.z, s.w));
    }
}

// The split partials summed and rounded as by split_reduce_bf16, then the
// leaky-ReLU + 2^3 max-pool of those bf16 values with the pool forward's rule
// (fp32 comparison, first strict maximum in window order, leaky ReLU on the
// maximum), so P and idx equal split_reduce_bf16 followed by the pool
// forward bit for bit, and the full-resolution conv output is never stored.
// Eight consecutive lanes take one (pooled voxel, 4 channels) item, lane q
// summing window position q = a*4 + b*2 + c.  The eight (value, position)
// pairs are combined in three butterfly steps, the right (later) pair taken
// only when it is valid and compares strictly greater (or the left one is
// not valid); position 0 is always valid, any other position only when it
// is not NaN.  That gives what the sequential scan gives: position 0's NaN
// if it is one, else the first occurrence of the maximum of the non-NaN
// values (a NaN after position 0 is never taken, ties keep the earlier one).
// D, H, W even, C % 4 == 0.
__global__ __launch_bounds__(256)
void split_reduce_pool_bf16(const float* __restrict__ part, uint16_t* __restrict__ P, uint8_t* __restrict__ idx,
                            int N, int D, int H, int W, int C, int splits, float slope)
{
    const int Dp = D / 2, Hp = H / 2, Wp = W / 2, cg = C / 4;
    const int64_t total = (int64_t)N * Dp * Hp * Wp * cg;
    const int64_t n4 = (int64_t)N * D * H * W * cg;   // float4 per split
    const float4* __restrict__ p4 = reinterpret_cast<const float4*>(part);
    const int q = threadIdx.x & 7;
    const int a = q >> 2, b = (q >> 1) & 1, c = q & 1;
    const int per_block = blockDim.x / 8;
    const int64_t stride = (int64_t)gridDim.x * per_block;
    // the trip count is the same for every lane of a block, so all lanes
    // reach the shuffles; an item's eight lanes are all in or all out
    for (int64_t e0 = (int64_t)blockIdx.x * per_block; e0 < total; e0 += stride) {
        const int64_t e = e0 + (threadIdx.x >> 3);
        const bool ok = e < total;
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        if (ok) {
            const int g = (int)(e % cg);
            int64_t r = e / cg;
            const int k = (int)(r % Wp); r /= Wp;
            const int j = (int)(r % Hp); r /= Hp;
            const int i = (int)(r % Dp);
            const int n = (int)(r / Dp);
            const int64_t vi = ((((int64_t)n * D + 2 * i + a) * H + 2 * j + b) * W + 2 * k + c) * cg + g;
            float4 sum = p4[vi];
            for (int sp = 1; sp < splits; ++sp) {
                const float4 t = p4[(int64_t)sp * n4 + vi];
                sum.x += t.x; sum.y += t.y; sum.z += t.z; sum.w += t.w;
            }
            const uint32_t lo = pack_bf16x2(sum.x, sum.y), hi = pack_bf16x2(sum.z, sum.w);
            v[0] = __uint_as_float(lo << 16); v[1] = __uint_as_float(lo & 0xffff0000u);
            v[2] = __uint_as_float(hi << 16); v[3] = __uint_as_float(hi & 0xffff0000u);
        }
        // per channel a nibble: position (3 bits) | valid << 3
        uint32_t meta = 0;
#pragma unroll
        for (int ch = 0; ch < 4; ++ch)
            meta |= ((uint32_t)q | ((q == 0 || v[ch] == v[ch]) ? 8u : 0u)) << (4 * ch);
#pragma unroll
        for (int m = 1; m < 8; m <<= 1) {
            const bool right = (q & m) != 0;   // this lane holds the later positions
            const uint32_t om = (uint32_t)__shfl_xor((int)meta, m, 8);
            uint32_t nm = 0;
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) {
                const float ov = __shfl_xor(v[ch], m, 8);
                const float lv = right ? ov : v[ch], rv = right ? v[ch] : ov;
                const uint32_t lm = ((right ? om : meta) >> (4 * ch)) & 15u, rm = ((right ? meta : om) >> (4 * ch)) & 15u;
                const bool take_r = (rm & 8u) && (!(lm & 8u) || rv > lv);
                v[ch] = take_r ? rv : lv;
                nm |= (take_r ? rm : lm) << (4 * ch);
            }
            meta = nm;
        }
        if (ok && q == 0) {
            float o[4];
#pragma unroll
            for (int ch = 0; ch < 4; ++ch) o[ch] = v[ch] > 0.f ? v[ch] : slope * v[ch];
            reinterpret_cast<uint2*>(P)[e] = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
            reinterpret_cast<uint32_t*>(idx)[e] = (meta & 7u) | ((meta >> 4) & 7u) << 8 | ((meta >> 8) & 7u) << 16 |
                                                  ((meta >> 12) & 7u) << 24;
        }
    }
}

// The split partials of a pooled-resolution gradient dP summed and rounded
// as by split_reduce_bf16, then the pool backward applied to it as the pool
// backward kernel does (dZ at the recorded window position = dP, times the
// slope where the pooled value P is not positive; the other seven positions
// zero; dZ written densely), so dZ equals split_reduce_bf16 followed by the
// pool backward bit for bit and dP is never stored.  One thread per (pooled
// voxel, 4 channels).  Dp, Hp, Wp: the pooled (partials') shape; dZ is
// 2Dp x 2Hp x 2Wp; C % 4 == 0.
__global__ __launch_bounds__(256)
void split_reduce_unpool_bf16(const float* __restrict__ part, const uint16_t* __restrict__ P,
                              const uint8_t* __restrict__ idx, uint16_t* __restrict__ dZ, int N, int Dp, int Hp, int Wp,
                              int C, int splits, float slope)
{
    const int cg = C / 4, D = 2 * Dp, H = 2 * Hp, W = 2 * Wp;
    const int64_t n4 = (int64_t)N * Dp * Hp * Wp * cg;   // float4 per split = items
    const float4* __restrict__ p4 = reinterpret_cast<const float4*>(part);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n4; e += stride) {
        float4 sum = p4[e];
        for (int sp = 1; sp < splits; ++sp) {
            const float4 t = p4[(int64_t)sp * n4 + e];
            sum.x += t.x; sum.y += t.y; sum.z += t.z; sum.w += t.w;
        }
        const uint32_t lo = pack_bf16x2(sum.x, sum.y), hi = pack_bf16x2(sum.z, sum.w);
        float gv[4] = {__uint_as_float(lo << 16), __uint_as_float(lo & 0xffff0000u), __uint_as_float(hi << 16),
                       __uint_as_float(hi & 0xffff0000u)};
        const uint2 pp = reinterpret_cast<const uint2*>(P)[e];
        const float pv[4] = {__uint_as_float(pp.x << 16), __uint_as_float(pp.x & 0xffff0000u),
                             __uint_as_float(pp.y << 16), __uint_as_float(pp.y & 0xffff0000u)};
        const uint32_t ib = reinterpret_cast<const uint32_t*>(idx)[e];
#pragma unroll
        for (int c = 0; c < 4; ++c) gv[c] = pv[c] > 0.f ? gv[c] : slope * gv[c];
        const int g = (int)(e % cg);
        int64_t r = e / cg;
        const int k = (int)(r % Wp); r /= Wp;
        const int j = (int)(r % Hp); r /= Hp;
        const int i = (int)(r % Dp);
        const int n = (int)(r / Dp);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int a = q >> 2, b = (q >> 1) & 1, c2 = q & 1;
            float o[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) o[c] = ((ib >> (8 * c)) & 0xffu) == (uint32_t)q ? gv[c] : 0.f;
            const int64_t vox = (((int64_t)n * D + 2 * i + a) * H + 2 * j + b) * W + 2 * k + c2;
            reinterpret_cast<uint2*>(dZ)[vox * cg + g] = make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
        }
    }
}

template <int BM, int WM, int WN, int TD, int TH, int TW, int LS, int AS, bool POOL = false>
hipError_t launch_kdr(const uint16_t* X, const uint16_t* Wk, uint16_t* Y, float* part, const cf_dims& x, int cout,
                      int coutpad, int splits, hipStream_t s, uint8_t* pidx = nullptr, float slope = 0.f)
{
    using T = Tile<BM, WM, WN, TD, TH, TW, LS>;
    // the kernel's 32-bit buffer offsets: a tile's TD + 2 input planes and
    // the weight copy must stay below 2^31 bytes
    if ((int64_t)(TD + 2) * x.h * x.w * x.c * 2 >= ((int64_t)1 << 31) ||
        (int64_t)27 * coutpad * x.c * 2 >= ((int64_t)1 << 31))
        return hipErrorInvalidValue;
    const int tD = (int)((x.d + TD - 1) / TD), tH = (int)((x.h + TH - 1) / TH), tW = (int)((x.w + TW - 1) / TW);
    const int nchunks = (int)(x.c / 32);
    const int cps = (nchunks + splits - 1) / splits;
    dim3 grid((unsigned)(x.n * tD * tH * tW), (unsigned)((cout + BM - 1) / BM), (unsigned)splits);
    hipLaunchKernelGGL((conv3d_mfma_kdr_kernel<BM, WM, WN, TD, TH, TW, LS, AS, POOL>), grid, dim3(T::NT), 0, s,
                       X, Wk, Y, splits > 1 ? part : nullptr, (int)x.n, (int)x.d, (int)x.h, (int)x.w, (int)x.c, cout,
                       coutpad, tD, tH, tW, cps, pidx, slope);
    return hipGetLastError();
}

struct CfgInfo { int bm, wm, wn, td, th, tw, ls; };
constexpr CfgInfo kCfgs[] = {
    {64, 32, 128, 4, 4, 16, 32},    // 0
    {64, 32, 128, 4, 8, 8, 32},     // 1
    {32, 32, 64, 4, 8, 8, 32},      // 2
    {16, 16, 64, 4, 4, 16, 32},     // 3
    {16, 16, 64, 4, 8, 8, 32},      // 4
};

template <int BM, int WM, int WN, int TD, int TH, int TW, int LS, int WPE_ = 0, bool POOL = false>
hipError_t launch_cfg(const uint16_t* X, const uint16_t* Wk, uint16_t* Y, float* part, const cf_dims& x,
                      int cout, int coutpad, int splits, hipStream_t s, uint8_t* pidx = nullptr, float slope = 0.f)
{
    using T = Tile<BM, WM, WN, TD, TH, TW, LS, WPE_>;
    const int tD = (int)((x.d + TD - 1) / TD), tH = (int)((x.h + TH - 1) / TH), tW = (int)((x.w + TW - 1) / TW);
    const int nchunks = (int)(x.c / 32);
    const int cps = (nchunks + splits - 1) / splits;
    dim3 grid((unsigned)(x.n * tD * tH * tW), (unsigned)((cout + BM - 1) / BM), (unsigned)splits);
    hipLaunchKernelGGL((conv3d_mfma_kernel<BM, WM, WN, TD, TH, TW, LS, WPE_, POOL>), grid, dim3(T::NT), 0, s, X, Wk,
                       Y, splits > 1 ? part : nullptr, (int)x.n, (int)x.d, (int)x.h, (int)x.w, (int)x.c, cout,
                       coutpad, tD, tH, tW, cps, pidx, slope);
    return hipGetLastError();
}

}  // namespace

ConvPlan plan_conv_mfma(const cf_dims& x, int cout)
{
    // 64-channel 4-wave blocks for every output width above 32: two of them
    // share a CU and hide each other's halo staging, which measured faster
    // than 128-channel 8-wave blocks (one per CU) at every layer shape.
    ConvPlan p{};
    const bool narrow = x.w < 16;
    if (cout > 32) p.cfg = narrow ? 1 : 0;
    // 17..32 channels: the 4x8x8 tile (its halo takes the bank swizzle; the
    // 4x8x16 tile is at the register limit without it) measured faster
    else if (cout > 16) p.cfg = 2;
    else p.cfg = narrow ? 4 : 3;
    const CfgInfo& c = kCfgs[p.cfg];
    p.bm = c.bm;
    const int64_t tiles = x.n * ((x.d + c.td - 1) / c.td) * ((x.h + c.th - 1) / c.th) * ((x.w + c.tw - 1) / c.tw);
    const int64_t blocks = tiles * ((cout + c.bm - 1) / c.bm);
    const int nchunks = (int)(x.c / 32);
    // split the channel reduction only while the grid has fewer than two
    // blocks per CU (the split costs fp32 partials and a reduction launch)
    int splits = 1;
    if (blocks < 512 && nchunks > 1) {
        splits = (int)((512 + blocks - 1) / blocks);
        if (splits > nchunks) splits = nchunks;
        // equalise chunk counts per split
        const int cps = (nchunks + splits - 1) / splits;
        splits = (nchunks + cps - 1) / cps;
    }
    p.splits = splits;
    // The weight ring (conv3d_mfma_kdr_kernel) loads each tap's weights once
    // per block instead of once per wave, six taps ahead; it pays off where
    // four waves share a 32-channel slice, where a block walks several
    // channel chunks, and on the narrow (8-wide) tiles of the small late
    // layers, whose per-wave weight loads three taps ahead left their few
    // waves waiting on L2 (8^3 x 256 -> 256: 0.046 -> 0.042 ms).  A
    // single-chunk 64-channel block on a 16-wide tile is faster with per-wave
    // weight loads and three waves per SIMD (conv3d_mfma_kernel).  The
    // 16-channel tiles always take per-wave loads.
    const int cps = (nchunks + splits - 1) / splits;
    p.ring = p.cfg <= 2 && !(p.cfg == 0 && cps == 1);
    p.part_bytes = splits > 1 ? (size_t)splits * (size_t)(x.n * x.d * x.h * x.w) * (size_t)cout * sizeof(float) : 0;
    return p;
}

namespace {

// The plan's conv kernel alone: with a split, the fp32 partials go to part
// ([splits][voxels][cout]) for one of the two reductions below.
hipError_t launch_conv_mfma_kernel(const ConvPlan& p, const uint16_t* X, const uint16_t* Wk, uint16_t* Y, float* part,
                                   const cf_dims& x, int cout, int coutpad, hipStream_t s)
{
    hipError_t e;
    if (p.ring) {
        switch (p.cfg) {
        case 0: e = launch_kdr<64, 32, 128, 4, 4, 16, 32, 48>(X, Wk, Y, part, x, cout, coutpad, p.splits, s); break;
        case 1: e = launch_kdr<64, 32, 128, 4, 8, 8, 32, 48>(X, Wk, Y, part, x, cout, coutpad, p.splits, s); break;
        case 2: e = launch_kdr<32, 32, 64, 4, 8, 8, 32, 40>(X, Wk, Y, part, x, cout, coutpad, p.splits, s); break;
        default: return hipErrorInvalidValue;
        }
    } else {
        switch (p.cfg) {
        case 0: e = launch_cfg<64, 32, 128, 4, 4, 16, 32, 3>(X, Wk, Y, part, x, cout, coutpad, p.splits, s); break;
        case 3: e = launch_cfg<16, 16, 64, 4, 4, 16, 32>(X, Wk, Y, part, x, cout, coutpad, p.splits, s); break;
        case 4: e = launch_cfg<16, 16, 64, 4, 8, 8, 32>(X, Wk, Y, part, x, cout, coutpad, p.splits, s); break;
        default: return hipErrorInvalidValue;
        }
    }
    return e;
}

}  // namespace

hipError_t launch_conv_mfma(const ConvPlan& p, const uint16_t* X, const uint16_t* Wk, uint16_t* Y, float* part,
                            const cf_dims& x, int cout, int coutpad, hipStream_t s)
{
    const hipError_t e = launch_conv_mfma_kernel(p, X, Wk, Y, part, x, cout, coutpad, s);
    if (e != hipSuccess || p.splits == 1) return e;
    const int64_t n4 = x.n * x.d * x.h * x.w * (int64_t)cout / 4;
    int64_t blocks = (n4 + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(split_reduce_bf16, dim3((unsigned)blocks), dim3(256), 0, s, part, Y, n4, p.splits);
    return hipGetLastError();
}

// Only split plans apply the pool backward of the layer below (in the
// reduction of their partials).  An epilogue doing the same in the unsplit
// weight-ring kernel writes eight 8-byte stores per accumulator and waits on
// the pooled values and indices at the end of the kernel; in the 128^3 step
// it measured slower than that kernel plus the separate pool backward.
bool conv_mfma_can_unpool(const ConvPlan& p) { return p.splits > 1; }

hipError_t launch_conv_mfma_unpool(const ConvPlan& p, const uint16_t* X, const uint16_t* Wk, float* part,
                                   const uint16_t* P, const uint8_t* idx, uint16_t* dZ, float slope, const cf_dims& x,
                                   int cout, int coutpad, hipStream_t s)
{
    if (cout % 4 != 0 || !conv_mfma_can_unpool(p)) return hipErrorInvalidValue;
    if (!part) return hipErrorInvalidValue;
    const hipError_t e = launch_conv_mfma_kernel(p, X, Wk, nullptr, part, x, cout, coutpad, s);
    if (e != hipSuccess) return e;
    const int64_t n4 = x.n * x.d * x.h * x.w * (int64_t)cout / 4;
    int64_t blocks = (n4 + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(split_reduce_unpool_bf16, dim3((unsigned)blocks), dim3(256), 0, s, part, P, idx, dZ, (int)x.n,
                       (int)x.d, (int)x.h, (int)x.w, cout, p.splits, slope);
    return hipGetLastError();
}

// Unsplit 4x4x16-tile plans pool in the conv kernel's epilogue (same kernel
// and tap order as the plain launch); split plans pool in the reduction of
// their partials (same summation order as split_reduce_bf16).  Either way
// the fused result equals conv then pool bit for bit.
bool conv_mfma_can_pool(const ConvPlan& p, const cf_dims& x)
{
    return (p.splits > 1 || p.cfg == 0) && (x.d % 2 == 0) && (x.h % 2 == 0) && (x.w % 2 == 0);
}

hipError_t launch_conv_mfma_pool(const ConvPlan& p, const uint16_t* X, const uint16_t* Wk, uint16_t* P, uint8_t* idx,
                                 float slope, const cf_dims& x, int cout, int coutpad, float* part, hipStream_t s)
{
    if (!conv_mfma_can_pool(p, x)) return hipErrorInvalidValue;
    if (p.splits > 1) {
        if (!part) return hipErrorInvalidValue;
        const hipError_t e = launch_conv_mfma_kernel(p, X, Wk, nullptr, part, x, cout, coutpad, s);
        if (e != hipSuccess) return e;
        const int64_t total = x.n * (x.d / 2) * (x.h / 2) * (x.w / 2) * (int64_t)cout / 4;   // 8 lanes each
        int64_t blocks = (total + 31) / 32;
        if (blocks > 65536) blocks = 65536;
        hipLaunchKernelGGL(split_reduce_pool_bf16, dim3((unsigned)blocks), dim3(256), 0, s, part, P, idx, (int)x.n,
                           (int)x.d, (int)x.h, (int)x.w, cout, p.splits, slope);
        return hipGetLastError();
    }
    if (p.ring)
        return launch_kdr<64, 32, 128, 4, 4, 16, 32, 48, true>(X, Wk, P, nullptr, x, cout, coutpad, 1, s, idx, slope);
    return launch_cfg<64, 32, 128, 4, 4, 16, 32, 3, true>(X, Wk, P, nullptr, x, cout, coutpad, 1, s, idx, slope);
}

}  // namespace cf
