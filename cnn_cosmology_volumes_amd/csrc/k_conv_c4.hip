// First-layer 3^3 convolution forward for 4 input channels on bf16 MFMA.
//
// Same definition as the general forward (Oyama et al., Sec. IV / Table I:
// stride 1, "same" zero padding, no bias), specialised for the 4-channel
// input volume: the reduction K = 27 taps x 4 channels = 108 is packed into
// 32 tap slots x 4 channels = 128 (four 32-deep MFMA steps) in the order of
// c4_slot_tap.  A lane's 8 K-values are two taps x 4 channels, i.e. two
// 8-byte LDS reads from an [halo voxel][4] tile; the slot order makes the
// second tap a fixed offset from the first within each step, so both reads
// use one base register with immediate offsets and land in the operand's
// registers directly.  The halo is cheap (8 bytes per voxel) and the tile
// large.
#include "cf_internal.h"

namespace cf {

namespace {

constexpr int TD = 4, TH = 8, TW = 16, WN = 128;
constexpr int VT = TD * TH * TW, NW = VT / WN, NT = NW * 64;
constexpr int HD = TD + 2, HH = TH + 2, HW = TW + 2, HV = HD * HH * HW;

// POOL = false: writes Y (the conv output).
// POOL = true : rounds the tile to bf16 in LDS and writes only the leaky-ReLU
//               + 2^3 max-pooled P and its window index (the same values the
//               unfused conv -> pool pair produces), so the full-resolution
//               conv output never goes to HBM.
constexpr int ZS = 40;          // bf16 per voxel row of the pooled-epilogue tile (80 B)

// q = x / d for the tile decode, on uniform values: the divisor's magic
// numbers come from the host (make_fastdiv), so the decode is scalar
// multiplies instead of a per-wave integer division; exact for every 32-bit x.
struct FastDiv { uint32_t d, m, s; };
__device__ __forceinline__ uint32_t fdiv(uint32_t x, const FastDiv& f)
{
    return (uint32_t)(((uint64_t)__umulhi(x, f.m) + x) >> f.s);
}
FastDiv make_fastdiv(uint32_t d)
{
    uint32_t s = 0;
    while ((1ull << s) < d) ++s;
    return FastDiv{d, (uint32_t)(((1ull << 32) * ((1ull << s) - d)) / d + 1), s};
}

template <int BM, bool POOL>
__global__ __launch_bounds__(NT)
void conv3d_c4_fwd_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wk,
                          uint16_t* __restrict__ Y, uint8_t* __restrict__ idx, float slope,
                          int N, int D, int H, int W, int Cout, FastDiv ftD, FastDiv ftH, FastDiv ftW)
{
    constexpr int MI = BM / 16, NJ = WN / 16;
    // Halo: 4 bf16 per voxel, plus one zero voxel past the end (read, with
    // zero weight, as the padded partner of the last tap).  The pooled
    // epilogue's bf16 tile reuses the same LDS once every wave has finished
    // reading the halo, which keeps a block at 40 KB (four blocks per CU).
    constexpr int HALO_BYTES = (HV + 1) * 8, ZT_BYTES = POOL ? VT * ZS * 2 : 0;
    __shared__ __attribute__((aligned(16))) uint8_t lds[HALO_BYTES > ZT_BYTES ? HALO_BYTES : ZT_BYTES];
    uint2* const halo = reinterpret_cast<uint2*>(lds);
    uint16_t* const zt = reinterpret_cast<uint16_t*>(lds);

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    uint32_t tile = xcd_remap(blockIdx.x, gridDim.x);
    uint32_t q = fdiv(tile, ftW);
    const int tw_ = (int)(tile - q * ftW.d);
    tile = q;
    q = fdiv(tile, ftH);
    const int th_ = (int)(tile - q * ftH.d);
    tile = q;
    q = fdiv(tile, ftD);
    const int td_ = (int)(tile - q * ftD.d);
    const int n = (int)q;
    const int d0 = td_ * TD, h0 = th_ * TH, w0 = tw_ * TW;
    const int co_base = blockIdx.y * BM;
    const int64_t plane = (int64_t)H * W;

    // All weight fragments of this block (K = 128 is four MFMA steps) are
    // loaded up front so their latency overlaps the halo staging.
    bf16x8 afr[4][MI];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < MI; ++i)
            afr[s][i] = *reinterpret_cast<const bf16x8*>(Wk + (int64_t)(co_base + 16 * i + l16) * 128 + 32 * s + 8 * lg);

    // Halo staging: a thread owns one halo column w and every RS-th halo
    // row (d, h) from its first, so the column's bounds and offset are
    // computed once; the loads are raw buffer loads at 32-bit byte offsets
    // from the sample (the host keeps a sample below 2^31 bytes), and a voxel
    // outside the volume gets an offset beyond the buffer, which reads zeros.
    // Every global load of this thread is issued before its LDS stores, so
    // the load latencies overlap.
    {
        constexpr int NR = HD * HH, RS = NT / HW, IT = (NR + RS - 1) / RS;
        const int cw = threadIdx.x % HW, rr = threadIdx.x / HW;
        const int gw = w0 + cw - 1;
        const bool col_ok = rr < RS && (unsigned)gw < (unsigned)W;
        const auto rx = buf_rsrc(X + (int64_t)n * D * plane * 4, (uint32_t)((int64_t)D * plane * 8));
        uint2 v[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int r = rr + it * RS;
            const int gd = d0 + r / HH - 1, gh = h0 + r % HH - 1;
            // 24-bit multiplies: the host keeps (D + 2)(H + 2) and W below 2^24
            // (an out-of-volume gd or gh gives garbage that the select drops)
            uint32_t off = (__umul24(__umul24((uint32_t)gd, (uint32_t)H) + (uint32_t)gh, (uint32_t)W) + (uint32_t)gw) * 8u;
            off = (col_ok && r < NR && (unsigned)gd < (unsigned)D && (unsigned)gh < (unsigned)H) ? off : 0x80000000u;
            asm volatile("" : "+v"(off));     // a select, not a branch around the load
            v[it] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rx, off, 0, 0));
        }
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int r = rr + it * RS;
            if (rr < RS && r < NR) halo[r * HW + cw] = v[it];
        }
        if (threadIdx.x == 0) halo[HV] = make_uint2(0u, 0u);
    }
    __syncthreads();

    // A wave owns one depth plane of the tile: fragment j is row th = j, lane
    // l16 is tw, so fragment j's halo voxel is hb0 + j * HW.
    static_assert(WN == TH * TW && NJ == TH, "one depth plane per wave");
    const int hb0 = wave * HH * HW + l16;

    f32x4 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // halo voxel offset of a tap (an empty slot reads tap 0's voxel)
    auto voff = [](int t) { return t < 0 ? 0 : ((t / 9) * HH + (t / 3) % 3) * HW + t % 3; };
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const bf16x8* a = afr[s];
        // This lane group's first tap at this step, and the offset of the
        // second tap (the same for every lane group of the step).  A zero
        // slot has zero weights, so the finite halo value it reads (a
        // neighbouring voxel, or the zero voxel past the end) adds nothing.
        // (the four lane groups' offsets packed 16 bits each and picked by a
        // shift, which stays free of branches)
        const uint64_t tab = (uint64_t)voff(c4_slot_tap(8 * s)) | (uint64_t)voff(c4_slot_tap(8 * s + 2)) << 16 |
                             (uint64_t)voff(c4_slot_tap(8 * s + 4)) << 32 | (uint64_t)voff(c4_slot_tap(8 * s + 6)) << 48;
        const int ta = (int)((tab >> (16 * lg)) & 0xffffu);
        const int dt = s == 2 ? HW : 1;
        const uint2* hp = halo + hb0 + ta;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const uint2 u0 = hp[j * HW];
            const uint2 u1 = hp[j * HW + dt];
            const uint4 u = make_uint4(u0.x, u0.y, u1.x, u1.y);
            const bf16x8 b = __builtin_bit_cast(bf16x8, u);
#pragma unroll
            for (int i = 0; i < MI; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b, acc[i][j], 0, 0, 0);
        }
    }

    if (!POOL) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int v = wave * WN + 16 * j + l16;
            const int td = v / (TH * TW), th = (v / TW) % TH, tw = v % TW;
            const int gd = d0 + td, gh = h0 + th, gw = w0 + tw;
            if (gd >= D || gh >= H || gw >= W) continue;
            const int64_t gv = ((int64_t)n * D + gd) * plane + (int64_t)gh * W + gw;
#pragma unroll
            for (int i = 0; i < MI; ++i) {
                const int co = co_base + 16 * i + 4 * lg;
                if (co >= Cout) continue;
                const f32x4 r = acc[i][j];
                *reinterpret_cast<uint2*>(Y + gv * Cout + co) =
                    make_uint2(pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]));
            }
        }
        return;
    }
    // Pooled epilogue: bf16 tile in LDS, then one thread per (pooled voxel,
    // 8-channel group) takes the window maximum (first strict maximum in
    // window order), applies leaky ReLU to it and stores P and idx.  The
    // tile overwrites the halo, so every wave's halo reads come first.
    lds_barrier();
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int v = wave * WN + 16 * j + l16;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
            const f32x4 r = acc[i][j];
            *reinterpret_cast<uint2*>(&zt[v * ZS + 16 * i + 4 * lg]) =
                make_uint2(pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3]));
        }
    }
    __syncthreads();
    constexpr int PD = TD / 2, PH = TH / 2, PW = TW / 2, NG = BM / 8;
    const int Dp = D / 2, Hp = H / 2, Wp = W / 2;
    for (int e = threadIdx.x; e < PD * PH * PW * NG; e += NT) {
        const int g = e % NG, pv = e / NG;
        const int pk = pv % PW, pj = (pv / PW) % PH, pi = pv / (PW * PH);
        const int gpd = d0 / 2 + pi, gph = h0 / 2 + pj, gpw = w0 / 2 + pk;
        const int co = co_base + 8 * g;
        if (gpd >= Dp || gph >= Hp || gpw >= Wp || co >= Cout) continue;
        float best[8];
        uint32_t bi[8];
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int a = p >> 2, b = (p >> 1) & 1, c = p & 1;
            const int v = ((2 * pi + a) * TH + 2 * pj + b) * TW + 2 * pk + c;
            const uint4 u = *reinterpret_cast<const uint4*>(&zt[v * ZS + 8 * g]);
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
        // the sample's pooled outputs start at a scalar 64-bit offset; within
        // a sample 32 bits suffice (the host keeps a sample's P below 2^31
        // bytes), with 24-bit multiplies as for the halo
        const int64_t obase = (int64_t)n * Dp * Hp * Wp * Cout;
        const uint32_t o = __umul24(__umul24(__umul24((uint32_t)gpd, (uint32_t)Hp) + (uint32_t)gph, (uint32_t)Wp) +
                                    (uint32_t)gpw, (uint32_t)Cout) + (uint32_t)co;
        *reinterpret_cast<uint4*>(Y + obase + o) = make_uint4(pack_bf16x2(out[0], out[1]), pack_bf16x2(out[2], out[3]),
                                                              pack_bf16x2(out[4], out[5]), pack_bf16x2(out[6], out[7]));
        *reinterpret_cast<uint2*>(idx + obase + o) = make_uint2(bi[0] | (bi[1] << 8) | (bi[2] << 16) | (bi[3] << 24),
                                                                bi[4] | (bi[5] << 8) | (bi[6] << 16) | (bi[7] << 24));
    }
}

}  // namespace

// The kernel addresses a sample's input with 32-bit byte offsets built from
// 24-bit multiplies, and (pooled) a sample's P with 32-bit offsets.
bool conv_c4_fits(const cf_dims& x)
{
    return x.d * x.h * x.w * 8 < ((int64_t)1 << 31) && (x.d + 2) * (x.h + 2) < ((int64_t)1 << 24) &&
           x.w < ((int64_t)1 << 24);
}

bool conv_c4_pool_fits(const cf_dims& x, int cout)
{
    return conv_c4_fits(x) && (x.d / 2) * (x.h / 2) * (x.w / 2) * (int64_t)cout * 2 < ((int64_t)1 << 31);
}

namespace {
dim3 c4_grid(const cf_dims& x, int bm, int cout, FastDiv& fd, FastDiv& fh, FastDiv& fw)
{
    const int64_t tD = (x.d + TD - 1) / TD, tH = (x.h + TH - 1) / TH, tW = (x.w + TW - 1) / TW;
    fd = make_fastdiv((uint32_t)tD);
    fh = make_fastdiv((uint32_t)tH);
    fw = make_fastdiv((uint32_t)tW);
    return dim3((unsigned)(x.n * tD * tH * tW), (unsigned)((cout + bm - 1) / bm));
}
}  // namespace

hipError_t launch_conv_c4_fwd(const uint16_t* X, const uint16_t* Wk, uint16_t* Y, const cf_dims& x, int cout,
                              int copad, hipStream_t s)
{
    (void)copad;
    if (!conv_c4_fits(x)) return hipErrorInvalidValue;
    FastDiv fd, fh, fw;
    if (cout <= 16) {
        const dim3 g = c4_grid(x, 16, cout, fd, fh, fw);
        hipLaunchKernelGGL((conv3d_c4_fwd_kernel<16, false>), g, dim3(NT), 0, s, X, Wk, Y, nullptr, 0.f, (int)x.n,
                           (int)x.d, (int)x.h, (int)x.w, cout, fd, fh, fw);
    } else {
        const dim3 g = c4_grid(x, 32, cout, fd, fh, fw);
        hipLaunchKernelGGL((conv3d_c4_fwd_kernel<32, false>), g, dim3(NT), 0, s, X, Wk, Y, nullptr, 0.f, (int)x.n,
                           (int)x.d, (int)x.h, (int)x.w, cout, fd, fh, fw);
    }
    return hipGetLastError();
}

hipError_t launch_conv_c4_pool_fwd(const uint16_t* X, const uint16_t* Wk, uint16_t* P, uint8_t* idx, float slope,
                                   const cf_dims& x, int cout, hipStream_t s)
{
    if (!conv_c4_pool_fits(x, cout)) return hipErrorInvalidValue;
    FastDiv fd, fh, fw;
    const dim3 g = c4_grid(x, 32, cout, fd, fh, fw);
    hipLaunchKernelGGL((conv3d_c4_fwd_kernel<32, true>), g, dim3(NT), 0, s, X, Wk, P, idx, slope, (int)x.n, (int)x.d,
                       (int)x.h, (int)x.w, cout, fd, fh, fw);
    return hipGetLastError();
}

}  // namespace cf
