// First-layer 3^3 convolution forward for 4 input channels on bf16 MFMA.
//
// Same definition as the general forward (Oyama et al., Sec. IV / Table I:
// stride 1, "same" zero padding, no bias), specialised for the 4-channel
// input volume: the reduction K = 27 taps x 4 channels = 108 is packed as
// k = tap*4 + ci and padded with zero taps to 128 (four 32-deep MFMA steps).
// A lane's 8 K-values are then two taps x 4 channels, i.e. two 8-byte LDS
// reads from an [halo voxel][4] tile.  This layer is bound by HBM bandwidth
// (it writes 32 output channels per voxel while reading 4), so the tile is
// large and the halo cheap: 8 bytes per voxel.
#include "cf_internal.h"

namespace cf {

namespace {

constexpr int TD = 4, TH = 8, TW = 16, WN = 128;
constexpr int VT = TD * TH * TW, NW = VT / WN, NT = NW * 64;
constexpr int HD = TD + 2, HH = TH + 2, HW = TW + 2, HV = HD * HH * HW;

template <int BM>
__global__ __launch_bounds__(NT)
void conv3d_c4_fwd_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wk,
                          uint16_t* __restrict__ Y, int N, int D, int H, int W, int Cout,
                          int tD, int tH, int tW)
{
    constexpr int MI = BM / 16, NJ = WN / 16;
    __shared__ __attribute__((aligned(16))) uint2 halo[HV];   // 4 bf16 per voxel

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    uint32_t tile = xcd_remap(blockIdx.x, gridDim.x);
    const int tw_ = tile % tW; tile /= tW;
    const int th_ = tile % tH; tile /= tH;
    const int td_ = tile % tD;
    const int n = tile / tD;
    const int d0 = td_ * TD, h0 = th_ * TH, w0 = tw_ * TW;
    const int co_base = blockIdx.y * BM;
    const int64_t plane = (int64_t)H * W;

    for (int hv = threadIdx.x; hv < HV; hv += NT) {
        const int hw_ = hv % HW, hh_ = (hv / HW) % HH, hd_ = hv / (HW * HH);
        const int gd = d0 + hd_ - 1, gh = h0 + hh_ - 1, gw = w0 + hw_ - 1;
        uint2 v = make_uint2(0u, 0u);
        if ((unsigned)gd < (unsigned)D && (unsigned)gh < (unsigned)H && (unsigned)gw < (unsigned)W)
            v = *reinterpret_cast<const uint2*>(X + (((int64_t)n * D + gd) * plane + (int64_t)gh * W + gw) * 4);
        halo[hv] = v;
    }
    __syncthreads();

    int hb[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int v = wave * WN + 16 * j + l16;
        const int td = v / (TH * TW), th = (v / TW) % TH, tw = v % TW;
        hb[j] = (td * HH + th) * HW + tw;
    }

    f32x4 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int s = 0; s < 4; ++s) {
        bf16x8 a[MI];
#pragma unroll
        for (int i = 0; i < MI; ++i)
            a[i] = *reinterpret_cast<const bf16x8*>(Wk + (int64_t)(co_base + 16 * i + l16) * 128 + 32 * s + 8 * lg);
        // taps covered by this lane group at this step
        const int t0 = 8 * s + 2 * lg, t1 = t0 + 1;
        const int off0 = ((t0 / 9) * HH + (t0 / 3) % 3) * HW + t0 % 3;
        const int off1 = ((t1 / 9) * HH + (t1 / 3) % 3) * HW + t1 % 3;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            uint2 u0 = make_uint2(0u, 0u), u1 = make_uint2(0u, 0u);
            if (t0 < 27) u0 = halo[hb[j] + off0];
            if (t1 < 27) u1 = halo[hb[j] + off1];
            const uint4 u = make_uint4(u0.x, u0.y, u1.x, u1.y);
            const bf16x8 b = __builtin_bit_cast(bf16x8, u);
#pragma unroll
            for (int i = 0; i < MI; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b, acc[i][j], 0, 0, 0);
        }
    }

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
}

}  // namespace

hipError_t launch_conv_c4_fwd(const uint16_t* X, const uint16_t* Wk, uint16_t* Y, const cf_dims& x, int cout,
                              int copad, hipStream_t s)
{
    (void)copad;
    const int tD = (int)((x.d + TD - 1) / TD), tH = (int)((x.h + TH - 1) / TH), tW = (int)((x.w + TW - 1) / TW);
    const unsigned ntile = (unsigned)(x.n * tD * tH * tW);
    if (cout <= 16) {
        hipLaunchKernelGGL(conv3d_c4_fwd_kernel<16>, dim3(ntile, (unsigned)((cout + 15) / 16)), dim3(NT), 0, s, X, Wk,
                           Y, (int)x.n, (int)x.d, (int)x.h, (int)x.w, cout, tD, tH, tW);
    } else {
        hipLaunchKernelGGL(conv3d_c4_fwd_kernel<32>, dim3(ntile, (unsigned)((cout + 31) / 32)), dim3(NT), 0, s, X, Wk,
                           Y, (int)x.n, (int)x.d, (int)x.h, (int)x.w, cout, tD, tH, tW);
    }
    return hipGetLastError();
}

}  // namespace cf
