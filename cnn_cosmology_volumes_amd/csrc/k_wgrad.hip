// Backward-weight of the 3^3 stride-1 pad-1 convolution on bf16 MFMA.
//
//   dW[tap][ci][co] = sum over voxels v of X[v + off(tap)][ci] * dY[v][co]
//
// (the separate backward-weight operator of CosmoFlow, Sec. III-C; the
// convolution itself is the "same"-padded stride-1 one of Oyama et al.,
// Sec. IV / Table I).  This is a GEMM whose reduction runs over voxels, while
// NDHWC stores channels contiguously: every MFMA operand needs 8 consecutive
// voxels of one channel per lane.  gfx950's LDS transpose read
// (ds_read_b64_tr_b16) provides exactly that from the natural [voxel][channel]
// tiles: within each 16-lane group, lane 4r+q names row r (a voxel) and
// columns 4q..4q+3 (channels); lane j receives column j of the 4 rows.  A tap
// shift only changes which halo row a lane names, so the X halo is staged
// once per voxel box and reused by all 27 taps.
//
// Orientation: C[co][ci] += dY^T[co][k] * Xshift[k][ci] (16x16x32 MFMA), so
// a lane's accumulator holds 4 consecutive co of one ci -> one 16-byte store
// into the [tap][ci][co] result.  The voxel reduction is split into fixed
// ranges (one per block), written as fp32 partials and summed in a fixed
// order by wgrad_reduce: the result is deterministic.
#include "cf_internal.h"

namespace cf {

namespace {

__device__ __forceinline__ s16x4 lds_tr16(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((CF_LDS s16x4*)(p));
}

__device__ __forceinline__ bf16x8 join8(s16x4 lo, s16x4 hi) {
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// ---------------------------------------------------------------- general
// Block: 9 waves; wave w handles taps (kd, kh) = (w / 3, w % 3), kw = 0..2,
// for 32 input channels (ci block) x BO output channels (co block).
// Voxel box: TD x TH x TW voxels of one sample (128), 4 K-steps of 32.
constexpr int GW_TD = 2, GW_TH = 4, GW_TW = 16;
constexpr int GW_VB = GW_TD * GW_TH * GW_TW;                         // 128 voxels
constexpr int GW_HD = GW_TD + 2, GW_HH = GW_TH + 2, GW_HW = GW_TW + 2;
constexpr int GW_HV = GW_HD * GW_HH * GW_HW;                         // 432 halo voxels
constexpr int GW_XS = 48;        // bf16 per halo row: 32 data + 16 pad (96 B)
constexpr int GW_NT = 9 * 64;

template <int BO>
__global__ __launch_bounds__(GW_NT)
void wgrad_mfma_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ dY,
                       float* __restrict__ part, int N, int D, int H, int W, int Cin, int Cout,
                       int bD, int bH, int bW, int64_t nbox, int boxes_per_split)
{
    constexpr int DS = BO + 16;          // bf16 per dY row (pad 32 B)
    constexpr int CI = BO / 16;          // co fragments
    __shared__ __attribute__((aligned(16))) uint16_t xs[GW_HV * GW_XS];
    __shared__ __attribute__((aligned(16))) uint16_t ds[GW_VB * DS];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const int r4 = l16 >> 2, q4 = l16 & 3;      // transpose-read row / column quad
    const int kd = wave / 3, kh = wave % 3;
    const int co0 = blockIdx.x * BO, ci0 = blockIdx.y * 32;
    const int split = blockIdx.z;
    const int64_t plane = (int64_t)H * W;

    f32x4 acc[3][CI][2];
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int i = 0; i < CI; ++i) {
            acc[t][i][0] = f32x4{0.f, 0.f, 0.f, 0.f};
            acc[t][i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

    const int64_t b_begin = (int64_t)split * boxes_per_split;
    const int64_t b_end = min(b_begin + boxes_per_split, nbox);
    for (int64_t box = b_begin; box < b_end; ++box) {
        int64_t bb = box;
        const int bw = (int)(bb % bW); bb /= bW;
        const int bh = (int)(bb % bH); bb /= bH;
        const int bd = (int)(bb % bD);
        const int n = (int)(bb / bD);
        const int d0 = bd * GW_TD, h0 = bh * GW_TH, w0 = bw * GW_TW;

        __syncthreads();
        // X halo (32 channels of this ci block), zero outside the volume.
        for (int e = threadIdx.x; e < GW_HV * 4; e += GW_NT) {
            const int q = e & 3, hv = e >> 2;
            const int hw_ = hv % GW_HW, hh_ = (hv / GW_HW) % GW_HH, hd_ = hv / (GW_HW * GW_HH);
            const int gd = d0 + hd_ - 1, gh = h0 + hh_ - 1, gw = w0 + hw_ - 1;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if ((unsigned)gd < (unsigned)D && (unsigned)gh < (unsigned)H && (unsigned)gw < (unsigned)W)
                v = *reinterpret_cast<const uint4*>(X + (((int64_t)n * D + gd) * plane + (int64_t)gh * W + gw) * Cin +
                                                    ci0 + q * 8);
            *reinterpret_cast<uint4*>(xs + hv * GW_XS + q * 8) = v;
        }
        // dY box (BO channels of this co block), zero outside the volume.
        for (int e = threadIdx.x; e < GW_VB * (BO / 8); e += GW_NT) {
            const int q = e % (BO / 8), v = e / (BO / 8);
            const int tw = v % GW_TW, th = (v / GW_TW) % GW_TH, td = v / (GW_TW * GW_TH);
            const int gd = d0 + td, gh = h0 + th, gw = w0 + tw;
            uint4 val = make_uint4(0u, 0u, 0u, 0u);
            if (gd < D && gh < H && gw < W)
                val = *reinterpret_cast<const uint4*>(dY + (((int64_t)n * D + gd) * plane + (int64_t)gh * W + gw) * Cout +
                                                      co0 + q * 8);
            *reinterpret_cast<uint4*>(ds + v * DS + q * 8) = val;
        }
        __syncthreads();

#pragma unroll
        for (int s = 0; s < GW_VB / 32; ++s) {
            // voxel rows read by this lane: k = 32 s + 8 lg + r4 (+4)
            const int k0 = 32 * s + 8 * lg + r4, k1 = k0 + 4;
            bf16x8 a[CI];
#pragma unroll
            for (int i = 0; i < CI; ++i)
                a[i] = join8(lds_tr16(ds + k0 * DS + 16 * i + 4 * q4), lds_tr16(ds + k1 * DS + 16 * i + 4 * q4));
            const int tw0 = k0 % GW_TW, th0 = (k0 / GW_TW) % GW_TH, td0 = k0 / (GW_TW * GW_TH);
            const int tw1 = k1 % GW_TW, th1 = (k1 / GW_TW) % GW_TH, td1 = k1 / (GW_TW * GW_TH);
            const int hv0 = ((td0 + kd) * GW_HH + th0 + kh) * GW_HW + tw0;
            const int hv1 = ((td1 + kd) * GW_HH + th1 + kh) * GW_HW + tw1;
#pragma unroll
            for (int kw = 0; kw < 3; ++kw) {
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) {
                    const bf16x8 b = join8(lds_tr16(xs + (hv0 + kw) * GW_XS + 16 * jj + 4 * q4),
                                           lds_tr16(xs + (hv1 + kw) * GW_XS + 16 * jj + 4 * q4));
#pragma unroll
                    for (int i = 0; i < CI; ++i)
                        acc[kw][i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b, acc[kw][i][jj], 0, 0, 0);
                }
            }
        }
    }

    // partial[split][tap][ci][co]; lane holds co rows 4 lg..4 lg+3 of column ci = l16
    const int64_t dwsize = (int64_t)27 * Cin * Cout;
#pragma unroll
    for (int kw = 0; kw < 3; ++kw) {
        const int tap = (kd * 3 + kh) * 3 + kw;
#pragma unroll
        for (int i = 0; i < CI; ++i)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int ci = ci0 + 16 * jj + l16;
                const int co = co0 + 16 * i + 4 * lg;
                const f32x4 r = acc[kw][i][jj];
                *reinterpret_cast<float4*>(part + split * dwsize + ((int64_t)tap * Cin + ci) * Cout + co) =
                    make_float4(r[0], r[1], r[2], r[3]);
            }
    }
}

// --------------------------------------------------------- Cin == 4 layer
// dW[tap][ci][co] for 4 input channels: N = 27 taps x 4 ci packed as 7
// fragments of (4 taps x 4 ci) = 16 columns; every wave accumulates the whole
// 32 x 108 result over its own quarter of each voxel box, and the four waves
// are summed through LDS at the end (fixed order).
constexpr int C4_TD = 4, C4_TH = 4, C4_TW = 16;
constexpr int C4_VB = C4_TD * C4_TH * C4_TW;                          // 256 voxels
constexpr int C4_HD = C4_TD + 2, C4_HH = C4_TH + 2, C4_HW = C4_TW + 2;
constexpr int C4_HV = C4_HD * C4_HH * C4_HW;                          // 648
constexpr int C4_NT = 256;

__device__ __forceinline__ int c4_tapoff(int t) {
    return ((t / 9) * C4_HH + (t / 3) % 3) * C4_HW + t % 3;
}

__global__ __launch_bounds__(C4_NT)
void wgrad_c4_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ dY, float* __restrict__ part,
                     int N, int D, int H, int W, int bD, int bH, int bW, int64_t nbox, int boxes_per_split)
{
    constexpr int CO = 32, DS = CO + 16;     // dY row: 32 data + 16 pad bf16
    __shared__ __attribute__((aligned(16))) uint16_t xs[C4_HV * 4];
    __shared__ __attribute__((aligned(16))) uint16_t ds[C4_VB * DS];
    __shared__ float red[3][64 * 56];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const int r4 = l16 >> 2, q4 = l16 & 3;
    const int split = blockIdx.x;
    const int64_t plane = (int64_t)H * W;

    f32x4 acc[2][7];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int f = 0; f < 7; ++f) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};

    // tap of the row this lane names in each N fragment (taps >= 27 padded)
    int toff[7];
#pragma unroll
    for (int f = 0; f < 7; ++f) {
        const int t = 4 * f + q4;
        toff[f] = t < 27 ? c4_tapoff(t) : 0;
    }

    const int64_t b_begin = (int64_t)split * boxes_per_split;
    const int64_t b_end = min(b_begin + boxes_per_split, nbox);
    for (int64_t box = b_begin; box < b_end; ++box) {
        int64_t bb = box;
        const int bw = (int)(bb % bW); bb /= bW;
        const int bh = (int)(bb % bH); bb /= bH;
        const int bd = (int)(bb % bD);
        const int n = (int)(bb / bD);
        const int d0 = bd * C4_TD, h0 = bh * C4_TH, w0 = bw * C4_TW;
        __syncthreads();
        for (int hv = threadIdx.x; hv < C4_HV; hv += C4_NT) {
            const int hw_ = hv % C4_HW, hh_ = (hv / C4_HW) % C4_HH, hd_ = hv / (C4_HW * C4_HH);
            const int gd = d0 + hd_ - 1, gh = h0 + hh_ - 1, gw = w0 + hw_ - 1;
            uint2 v = make_uint2(0u, 0u);
            if ((unsigned)gd < (unsigned)D && (unsigned)gh < (unsigned)H && (unsigned)gw < (unsigned)W)
                v = *reinterpret_cast<const uint2*>(X + (((int64_t)n * D + gd) * plane + (int64_t)gh * W + gw) * 4);
            *reinterpret_cast<uint2*>(xs + hv * 4) = v;
        }
        for (int e = threadIdx.x; e < C4_VB * 4; e += C4_NT) {
            const int q = e & 3, v = e >> 2;
            const int tw = v % C4_TW, th = (v / C4_TW) % C4_TH, td = v / (C4_TW * C4_TH);
            const int gd = d0 + td, gh = h0 + th, gw = w0 + tw;
            uint4 val = make_uint4(0u, 0u, 0u, 0u);
            if (gd < D && gh < H && gw < W)
                val = *reinterpret_cast<const uint4*>(dY + (((int64_t)n * D + gd) * plane + (int64_t)gh * W + gw) * CO +
                                                      q * 8);
            *reinterpret_cast<uint4*>(ds + v * DS + q * 8) = val;
        }
        __syncthreads();

#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int k0 = wave * 64 + 32 * s + 8 * lg + r4, k1 = k0 + 4;
            bf16x8 a[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                a[i] = join8(lds_tr16(ds + k0 * DS + 16 * i + 4 * q4), lds_tr16(ds + k1 * DS + 16 * i + 4 * q4));
            const int hv0 = ((k0 / (C4_TW * C4_TH)) * C4_HH + (k0 / C4_TW) % C4_TH) * C4_HW + k0 % C4_TW;
            const int hv1 = ((k1 / (C4_TW * C4_TH)) * C4_HH + (k1 / C4_TW) % C4_TH) * C4_HW + k1 % C4_TW;
#pragma unroll
            for (int f = 0; f < 7; ++f) {
                const bf16x8 b = join8(lds_tr16(xs + (hv0 + toff[f]) * 4), lds_tr16(xs + (hv1 + toff[f]) * 4));
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    acc[i][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b, acc[i][f], 0, 0, 0);
            }
        }
    }

    // Sum the four waves' accumulators in wave order 0 + 1 + 2 + 3.
    __syncthreads();
    if (wave > 0) {
        float* dst = red[wave - 1] + lane * 56;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int f = 0; f < 7; ++f)
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[(i * 7 + f) * 4 + r] = acc[i][f][r];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int w = 0; w < 3; ++w) {
            const float* src = red[w] + lane * 56;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int f = 0; f < 7; ++f)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[i][f][r] += src[(i * 7 + f) * 4 + r];
        }
        float* out = part + (int64_t)split * (27 * 4 * CO);
#pragma unroll
        for (int f = 0; f < 7; ++f) {
            const int t = 4 * f + (l16 >> 2), ci = l16 & 3;
            if (t >= 27) continue;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int co = 16 * i + 4 * lg;
                const f32x4 r = acc[i][f];
                *reinterpret_cast<float4*>(out + (t * 4 + ci) * CO + co) = make_float4(r[0], r[1], r[2], r[3]);
            }
        }
    }
}

// dW[e] = sum over splits of part[s][e].  A block owns 64 consecutive
// elements; its 16 split-lanes each sum the splits s = lane, lane + 16, ...
// in increasing order, and the 16 lane sums are added in lane order.  The
// order is fixed, so the result is deterministic.
constexpr int RD_E = 64, RD_L = 16;

__global__ __launch_bounds__(RD_E * RD_L)
void wgrad_reduce_kernel(const float* __restrict__ part, float* __restrict__ dW, int64_t n, int splits)
{
    __shared__ float red[RD_L][RD_E];
    const int el = threadIdx.x % RD_E, sl = threadIdx.x / RD_E;
    const int64_t i = (int64_t)blockIdx.x * RD_E + el;
    float s = 0.f;
    if (i < n) {
#pragma unroll 4
        for (int k = sl; k < splits; k += RD_L) s += part[(int64_t)k * n + i];
    }
    red[sl][el] = s;
    __syncthreads();
    if (sl == 0 && i < n) {
        float t = red[0][el];
#pragma unroll
        for (int k = 1; k < RD_L; ++k) t += red[k][el];
        dW[i] = t;
    }
}

}  // namespace

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
        const int bo = (cout % 64 == 0) ? 64 : 32;
        const int64_t nbox = x.n * ((x.d + GW_TD - 1) / GW_TD) * ((x.h + GW_TH - 1) / GW_TH) *
                             ((x.w + GW_TW - 1) / GW_TW);
        const int64_t outer = (int64_t)(cout / bo) * (x.c / 32);
        int64_t want = (512 + outer - 1) / outer;
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
        const int bD = (int)((x.d + C4_TD - 1) / C4_TD), bH = (int)((x.h + C4_TH - 1) / C4_TH),
                  bW = (int)((x.w + C4_TW - 1) / C4_TW);
        const int64_t nbox = x.n * bD * bH * bW;
        hipLaunchKernelGGL(wgrad_c4_kernel, dim3((unsigned)p.splits), dim3(C4_NT), 0, s, X, dY, part, (int)x.n,
                           (int)x.d, (int)x.h, (int)x.w, bD, bH, bW, nbox, (int)p.vox_per_split);
    } else {
        const int bD = (int)((x.d + GW_TD - 1) / GW_TD), bH = (int)((x.h + GW_TH - 1) / GW_TH),
                  bW = (int)((x.w + GW_TW - 1) / GW_TW);
        const int64_t nbox = x.n * bD * bH * bW;
        const int bo = (cout % 64 == 0) ? 64 : 32;
        dim3 grid((unsigned)(cout / bo), (unsigned)(x.c / 32), (unsigned)p.splits);
        if (bo == 64)
            hipLaunchKernelGGL(wgrad_mfma_kernel<64>, grid, dim3(GW_NT), 0, s, X, dY, part, (int)x.n, (int)x.d,
                               (int)x.h, (int)x.w, (int)x.c, cout, bD, bH, bW, nbox, (int)p.vox_per_split);
        else
            hipLaunchKernelGGL(wgrad_mfma_kernel<32>, grid, dim3(GW_NT), 0, s, X, dY, part, (int)x.n, (int)x.d,
                               (int)x.h, (int)x.w, (int)x.c, cout, bD, bH, bW, nbox, (int)p.vox_per_split);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)27 * x.c * cout;
    hipLaunchKernelGGL(wgrad_reduce_kernel, dim3((unsigned)((n + RD_E - 1) / RD_E)), dim3(RD_E * RD_L), 0, s, part, dW,
                       n, p.splits);
    return hipGetLastError();
}

}  // namespace cf
