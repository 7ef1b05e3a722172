// fp32 3^3 convolution on the matrix cores (v_mfma_f32_16x16x4_f32): the
// forward and backward-data (forward orientation on flipped, transposed
// weights) and the backward-weight of the fp32 path, for any channel counts
// that are multiples of 4.  Same definitions as the bf16 kernels (Oyama et
// al., Sec. IV / Table I: stride 1, "same" zero padding, no bias).
//
// Fragments.  One 16x16x4 MFMA takes, per lane l, A[l % 16][l / 16] and
// B[l / 16][l % 16] and accumulates D[4 (l / 16) + r][l % 16], r = 0..3.  A
// lane here loads four consecutive K values as one float4 and the wave runs
// four MFMAs q = 0..3 on them: MFMA q's K index k stands for K value 4k + q,
// so the four MFMAs cover 16 K values and every operand fetch is one
// aligned 16-byte read.
//
// Forward tile: 64 output channels x a 4x4x4 voxel box per block (4 waves;
// wave w owns output-channel tiles 2 (w & 1) .. + 1 and the box's depth
// planes 2 (w >> 1) .. + 1).  The 6x6x6 input halo of 16 channels is staged
// in LDS per channel chunk; B fragments read it at a per-tap offset, A
// fragments (weights [tap][co][ci], padded) come from global/L2 one tap ahead.
//
// Backward-weight tile: 16 input channels x 64 output channels x all 27 taps
// per block (wave w owns output channels 16 w .. 16 w + 15), over a fixed
// range of 4x4x4 boxes.  Per box the input halo is staged transposed as
// three w-shifted copies XT[kw][ci][hd][hh][w] (so a tap's operand is an
// aligned float4 of four consecutive voxels) and the output gradient as
// DT[co][voxel].  Each block writes its fp32 partial dW; a fixed-order
// reduction adds the splits in fp64.
//
// Summation length.  fp32 chains grow their rounding error with their
// length, and these sums are long (27 x 256 terms per forward output, up to
// ~10^7 voxels per weight gradient).  The forward accumulates each 16-channel
// chunk (432 products) in fresh registers and adds the chunk sums into the
// total; the backward-weight gives each split at most BOX_PER_SPLIT boxes
// (1024 products per accumulator) and adds the splits in fp64.
//
// bf16 storage.  The same kernels serve bf16 layers whose channel counts the
// bf16 kernels do not cover (multiples of 4 but not of 32, other than the
// 4-channel first layer): activations and gradients are read as bf16 and
// widened exactly, the weights are the bf16-rounded values held in fp32, and
// outputs are rounded to bf16 at the store.  A product of two bf16 values is
// exact in fp32, so this is the bf16 path's arithmetic (bf16 operands, fp32
// accumulation) on the fp32 matrix cores.
#include "cf_internal.h"

namespace cf {
namespace {

constexpr int F_T = 256;        // threads per block (4 waves)
constexpr int F_BM = 64;        // output channels per forward block
constexpr int F_CC = 16;        // channels per staged chunk
constexpr int F_B = 4;          // box edge (voxels)
constexpr int F_H = F_B + 2;    // halo edge
constexpr int F_HV = F_H * F_H * F_H;

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mfma4(const f4& a, const f4& b, f4 acc)
{
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
    return acc;
}

__device__ __forceinline__ f4 ld4g(const float* p) { return *reinterpret_cast<const f4*>(p); }
__device__ __forceinline__ f4 ld4g(const uint16_t* p)
{
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    return f4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
              __uint_as_float(u.y & 0xffff0000u)};
}
__device__ __forceinline__ void st4g(float* p, const f4& v) { *reinterpret_cast<f4*>(p) = v; }
__device__ __forceinline__ void st4g(uint16_t* p, const f4& v)
{
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}

// Y[n, d, h, w, co] = sum_tap sum_ci X[n, d+kd-1, h+kh-1, w+kw-1, ci] Wk[tap][co][ci]
// Wk: [27][copad][cipad] fp32, zero beyond cout / cin; copad % 64 == 0, cipad % 16 == 0.
// T: storage type of X and Y (float, or uint16_t for bf16).
// CIN4 (4 input channels): a K group of 16 is four taps x 4 channels (lane
//   group k4 takes tap 4 g + k4, its float4 the 4 channels), so 7 groups
//   cover the 27 taps where the 16-channel chunks would take 27 groups with
//   a quarter of K live.  The weights are read from the same layout (channel
//   offset 0 of the lane's tap); the 28th slot has zero weights.
// CO32 (at most 32 output channels): a block is 32 output channels x the
//   box and each wave owns one depth plane, instead of 64-channel blocks
//   whose second half would be idle.
template <typename T, bool CIN4, bool CO32>
__global__ __launch_bounds__(F_T) void conv_f32_mfma_kernel(const T* __restrict__ X, const float* __restrict__ Wk,
                                                            T* __restrict__ Y, int N, int D, int H, int W,
                                                            int Cin, int Cout, int cipad, int copad, int bD, int bH,
                                                            int bW, int ncb)
{
    constexpr int BMK = CO32 ? 32 : F_BM;     // output channels per block
    constexpr int NV = CO32 ? 1 : 2;          // depth planes per wave
    __shared__ f4 halo[F_HV * (F_CC / 4)];       // [halo voxel][4 channel quads]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int b = blockIdx.x;
    const int cb = b % ncb; b /= ncb;
    const int bw = b % bW; b /= bW;
    const int bh = b % bH; b /= bH;
    const int bd = b % bD;
    const int n = b / bD;
    const int d0 = bd * F_B, h0 = bh * F_B, w0 = bw * F_B;
    const int i16 = lane & 15, k4 = lane >> 4;
    // this lane's voxel in its wave's depth planes: h = i16 / 4, w = i16 % 4
    const int vh = i16 >> 2, vw = i16 & 3;
    const int dp0 = CO32 ? wave : 2 * (wave >> 1);
    const int co_w = cb * BMK + (CO32 ? 0 : 32 * (wave & 1));
    f4 tot[2][NV];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int c = 0; c < NV; ++c) tot[a][c] = f4{0.f, 0.f, 0.f, 0.f};

    if constexpr (CIN4) {
        // one chunk: the 4 channels of every halo voxel (quad 0 of its row)
        for (int hv = tid; hv < F_HV; hv += F_T) {
            const int hx = hv % F_H, hy = (hv / F_H) % F_H, hz = hv / (F_H * F_H);
            const int id = d0 + hz - 1, ih = h0 + hy - 1, iw = w0 + hx - 1;
            f4 v = f4{0.f, 0.f, 0.f, 0.f};
            if ((unsigned)id < (unsigned)D && (unsigned)ih < (unsigned)H && (unsigned)iw < (unsigned)W)
                v = ld4g(X + ((((int64_t)n * D + id) * H + ih) * W + iw) * 4);
            halo[hv * 4] = v;
        }
        __syncthreads();
        const int64_t tapstride = (int64_t)copad * cipad;
        const float* wrow = Wk + (int64_t)(co_w + i16) * cipad;
#pragma unroll
        for (int g = 0; g < 7; ++g) {
            const int t = 4 * g + k4;
            const bool live = t < 27;
            const int tt = live ? t : 26;
            const int kd = tt / 9, kh = (tt / 3) % 3, kw = tt % 3;
            f4 a0 = ld4g(wrow + tt * tapstride), a1 = ld4g(wrow + tt * tapstride + 16 * cipad);
            if (!live) a0 = a1 = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int vt = 0; vt < NV; ++vt) {
                const int hv = ((dp0 + vt + kd) * F_H + vh + kh) * F_H + vw + kw;
                const f4 bv = halo[hv * 4];
                tot[0][vt] = mfma4(a0, bv, tot[0][vt]);
                tot[1][vt] = mfma4(a1, bv, tot[1][vt]);
            }
        }
    } else {
        for (int c0 = 0; c0 < Cin; c0 += F_CC) {
            f4 acc[2][NV];
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int c = 0; c < NV; ++c) acc[a][c] = f4{0.f, 0.f, 0.f, 0.f};
            __syncthreads();
            for (int i = tid; i < F_HV * 4; i += F_T) {
                const int q = i & 3, hv = i >> 2;
                const int hx = hv % F_H, hy = (hv / F_H) % F_H, hz = hv / (F_H * F_H);
                const int id = d0 + hz - 1, ih = h0 + hy - 1, iw = w0 + hx - 1, ci = c0 + 4 * q;
                f4 v = f4{0.f, 0.f, 0.f, 0.f};
                if ((unsigned)id < (unsigned)D && (unsigned)ih < (unsigned)H && (unsigned)iw < (unsigned)W && ci < Cin)
                    v = ld4g(X + ((((int64_t)n * D + id) * H + ih) * W + iw) * Cin + ci);
                halo[i] = v;
            }
            __syncthreads();
            const float* wbase = Wk + (int64_t)(co_w + i16) * cipad + c0 + 4 * k4;
            const int64_t tapstride = (int64_t)copad * cipad;
            f4 a0 = ld4g(wbase), a1 = ld4g(wbase + 16 * cipad);
#pragma unroll 1
            for (int t = 0; t < 27; ++t) {
                const int kd = t / 9, kh = (t / 3) % 3, kw = t % 3;
                f4 n0 = a0, n1 = a1;
                if (t + 1 < 27) {
                    n0 = ld4g(wbase + (t + 1) * tapstride);
                    n1 = ld4g(wbase + (t + 1) * tapstride + 16 * cipad);
                }
#pragma unroll
                for (int vt = 0; vt < NV; ++vt) {
                    const int hv = ((dp0 + vt + kd) * F_H + vh + kh) * F_H + vw + kw;
                    const f4 bv = halo[hv * 4 + k4];
                    acc[0][vt] = mfma4(a0, bv, acc[0][vt]);
                    acc[1][vt] = mfma4(a1, bv, acc[1][vt]);
                }
                a0 = n0;
                a1 = n1;
            }
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int c = 0; c < NV; ++c) tot[a][c] += acc[a][c];
        }
    }
    // D[4 k4 + r][i16]: output channels co_w + 16 ct + 4 k4 + r, voxel i16 of plane dp0 + vt
#pragma unroll
    for (int vt = 0; vt < NV; ++vt) {
        const int d = d0 + dp0 + vt, h = h0 + vh, w = w0 + vw;
        if (d >= D || h >= H || w >= W) continue;
        T* yp = Y + ((((int64_t)n * D + d) * H + h) * W + w) * Cout;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const int co = co_w + 16 * ct + 4 * k4;
            if (co < Cout) st4g(yp + co, tot[ct][vt]);
        }
    }
}

constexpr int G_BN = 64;         // output channels staged per backward-weight block (at most)
constexpr int G_XT = 3 * F_CC * F_H * F_H * 4;   // floats of the three shifted halo copies
constexpr int G_DT = G_BN * 64;                  // floats of the transposed output gradient

// part[split][tap][ci][co] over the boxes [split * per, min(nbox, (split+1) * per)).
// T: storage type of X and dY (float, or uint16_t for bf16).
//
// The MFMA rows are 16 input channels of one tap (A = the shifted halo), the
// columns 16 output channels (B = the transposed gradient).  Two shapes
// would leave most of that idle, and each has its own mapping:
//  - CIN4 (4 input channels): the rows are (kw, ci) pairs, 3 x 4 = 12 of 16,
//    so one MFMA group covers the three kw taps of a (kd, kh) pair and a box
//    takes 9 groups per output-channel tile instead of 27 with a quarter of
//    the rows live.  (Rows 12-15 read input channels 4-7 of the kw = 0 copy,
//    which are zeros.)
//  - NWCO < 4 (at most 16 or 32 output channels): NWCO waves cover the
//    output channels and the 4 / NWCO wave sets split the taps (or pairs)
//    between them, instead of idle waves computing channels past Cout.
template <typename T, bool CIN4, int NWCO>
__global__ __launch_bounds__(F_T) void wgrad_f32_mfma_kernel(const T* __restrict__ X, const T* __restrict__ dY,
                                                             float* __restrict__ part, int N, int D, int H, int W,
                                                             int Cin, int Cout, int bD, int bH, int bW, int nci,
                                                             int nco, int64_t nbox, int per)
{
    constexpr int NTS = 4 / NWCO;                  // wave sets splitting the taps
    constexpr int NTAP = CIN4 ? 9 : 27;            // MFMA groups per box and depth plane
    constexpr int NA = (NTAP + NTS - 1) / NTS;     // groups per wave
    constexpr int BN = 16 * NWCO;                  // output channels per block
    __shared__ float xt[G_XT];     // [kw][ci 16][hd 6][hh 6][w 4]
    __shared__ float dt[G_DT];     // [co][voxel 64], voxel = (d * 4 + h) * 4 + w
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int cog = wave % NWCO, tsub = wave / NWCO;
    int b = blockIdx.x;
    const int cit = b % nci; b /= nci;
    const int cot = b % nco;
    const int split = b / nco;
    const int ci0 = cit * F_CC, co0 = cot * BN;
    const int i16 = lane & 15, k4 = lane >> 4;
    // CIN4: this lane's row is (kw, ci) = (i16 / 4, i16 % 4); row 3 x 4 + c
    // reads channel 4 + c of the kw = 0 copy (zero, as Cin = 4)
    const int aplane = CIN4 ? ((i16 >> 2) < 3 ? (i16 >> 2) * F_CC + (i16 & 3) : 4 + (i16 & 3)) : i16;
    f4 acc[NA];
#pragma unroll
    for (int j = 0; j < NA; ++j) acc[j] = f4{0.f, 0.f, 0.f, 0.f};
    const int64_t bb0 = (int64_t)split * per;
    const int64_t bb1 = min(nbox, bb0 + per);
    for (int64_t bx = bb0; bx < bb1; ++bx) {
        int64_t r = bx;
        const int bw = (int)(r % bW); r /= bW;
        const int bh = (int)(r % bH); r /= bH;
        const int bd = (int)(r % bD);
        const int n = (int)(r / bD);
        const int d0 = bd * F_B, h0 = bh * F_B, w0 = bw * F_B;
        __syncthreads();
        // input halo: 216 voxels x 4 channel quads, scattered into the three w-shifted copies
        for (int i = tid; i < F_HV * 4; i += F_T) {
            const int q = i & 3, hv = i >> 2;
            const int hx = hv % F_H, hy = (hv / F_H) % F_H, hz = hv / (F_H * F_H);
            const int id = d0 + hz - 1, ih = h0 + hy - 1, iw = w0 + hx - 1, ci = ci0 + 4 * q;
            f4 v = f4{0.f, 0.f, 0.f, 0.f};
            if ((unsigned)id < (unsigned)D && (unsigned)ih < (unsigned)H && (unsigned)iw < (unsigned)W && ci < Cin)
                v = ld4g(X + ((((int64_t)n * D + id) * H + ih) * W + iw) * Cin + ci);
#pragma unroll
            for (int kw = 0; kw < 3; ++kw) {
                const int w = hx - kw;
                if (w < 0 || w >= F_B) continue;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    xt[(((kw * F_CC + 4 * q + e) * F_H + hz) * F_H + hy) * 4 + w] = v[e];
            }
        }
        // output gradient: 64 voxels x BN / 4 channel quads, transposed to [co][voxel]
        for (int i = tid; i < 64 * (BN / 4); i += F_T) {
            const int q = i % (BN / 4), v = i / (BN / 4);
            const int vw = v & 3, vh = (v >> 2) & 3, vd = v >> 4;
            const int d = d0 + vd, h = h0 + vh, w = w0 + vw, co = co0 + 4 * q;
            f4 g = f4{0.f, 0.f, 0.f, 0.f};
            if (d < D && h < H && w < W && co < Cout)
                g = ld4g(dY + ((((int64_t)n * D + d) * H + h) * W + w) * Cout + co);
#pragma unroll
            for (int e = 0; e < 4; ++e) dt[(4 * q + e) * 64 + v] = g[e];
        }
        __syncthreads();
        // K = the box's 64 voxels: depth plane dp, lane group k4 = h, four w per float4
#pragma unroll 1
        for (int dp = 0; dp < F_B; ++dp) {
            const f4 bv = *reinterpret_cast<const f4*>(&dt[(16 * cog + i16) * 64 + dp * 16 + k4 * 4]);
#pragma unroll
            for (int j = 0; j < NA; ++j) {
                const int t = tsub + j * NTS;
                if (NTAP % NTS != 0 && t >= NTAP) break;
                // CIN4: t is the (kd, kh) pair; otherwise the tap
                const int kd = CIN4 ? t / 3 : t / 9, kh = CIN4 ? t % 3 : (t / 3) % 3, kw = CIN4 ? 0 : t % 3;
                const f4 av = *reinterpret_cast<const f4*>(
                    &xt[(((kw * F_CC + aplane) * F_H + dp + kd) * F_H + k4 + kh) * 4]);
                acc[j] = mfma4(av, bv, acc[j]);
            }
        }
    }
    // D[4 k4 + r][i16]: output channel co0 + 16 cog + i16; row 4 k4 + r is
    // input channel ci0 + 4 k4 + r of tap t, or (CIN4) tap (kd, kh, kw = k4)
    // and input channel r
    const int co = co0 + 16 * cog + i16;
    if (co >= Cout) return;
    const int64_t dws = (int64_t)27 * Cin * Cout;
    float* out = part + (int64_t)split * dws;
#pragma unroll
    for (int j = 0; j < NA; ++j) {
        const int t = tsub + j * NTS;
        if (NTAP % NTS != 0 && t >= NTAP) break;
        if (CIN4) {
            if (k4 == 3) continue;
            const int tap = t * 3 + k4;          // (kd * 3 + kh) * 3 + kw
#pragma unroll
            for (int e = 0; e < 4; ++e) out[((int64_t)tap * Cin + e) * Cout + co] = acc[j][e];
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int ci = ci0 + 4 * k4 + e;
                if (ci < Cin) out[((int64_t)t * Cin + ci) * Cout + co] = acc[j][e];
            }
        }
    }
}

// dW[e] = sum over splits of part[s][e] in fp64: a block owns 64 elements
// (4 per thread, 16-byte loads); its 16 split-lanes sum the splits s = lane,
// lane + 16, ... in increasing order and the lane sums are added in lane
// order, so the result is deterministic.  n is a multiple of 4.
constexpr int R64_T = 16, R64_E = R64_T * 4, R64_L = 16;

__global__ __launch_bounds__(R64_T * R64_L) void wgrad_reduce_f64_kernel(const float* __restrict__ part,
                                                                        float* __restrict__ dW, int64_t n, int splits)
{
    __shared__ double red[R64_L][R64_T][4];
    const int el = threadIdx.x % R64_T, sl = threadIdx.x / R64_T;
    const int64_t i = (int64_t)blockIdx.x * R64_E + 4 * el;
    const int64_t n4 = n / 4;
    const f4* p4 = reinterpret_cast<const f4*>(part);
    double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
    if (i < n) {
        int k = sl;
        for (; k + 7 * R64_L < splits; k += 8 * R64_L) {
            f4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = p4[(int64_t)(k + u * R64_L) * n4 + i / 4];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                s0 += (double)v[u][0]; s1 += (double)v[u][1]; s2 += (double)v[u][2]; s3 += (double)v[u][3];
            }
        }
        for (; k < splits; k += R64_L) {
            const f4 v = p4[(int64_t)k * n4 + i / 4];
            s0 += (double)v[0]; s1 += (double)v[1]; s2 += (double)v[2]; s3 += (double)v[3];
        }
    }
    red[sl][el][0] = s0; red[sl][el][1] = s1; red[sl][el][2] = s2; red[sl][el][3] = s3;
    __syncthreads();
    if (sl == 0 && i < n) {
        for (int e = 0; e < 4; ++e) {
            double t = red[0][el][e];
            for (int k = 1; k < R64_L; ++k) t += red[k][el][e];
            dW[i + e] = (float)t;
        }
    }
}

// Wk[t][a][b] (a < apad, b < bpad) from DHWIO W[tap][ci][co]:
// forward (flip = 0): a = co, b = ci, tap = t;  backward-data (flip = 1):
// a = ci, b = co, tap = 26 - t.  The source is fp32 taken as is, fp32
// rounded to bf16 (the bf16 path's weights from fp32 masters), or bf16.
__global__ void wprep_f32_kernel(const void* __restrict__ W, F32WSrc src, float* __restrict__ Wk, int cin, int cout,
                                 int apad, int bpad, int flip)
{
    const int64_t total = (int64_t)27 * apad * bpad;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    const int bi = (int)(i % bpad);
    const int ai = (int)((i / bpad) % apad);
    const int t = (int)(i / ((int64_t)bpad * apad));
    const int ci = flip ? ai : bi, co = flip ? bi : ai;
    const int tap = flip ? 26 - t : t;
    float v = 0.f;
    if (ci < cin && co < cout) {
        const int64_t e = ((int64_t)tap * cin + ci) * cout + co;
        if (src == F32WSrc::Bf16)
            v = __uint_as_float((uint32_t)static_cast<const uint16_t*>(W)[e] << 16);
        else
            v = static_cast<const float*>(W)[e];
        if (src == F32WSrc::F32RoundBf16) v = __uint_as_float(pack_bf16x2(v, 0.f) << 16);
    }
    Wk[i] = v;
}

int rup(int v, int m) { return (v + m - 1) / m * m; }

}  // namespace

bool conv_f32_mfma_ok(const cf_dims& x, int cout)
{
    // 32-bit block ids and channel multiples of 4 for the float4 accesses
    const int64_t nb = x.n * ((x.d + 3) / 4) * ((x.h + 3) / 4) * ((x.w + 3) / 4);
    return x.c % 4 == 0 && cout % 4 == 0 && nb * ((cout + 63) / 64) < ((int64_t)1 << 31);
}

size_t conv_f32_wk_bytes(int cin, int cout) { return (size_t)27 * rup(cout, 64) * rup(cin, 16) * 4; }

hipError_t launch_wprep_f32(const void* W, F32WSrc src, int cin, int cout, bool dgrad, float* Wk, hipStream_t s)
{
    // forward: [27][rup(cout, 64)][rup(cin, 16)]; backward-data: in = cout, out = cin
    const int apad = dgrad ? rup(cin, 64) : rup(cout, 64);
    const int bpad = dgrad ? rup(cout, 16) : rup(cin, 16);
    const int64_t total = (int64_t)27 * apad * bpad;
    hipLaunchKernelGGL(wprep_f32_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, W, src, Wk, cin, cout,
                       apad, bpad, dgrad ? 1 : 0);
    return hipGetLastError();
}

template <typename T, bool CIN4, bool CO32>
void conv_f32_mfma_kernel_launch(const T* X, const float* Wk, T* Y, const cf_dims& x, int cout, hipStream_t s)
{
    const int bD = (int)((x.d + 3) / 4), bH = (int)((x.h + 3) / 4), bW = (int)((x.w + 3) / 4);
    const int copad = rup(cout, 64), cipad = rup((int)x.c, 16);
    const int ncb = (cout + (CO32 ? 31 : 63)) / (CO32 ? 32 : 64);
    const int64_t nb = x.n * bD * bH * bW * ncb;
    hipLaunchKernelGGL((conv_f32_mfma_kernel<T, CIN4, CO32>), dim3((unsigned)nb), dim3(F_T), 0, s, X, Wk, Y, (int)x.n,
                       (int)x.d, (int)x.h, (int)x.w, (int)x.c, cout, cipad, copad, bD, bH, bW, ncb);
}

template <typename T>
hipError_t conv_f32_mfma_launch(const T* X, const float* Wk, T* Y, const cf_dims& x, int cout, hipStream_t s)
{
    const bool c4 = x.c == 4, co32 = cout <= 32;
    if (c4 && co32) conv_f32_mfma_kernel_launch<T, true, true>(X, Wk, Y, x, cout, s);
    else if (c4) conv_f32_mfma_kernel_launch<T, true, false>(X, Wk, Y, x, cout, s);
    else if (co32) conv_f32_mfma_kernel_launch<T, false, true>(X, Wk, Y, x, cout, s);
    else conv_f32_mfma_kernel_launch<T, false, false>(X, Wk, Y, x, cout, s);
    return hipGetLastError();
}

hipError_t launch_conv_f32_mfma(const float* X, const float* Wk, float* Y, const cf_dims& x, int cout, hipStream_t s)
{
    return conv_f32_mfma_launch(X, Wk, Y, x, cout, s);
}

hipError_t launch_conv_f32_mfma(const uint16_t* X, const float* Wk, uint16_t* Y, const cf_dims& x, int cout,
                                hipStream_t s)
{
    return conv_f32_mfma_launch(X, Wk, Y, x, cout, s);
}

namespace {
// output-channel waves of the backward-weight block: 16 or 32 channels take
// one or two waves, wider layers four
int wgrad_f32_nwco(int cout) { return cout <= 16 ? 1 : cout <= 32 ? 2 : 4; }
}  // namespace

WgradPlan plan_wgrad_f32(const cf_dims& x, int cout)
{
    WgradPlan p{};
    p.kind = 2;
    const int64_t nbox = x.n * ((x.d + 3) / 4) * ((x.h + 3) / 4) * ((x.w + 3) / 4);
    const int bn = 16 * wgrad_f32_nwco(cout);
    const int64_t outer = (int64_t)(x.c == 4 ? 1 : (x.c + 15) / 16) * ((cout + bn - 1) / bn);
    const int64_t dw_bytes = (int64_t)27 * x.c * cout * 4;
    // at least about four blocks per CU, and at most BOX_PER_SPLIT boxes per
    // split (the length of each fp32 chain), within ~256 MiB of partials
    constexpr int64_t BOX_PER_SPLIT = 16;
    int64_t want = (1024 + outer - 1) / outer;
    const int64_t need = (nbox + BOX_PER_SPLIT - 1) / BOX_PER_SPLIT;
    if (want < need) want = need;
    int64_t cap = (int64_t)(256ll << 20) / dw_bytes;
    if (cap < 1) cap = 1;
    if (want > cap) want = cap;
    if (want > nbox) want = nbox;
    if (want < 1) want = 1;
    const int64_t per = (nbox + want - 1) / want;
    p.splits = (int)((nbox + per - 1) / per);
    p.vox_per_split = per;    // boxes per split
    p.part_bytes = (size_t)p.splits * (size_t)dw_bytes;
    return p;
}

template <typename T, bool CIN4, int NWCO>
void wgrad_f32_mfma_kernel_launch(const WgradPlan& p, const T* X, const T* dY, float* part, const cf_dims& x,
                                  int cout, hipStream_t s)
{
    const int bD = (int)((x.d + 3) / 4), bH = (int)((x.h + 3) / 4), bW = (int)((x.w + 3) / 4);
    const int nci = CIN4 ? 1 : (int)((x.c + 15) / 16), nco = (cout + 16 * NWCO - 1) / (16 * NWCO);
    const int64_t nbox = x.n * bD * bH * bW;
    hipLaunchKernelGGL((wgrad_f32_mfma_kernel<T, CIN4, NWCO>), dim3((unsigned)((int64_t)nci * nco * p.splits)),
                       dim3(F_T), 0, s, X, dY, part, (int)x.n, (int)x.d, (int)x.h, (int)x.w, (int)x.c, cout, bD, bH,
                       bW, nci, nco, nbox, (int)p.vox_per_split);
}

template <typename T>
hipError_t wgrad_f32_mfma_launch(const WgradPlan& p, const T* X, const T* dY, float* part, float* dW, const cf_dims& x,
                                 int cout, hipStream_t s)
{
    const int nwco = wgrad_f32_nwco(cout);
    const bool c4 = x.c == 4;
    if (c4 && nwco == 1) wgrad_f32_mfma_kernel_launch<T, true, 1>(p, X, dY, part, x, cout, s);
    else if (c4 && nwco == 2) wgrad_f32_mfma_kernel_launch<T, true, 2>(p, X, dY, part, x, cout, s);
    else if (c4) wgrad_f32_mfma_kernel_launch<T, true, 4>(p, X, dY, part, x, cout, s);
    else if (nwco == 1) wgrad_f32_mfma_kernel_launch<T, false, 1>(p, X, dY, part, x, cout, s);
    else if (nwco == 2) wgrad_f32_mfma_kernel_launch<T, false, 2>(p, X, dY, part, x, cout, s);
    else wgrad_f32_mfma_kernel_launch<T, false, 4>(p, X, dY, part, x, cout, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t n = (int64_t)27 * x.c * cout;
    hipLaunchKernelGGL(wgrad_reduce_f64_kernel, dim3((unsigned)((n + R64_E - 1) / R64_E)), dim3(R64_T * R64_L), 0, s,
                       (const float*)part, dW, n, p.splits);
    return hipGetLastError();
}

hipError_t launch_wgrad_f32_mfma(const WgradPlan& p, const float* X, const float* dY, float* part, float* dW,
                                 const cf_dims& x, int cout, hipStream_t s)
{
    return wgrad_f32_mfma_launch(p, X, dY, part, dW, x, cout, s);
}

hipError_t launch_wgrad_f32_mfma(const WgradPlan& p, const uint16_t* X, const uint16_t* dY, float* part, float* dW,
                                 const cf_dims& x, int cout, hipStream_t s)
{
    return wgrad_f32_mfma_launch(p, X, dY, part, dW, x, cout, s);
}

}  // namespace cf
