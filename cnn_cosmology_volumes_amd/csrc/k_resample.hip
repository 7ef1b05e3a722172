// Resampling kernels for the stride-2 "same" convolution, and 2^3 average
// pooling with leaky ReLU.
//
// Stride 2.  With TensorFlow's "same" padding a 3^3 stride-2 convolution of
// an even-sized volume reads input voxels 2o, 2o+1, 2o+2 for output o (pad 0
// below, 1 above); of an odd-sized one 2o-1, 2o, 2o+1 (pad 1 on both sides).
// Either way output o is the stride-1, pad-1 convolution's output at 2o + q
// with q = 1 - pad.  So the forward is the stride-1 convolution followed by
// subsample_kernel, and, as subsampling's adjoint is placing the values back
// at 2o + q with zeros elsewhere, the backward passes are the stride-1 ones
// applied to upsample_kernel's output.
//
// Average pooling (CosmoFlow, Sec. III-A and III-C: stride-2 average pooling
// per channel with constant weights 1/(KS)^3): P = (1/8) sum over the 2^3
// window of lrelu(Z); backward dZ = lrelu'(Z) dP / 8.  Both bandwidth-bound:
// 8 channels (16 bytes of bf16) per thread.
#include "cf_internal.h"

namespace cf {
namespace {

constexpr int RS_T = 256;

unsigned grid_of(int64_t n)
{
    int64_t b = (n + RS_T - 1) / RS_T;
    if (b > 16384) b = 16384;
    return (unsigned)(b < 1 ? 1 : b);
}

// Y [n, Do, Ho, Wo, C] = Z [n, D, H, W, C] at (2o + q, 2p + q, 2r + q);
// one thread per (output voxel, 4-channel group).
template <typename T>
__global__ __launch_bounds__(RS_T) void subsample_kernel(const T* __restrict__ Z, T* __restrict__ Y, int N, int D,
                                                         int H, int W, int Do, int Ho, int Wo, int C, int q)
{
    const int G = C / 4;
    const int64_t total = (int64_t)N * Do * Ho * Wo * G;
    const int64_t stride = (int64_t)gridDim.x * RS_T;
    for (int64_t e = (int64_t)blockIdx.x * RS_T + threadIdx.x; e < total; e += stride) {
        const int g = (int)(e % G);
        int64_t v = e / G;
        const int ow = (int)(v % Wo); v /= Wo;
        const int oh = (int)(v % Ho); v /= Ho;
        const int od = (int)(v % Do);
        const int n = (int)(v / Do);
        const int64_t src = ((((int64_t)n * D + 2 * od + q) * H + 2 * oh + q) * W + 2 * ow + q) * C + 4 * g;
        const int64_t dst = ((((int64_t)n * Do + od) * Ho + oh) * Wo + ow) * C + 4 * g;
        if (sizeof(T) == 2)
            *reinterpret_cast<uint2*>(Y + dst) = *reinterpret_cast<const uint2*>(Z + src);
        else
            *reinterpret_cast<uint4*>(Y + dst) = *reinterpret_cast<const uint4*>(Z + src);
    }
}

// U [n, D, H, W, C]: dY at (2o + q, 2p + q, 2r + q), zero elsewhere; one
// thread per (full-resolution voxel, 4-channel group), every element written.
template <typename T>
__global__ __launch_bounds__(RS_T) void upsample_kernel(const T* __restrict__ dY, T* __restrict__ U, int N, int D,
                                                        int H, int W, int Do, int Ho, int Wo, int C, int q)
{
    const int G = C / 4;
    const int64_t total = (int64_t)N * D * H * W * G;
    const int64_t stride = (int64_t)gridDim.x * RS_T;
    for (int64_t e = (int64_t)blockIdx.x * RS_T + threadIdx.x; e < total; e += stride) {
        const int g = (int)(e % G);
        int64_t v = e / G;
        const int w = (int)(v % W); v /= W;
        const int h = (int)(v % H); v /= H;
        const int d = (int)(v % D);
        const int n = (int)(v / D);
        const int od = d - q, oh = h - q, ow = w - q;
        const bool hit = od >= 0 && oh >= 0 && ow >= 0 && !(od & 1) && !(oh & 1) && !(ow & 1) && (od >> 1) < Do &&
                         (oh >> 1) < Ho && (ow >> 1) < Wo;
        if (sizeof(T) == 2) {
            uint2 val = make_uint2(0u, 0u);
            if (hit)
                val = *reinterpret_cast<const uint2*>(
                    dY + ((((int64_t)n * Do + (od >> 1)) * Ho + (oh >> 1)) * Wo + (ow >> 1)) * C + 4 * g);
            *reinterpret_cast<uint2*>(U + e * 4) = val;
        } else {
            uint4 val = make_uint4(0u, 0u, 0u, 0u);
            if (hit)
                val = *reinterpret_cast<const uint4*>(
                    dY + ((((int64_t)n * Do + (od >> 1)) * Ho + (oh >> 1)) * Wo + (ow >> 1)) * C + 4 * g);
            *reinterpret_cast<uint4*>(U + e * 4) = val;
        }
    }
}

__device__ __forceinline__ float lrelu_f(float z, float slope) { return z > 0.f ? z : slope * z; }

// P = (1/8) sum_window lrelu(Z); one thread per (pooled voxel, 4 channels).
// The eight terms are added in window order (a, b, e), then scaled.
template <typename T>
__global__ __launch_bounds__(RS_T) void avgpool_fwd_kernel(const T* __restrict__ Z, T* __restrict__ P, int N, int D,
                                                           int H, int W, int C, float slope)
{
    const int G = C / 4, Dp = D / 2, Hp = H / 2, Wp = W / 2;
    const int64_t total = (int64_t)N * Dp * Hp * Wp * G;
    const int64_t stride = (int64_t)gridDim.x * RS_T;
    for (int64_t e = (int64_t)blockIdx.x * RS_T + threadIdx.x; e < total; e += stride) {
        const int g = (int)(e % G);
        int64_t v = e / G;
        const int k = (int)(v % Wp); v /= Wp;
        const int j = (int)(v % Hp); v /= Hp;
        const int i = (int)(v % Dp);
        const int n = (int)(v / Dp);
        float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int pos = 0; pos < 8; ++pos) {
            const int a = pos >> 2, b = (pos >> 1) & 1, c = pos & 1;
            const T* zp = Z + ((((int64_t)n * D + 2 * i + a) * H + 2 * j + b) * W + 2 * k + c) * C + 4 * g;
#pragma unroll
            for (int r = 0; r < 4; ++r) s[r] += lrelu_f(Elem<T>::load(zp, r), slope);
        }
        const int64_t o = e * 4;
#pragma unroll
        for (int r = 0; r < 4; ++r) Elem<T>::store(P, o + r, s[r] * 0.125f);
    }
}

// dZ = lrelu'(Z) * dP / 8 at every window position.
template <typename T>
__global__ __launch_bounds__(RS_T) void avgpool_bwd_kernel(const T* __restrict__ dP, const T* __restrict__ Z,
                                                           T* __restrict__ dZ, int N, int D, int H, int W, int C,
                                                           float slope)
{
    const int G = C / 4;
    const int64_t total = (int64_t)N * D * H * W * G;
    const int64_t stride = (int64_t)gridDim.x * RS_T;
    for (int64_t e = (int64_t)blockIdx.x * RS_T + threadIdx.x; e < total; e += stride) {
        const int g = (int)(e % G);
        int64_t v = e / G;
        const int w = (int)(v % W); v /= W;
        const int h = (int)(v % H); v /= H;
        const int d = (int)(v % D);
        const int n = (int)(v / D);
        const int64_t pi = ((((int64_t)n * (D / 2) + d / 2) * (H / 2) + h / 2) * (W / 2) + w / 2) * C + 4 * g;
        const int64_t zi = e * 4;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float gp = Elem<T>::load(dP, pi + r) * 0.125f;
            const float z = Elem<T>::load(Z, zi + r);
            Elem<T>::store(dZ, zi + r, z > 0.f ? gp : gp * slope);
        }
    }
}

}  // namespace

template <typename T>
hipError_t launch_subsample(const T* Z, T* Y, const cf_dims& z, int Do, int Ho, int Wo, int q, hipStream_t s)
{
    const int64_t n = z.n * Do * Ho * Wo * (z.c / 4);
    hipLaunchKernelGGL(subsample_kernel<T>, dim3(grid_of(n)), dim3(RS_T), 0, s, Z, Y, (int)z.n, (int)z.d, (int)z.h,
                       (int)z.w, Do, Ho, Wo, (int)z.c, q);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_upsample(const T* dY, T* U, const cf_dims& z, int Do, int Ho, int Wo, int q, hipStream_t s)
{
    const int64_t n = z.n * z.d * z.h * z.w * (z.c / 4);
    hipLaunchKernelGGL(upsample_kernel<T>, dim3(grid_of(n)), dim3(RS_T), 0, s, dY, U, (int)z.n, (int)z.d, (int)z.h,
                       (int)z.w, Do, Ho, Wo, (int)z.c, q);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_avgpool_fwd(const T* Z, T* P, const cf_dims& z, float slope, hipStream_t s)
{
    const int64_t n = z.n * (z.d / 2) * (z.h / 2) * (z.w / 2) * (z.c / 4);
    hipLaunchKernelGGL(avgpool_fwd_kernel<T>, dim3(grid_of(n)), dim3(RS_T), 0, s, Z, P, (int)z.n, (int)z.d, (int)z.h,
                       (int)z.w, (int)z.c, slope);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_avgpool_bwd(const T* dP, const T* Z, T* dZ, const cf_dims& z, float slope, hipStream_t s)
{
    const int64_t n = z.n * z.d * z.h * z.w * (z.c / 4);
    hipLaunchKernelGGL(avgpool_bwd_kernel<T>, dim3(grid_of(n)), dim3(RS_T), 0, s, dP, Z, dZ, (int)z.n, (int)z.d,
                       (int)z.h, (int)z.w, (int)z.c, slope);
    return hipGetLastError();
}

#define CF_INST(T)                                                                                                   \
    template hipError_t launch_subsample<T>(const T*, T*, const cf_dims&, int, int, int, int, hipStream_t);         \
    template hipError_t launch_upsample<T>(const T*, T*, const cf_dims&, int, int, int, int, hipStream_t);          \
    template hipError_t launch_avgpool_fwd<T>(const T*, T*, const cf_dims&, float, hipStream_t);                    \
    template hipError_t launch_avgpool_bwd<T>(const T*, const T*, T*, const cf_dims&, float, hipStream_t);
CF_INST(float)
CF_INST(uint16_t)
#undef CF_INST

namespace {

// Y[v][c] = X[v][c] for c < cin, 0 for cin <= c < cinp (bf16, NDHWC);
// one thread per (voxel, 8-channel group), 16-byte loads and stores.
__global__ void pad_channels_kernel(const uint16_t* __restrict__ X, uint16_t* __restrict__ Y, int64_t nvox, int cin,
                                    int cinp)
{
    const int gp = cinp / 8, gi = cin / 8;
    const int64_t total = nvox * gp;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t v = i / gp;
        const int g = (int)(i - v * gp);
        uint4 val = make_uint4(0u, 0u, 0u, 0u);
        if (g < gi) val = *reinterpret_cast<const uint4*>(X + v * cin + 8 * g);
        *reinterpret_cast<uint4*>(Y + v * cinp + 8 * g) = val;
    }
}

// dW[t][ci][co] = dWp[t][ci][co] for ci < cin (the rows of the padded input
// channels are dropped).
__global__ void unpad_dw_kernel(const float* __restrict__ dWp, float* __restrict__ dW, int cin, int cinp, int cout)
{
    const int64_t total = (int64_t)27 * cin * cout;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = e / ((int64_t)cin * cout);
        const int64_t r = e - t * cin * cout;
        dW[e] = dWp[t * cinp * cout + r];
    }
}

unsigned grid_for(int64_t n)
{
    int64_t b = (n + 255) / 256;
    if (b > 65536) b = 65536;
    return (unsigned)(b < 1 ? 1 : b);
}

}  // namespace

hipError_t launch_pad_channels(const uint16_t* X, uint16_t* Y, int64_t nvox, int cin, int cinp, hipStream_t s)
{
    if (cin % 8 || cinp % 8 || cinp < cin) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pad_channels_kernel, dim3(grid_for(nvox * (cinp / 8))), dim3(256), 0, s, X, Y, nvox, cin, cinp);
    return hipGetLastError();
}

hipError_t launch_unpad_dw(const float* dWp, float* dW, int cin, int cinp, int cout, hipStream_t s)
{
    hipLaunchKernelGGL(unpad_dw_kernel, dim3(grid_for((int64_t)27 * cin * cout)), dim3(256), 0, s, dWp, dW, cin, cinp,
                       cout);
    return hipGetLastError();
}

}  // namespace cf
