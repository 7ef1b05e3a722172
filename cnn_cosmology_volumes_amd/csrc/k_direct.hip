// Direct (non-MFMA) 3^3 convolution kernels: the fp32 path and any channel
// counts the MFMA kernels do not cover.  Same definitions as the MFMA path
// (Oyama et al., Sec. IV / Table I: stride 1, "same" zero padding, no bias):
//   forward  Y[v, co] = sum_{tap, ci} X[v + off(tap), ci] * W[tap][ci][co]
//   backward-weight dW[tap][ci][co] = sum_v X[v + off(tap), ci] * dY[v, co]
// Backward-data reuses the forward kernel with tap-flipped, channel-swapped
// weights.  Accumulation is fp32 in a fixed order.
#include "cf_internal.h"

namespace cf {

namespace {

// One thread per (voxel, group of 4 output channels); weights are read
// through L1 (all threads of a block share the same co group order).
template <typename T>
__global__ void conv_direct_kernel(const T* __restrict__ X, const T* __restrict__ Wt, T* __restrict__ Y,
                                   int N, int D, int H, int W, int Cin, int Cout)
{
    const int cg = (Cout + 3) / 4;
    const int64_t total = (int64_t)N * D * H * W * cg;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
        const int g = (int)(e % cg);
        int64_t v = e / cg;
        const int w = (int)(v % W); v /= W;
        const int h = (int)(v % H); v /= H;
        const int d = (int)(v % D);
        const int n = (int)(v / D);
        const int co0 = 4 * g;
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int kd = 0; kd < 3; ++kd) {
            const int id = d + kd - 1;
            if ((unsigned)id >= (unsigned)D) continue;
            for (int kh = 0; kh < 3; ++kh) {
                const int ih = h + kh - 1;
                if ((unsigned)ih >= (unsigned)H) continue;
                for (int kw = 0; kw < 3; ++kw) {
                    const int iw = w + kw - 1;
                    if ((unsigned)iw >= (unsigned)W) continue;
                    const T* xp = X + ((((int64_t)n * D + id) * H + ih) * W + iw) * Cin;
                    const T* wp = Wt + (int64_t)((kd * 3 + kh) * 3 + kw) * Cin * Cout;
                    for (int ci = 0; ci < Cin; ++ci) {
                        const float xv = Elem<T>::load(xp, ci);
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (co0 + r < Cout) acc[r] = fmaf(xv, Elem<T>::load(wp, (int64_t)ci * Cout + co0 + r), acc[r]);
                    }
                }
            }
        }
        const int64_t ob = ((((int64_t)n * D + d) * H + h) * W + w) * Cout;
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (co0 + r < Cout) Elem<T>::store(Y, ob + co0 + r, acc[r]);
    }
}

// part[split][tap][ci][co]: one thread per dW element, voxels of one split.
template <typename T>
__global__ void wgrad_direct_kernel(const T* __restrict__ X, const T* __restrict__ dY, float* __restrict__ part,
                                    int N, int D, int H, int W, int Cin, int Cout, int64_t vox_per_split)
{
    const int64_t ndw = (int64_t)27 * Cin * Cout;
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= ndw) return;
    const int co = (int)(e % Cout);
    const int ci = (int)((e / Cout) % Cin);
    const int tap = (int)(e / ((int64_t)Cout * Cin));
    const int kd = tap / 9, kh = (tap / 3) % 3, kw = tap % 3;
    const int64_t nvox = (int64_t)N * D * H * W;
    const int64_t v0 = (int64_t)blockIdx.y * vox_per_split;
    const int64_t v1 = min(v0 + vox_per_split, nvox);
    float s = 0.f;
    for (int64_t v = v0; v < v1; ++v) {
        int64_t r = v;
        const int w = (int)(r % W); r /= W;
        const int h = (int)(r % H); r /= H;
        const int d = (int)(r % D);
        const int n = (int)(r / D);
        const int id = d + kd - 1, ih = h + kh - 1, iw = w + kw - 1;
        if ((unsigned)id >= (unsigned)D || (unsigned)ih >= (unsigned)H || (unsigned)iw >= (unsigned)W) continue;
        const float xv = Elem<T>::load(X, ((((int64_t)n * D + id) * H + ih) * W + iw) * Cin + ci);
        s = fmaf(xv, Elem<T>::load(dY, v * Cout + co), s);
    }
    part[(int64_t)blockIdx.y * ndw + e] = s;
}

__global__ void wgrad_direct_reduce(const float* __restrict__ part, float* __restrict__ dW, int64_t n, int splits)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float s = 0.f;
    for (int k = 0; k < splits; ++k) s += part[(int64_t)k * n + i];
    dW[i] = s;
}

int64_t direct_splits(const cf_dims& x) {
    const int64_t nvox = x.n * x.d * x.h * x.w;
    int64_t sp = nvox / 2048;
    if (sp < 1) sp = 1;
    if (sp > 256) sp = 256;
    return sp;
}

}  // namespace

template <typename T>
hipError_t launch_conv_direct(const T* X, const T* W, T* Y, const cf_dims& x, int cout, hipStream_t s)
{
    const int64_t total = x.n * x.d * x.h * x.w * ((cout + 3) / 4);
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(conv_direct_kernel<T>, dim3((unsigned)blocks), dim3(256), 0, s, X, W, Y, (int)x.n, (int)x.d,
                       (int)x.h, (int)x.w, (int)x.c, cout);
    return hipGetLastError();
}

template <typename T>
size_t wgrad_direct_part_bytes(const cf_dims& x, int cout)
{
    return (size_t)direct_splits(x) * 27 * (size_t)x.c * (size_t)cout * sizeof(float);
}

template <typename T>
hipError_t launch_wgrad_direct(const T* X, const T* dY, float* part, float* dW, const cf_dims& x, int cout,
                               hipStream_t s)
{
    const int64_t sp = direct_splits(x);
    const int64_t nvox = x.n * x.d * x.h * x.w;
    const int64_t per = (nvox + sp - 1) / sp;
    const int64_t ndw = (int64_t)27 * x.c * cout;
    hipLaunchKernelGGL(wgrad_direct_kernel<T>, dim3((unsigned)((ndw + 255) / 256), (unsigned)sp), dim3(256), 0, s, X,
                       dY, part, (int)x.n, (int)x.d, (int)x.h, (int)x.w, (int)x.c, cout, per);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(wgrad_direct_reduce, dim3((unsigned)((ndw + 255) / 256)), dim3(256), 0, s, part, dW, ndw,
                       (int)sp);
    return hipGetLastError();
}

template hipError_t launch_conv_direct<float>(const float*, const float*, float*, const cf_dims&, int, hipStream_t);
template hipError_t launch_conv_direct<uint16_t>(const uint16_t*, const uint16_t*, uint16_t*, const cf_dims&, int,
                                                 hipStream_t);
template size_t wgrad_direct_part_bytes<float>(const cf_dims&, int);
template size_t wgrad_direct_part_bytes<uint16_t>(const cf_dims&, int);
template hipError_t launch_wgrad_direct<float>(const float*, const float*, float*, float*, const cf_dims&, int,
                                               hipStream_t);
template hipError_t launch_wgrad_direct<uint16_t>(const uint16_t*, const uint16_t*, float*, float*, const cf_dims&,
                                                  int, hipStream_t);

}  // namespace cf
