// Training-mode batch normalisation of NDHWC activations over (N, D, H, W),
// per channel: statistics from each channel's sum and sum of squares, then
// y = (x - mean) * (gamma * invstd) + beta; and its backward.
//
// Each reduction is a block pass over BN_VPB voxels writing per-channel
// partial sums (fp32 within the block, combined in a fixed order), then one
// wave per channel adding the blocks' partials in fp64 in block order: no
// atomics, so results are reproducible bit for bit.  Memory-bound: the
// forward reads x twice and writes y; the backward reads x and dy twice and
// writes dx.
#include "cf_internal.h"

namespace cf {
namespace {

constexpr int BN_T = 256;       // threads per block
constexpr int BN_VPB = 4096;    // voxels per reduction block

template <typename T> struct V4;
template <> struct V4<float> {
    __device__ __forceinline__ static float4 load(const float* p) { return *reinterpret_cast<const float4*>(p); }
    __device__ __forceinline__ static void store(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
};
template <> struct V4<uint16_t> {
    __device__ __forceinline__ static float4 load(const uint16_t* p)
    {
        const uint2 u = *reinterpret_cast<const uint2*>(p);
        return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                           __uint_as_float(u.y & 0xffff0000u));
    }
    __device__ __forceinline__ static void store(uint16_t* p, float4 v)
    {
        *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
    }
};

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }

int64_t n_blocks(int64_t nvox) { return (nvox + BN_VPB - 1) / BN_VPB; }

// Per-block partial sums over BN_VPB voxels: forward (BWD = false) x and
// x^2; backward dy and dy * xhat.  part[block][0..C) and [C..2C).
template <typename T, bool BWD>
__global__ __launch_bounds__(BN_T) void bn_reduce_kernel(const T* __restrict__ X, const T* __restrict__ dY,
                                                         const float* __restrict__ mean,
                                                         const float* __restrict__ invstd, float* __restrict__ part,
                                                         int64_t nvox, int C)
{
    __shared__ float lds[2 * 4 * BN_T];
    const int G = C >> 2;             // 4-channel groups
    const int R = BN_T / G;           // voxel rows in flight
    const int r = (int)threadIdx.x / G, g = (int)threadIdx.x % G;
    float4 s1 = make_float4(0.f, 0.f, 0.f, 0.f), s2 = s1;
    if (r < R) {
        const int64_t v0 = (int64_t)blockIdx.x * BN_VPB;
        const int64_t v1 = min(v0 + BN_VPB, nvox);
        float4 mu = s1, is = s1;
        if (BWD) {
            mu = ld4(mean + 4 * g);
            is = ld4(invstd + 4 * g);
        }
        for (int64_t v = v0 + r; v < v1; v += R) {
            const float4 x = V4<T>::load(X + v * C + 4 * g);
            if (!BWD) {
                s1.x += x.x; s1.y += x.y; s1.z += x.z; s1.w += x.w;
                s2.x += x.x * x.x; s2.y += x.y * x.y; s2.z += x.z * x.z; s2.w += x.w * x.w;
            } else {
                const float4 d = V4<T>::load(dY + v * C + 4 * g);
                s1.x += d.x; s1.y += d.y; s1.z += d.z; s1.w += d.w;
                s2.x += d.x * ((x.x - mu.x) * is.x);
                s2.y += d.y * ((x.y - mu.y) * is.y);
                s2.z += d.z * ((x.z - mu.z) * is.z);
                s2.w += d.w * ((x.w - mu.w) * is.w);
            }
        }
        *reinterpret_cast<float4*>(&lds[r * C + 4 * g]) = s1;
        *reinterpret_cast<float4*>(&lds[R * C + r * C + 4 * g]) = s2;
    }
    __syncthreads();
    for (int c = (int)threadIdx.x; c < C; c += BN_T) {
        float a = 0.f, b = 0.f;
        for (int rr = 0; rr < R; ++rr) {
            a += lds[rr * C + c];
            b += lds[R * C + rr * C + c];
        }
        part[(int64_t)blockIdx.x * 2 * C + c] = a;
        part[(int64_t)blockIdx.x * 2 * C + C + c] = b;
    }
}

// One wave per channel: the blocks' partials in fp64, block order.
__device__ __forceinline__ void sum_parts(const float* part, int64_t nb, int C, int c, double& s, double& q)
{
    s = 0.0;
    q = 0.0;
    for (int64_t b = threadIdx.x; b < nb; b += 64) {
        s += (double)part[b * 2 * C + c];
        q += (double)part[b * 2 * C + C + c];
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        s += __shfl_xor(s, m, 64);
        q += __shfl_xor(q, m, 64);
    }
}

__global__ __launch_bounds__(64) void bn_fwd_finalize(const float* __restrict__ part, int64_t nb, int C, int64_t M,
                                                      const float* __restrict__ gamma, float eps,
                                                      float* __restrict__ mean, float* __restrict__ invstd,
                                                      float* __restrict__ coef)
{
    const int c = blockIdx.x;
    double s, q;
    sum_parts(part, nb, C, c, s, q);
    if (threadIdx.x == 0) {
        const double mu = s / (double)M;
        double var = q / (double)M - mu * mu;
        if (var < 0.0) var = 0.0;
        const double is = 1.0 / sqrt(var + (double)eps);
        mean[c] = (float)mu;
        invstd[c] = (float)is;
        coef[c] = (float)((double)gamma[c] * is);
    }
}

__global__ __launch_bounds__(64) void bn_bwd_finalize(const float* __restrict__ part, int64_t nb, int C, int64_t M,
                                                      const float* __restrict__ gamma,
                                                      const float* __restrict__ invstd, float* __restrict__ dgamma,
                                                      float* __restrict__ dbeta, float* __restrict__ coef)
{
    const int c = blockIdx.x;
    double s, q;
    sum_parts(part, nb, C, c, s, q);
    if (threadIdx.x == 0) {
        dbeta[c] = (float)s;
        dgamma[c] = (float)q;
        coef[c] = (float)((double)gamma[c] * (double)invstd[c]);
        coef[C + c] = (float)(s / (double)M);
        coef[2 * C + c] = (float)(q / (double)M);
    }
}

// y = (x - mean) * coef + beta, 4 channels per thread.
template <typename T>
__global__ __launch_bounds__(BN_T) void bn_apply_kernel(const T* __restrict__ X, const float* __restrict__ mean,
                                                        const float* __restrict__ coef,
                                                        const float* __restrict__ beta, T* __restrict__ Y,
                                                        int64_t ngroups, int G)
{
    const int64_t stride = (int64_t)gridDim.x * BN_T;
    for (int64_t i = (int64_t)blockIdx.x * BN_T + threadIdx.x; i < ngroups; i += stride) {
        const int g = (int)(i % G);
        const float4 x = V4<T>::load(X + 4 * i);
        const float4 mu = ld4(mean + 4 * g), a = ld4(coef + 4 * g), b = ld4(beta + 4 * g);
        V4<T>::store(Y + 4 * i, make_float4((x.x - mu.x) * a.x + b.x, (x.y - mu.y) * a.y + b.y,
                                            (x.z - mu.z) * a.z + b.z, (x.w - mu.w) * a.w + b.w));
    }
}

// dx = gamma invstd (dy - sum(dy)/M - xhat sum(dy xhat)/M).
template <typename T>
__global__ __launch_bounds__(BN_T) void bn_dx_kernel(const T* __restrict__ X, const T* __restrict__ dY,
                                                     const float* __restrict__ mean, const float* __restrict__ invstd,
                                                     const float* __restrict__ coef, T* __restrict__ dX,
                                                     int64_t ngroups, int G)
{
    const int C = 4 * G;
    const int64_t stride = (int64_t)gridDim.x * BN_T;
    for (int64_t i = (int64_t)blockIdx.x * BN_T + threadIdx.x; i < ngroups; i += stride) {
        const int g = (int)(i % G);
        const float4 x = V4<T>::load(X + 4 * i), d = V4<T>::load(dY + 4 * i);
        const float4 mu = ld4(mean + 4 * g), is = ld4(invstd + 4 * g);
        const float4 k1 = ld4(coef + 4 * g), k2 = ld4(coef + C + 4 * g), k3 = ld4(coef + 2 * C + 4 * g);
        V4<T>::store(dX + 4 * i, make_float4(k1.x * (d.x - k2.x - ((x.x - mu.x) * is.x) * k3.x),
                                             k1.y * (d.y - k2.y - ((x.y - mu.y) * is.y) * k3.y),
                                             k1.z * (d.z - k2.z - ((x.z - mu.z) * is.z) * k3.z),
                                             k1.w * (d.w - k2.w - ((x.w - mu.w) * is.w) * k3.w)));
    }
}

size_t up256b(size_t b) { return (b + 255) & ~(size_t)255; }

unsigned grid_for(int64_t ngroups)
{
    int64_t b = (ngroups + BN_T - 1) / BN_T;
    if (b > 8192) b = 8192;
    return (unsigned)(b < 1 ? 1 : b);
}

}  // namespace

size_t bn_ws_bytes(const cf_dims& x)
{
    const int64_t nvox = x.n * x.d * x.h * x.w;
    return up256b((size_t)n_blocks(nvox) * 2 * x.c * sizeof(float)) + up256b((size_t)3 * x.c * sizeof(float));
}

template <typename T>
hipError_t launch_bn_fwd(const T* X, const float* gamma, const float* beta, float eps, T* Y, float* mean,
                         float* invstd, const cf_dims& x, void* ws, hipStream_t s)
{
    const int64_t nvox = x.n * x.d * x.h * x.w, nb = n_blocks(nvox);
    const int C = (int)x.c;
    float* part = (float*)ws;
    float* coef = (float*)((char*)ws + up256b((size_t)nb * 2 * C * sizeof(float)));
    hipLaunchKernelGGL((bn_reduce_kernel<T, false>), dim3((unsigned)nb), dim3(BN_T), 0, s, X, (const T*)nullptr,
                       (const float*)nullptr, (const float*)nullptr, part, nvox, C);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bn_fwd_finalize, dim3((unsigned)C), dim3(64), 0, s, (const float*)part, nb, C, nvox, gamma, eps,
                       mean, invstd, coef);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(bn_apply_kernel<T>, dim3(grid_for(nvox * (C / 4))), dim3(BN_T), 0, s, X, (const float*)mean,
                       (const float*)coef, beta, Y, nvox * (C / 4), C / 4);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_bn_bwd(const T* X, const T* dY, const float* gamma, const float* mean, const float* invstd, T* dX,
                         float* dgamma, float* dbeta, const cf_dims& x, void* ws, hipStream_t s)
{
    const int64_t nvox = x.n * x.d * x.h * x.w, nb = n_blocks(nvox);
    const int C = (int)x.c;
    float* part = (float*)ws;
    float* coef = (float*)((char*)ws + up256b((size_t)nb * 2 * C * sizeof(float)));
    hipLaunchKernelGGL((bn_reduce_kernel<T, true>), dim3((unsigned)nb), dim3(BN_T), 0, s, X, dY, mean, invstd, part,
                       nvox, C);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bn_bwd_finalize, dim3((unsigned)C), dim3(64), 0, s, (const float*)part, nb, C, nvox, gamma,
                       invstd, dgamma, dbeta, coef);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(bn_dx_kernel<T>, dim3(grid_for(nvox * (C / 4))), dim3(BN_T), 0, s, X, dY, mean, invstd,
                       (const float*)coef, dX, nvox * (C / 4), C / 4);
    return hipGetLastError();
}

template hipError_t launch_bn_fwd<float>(const float*, const float*, const float*, float, float*, float*, float*,
                                         const cf_dims&, void*, hipStream_t);
template hipError_t launch_bn_fwd<uint16_t>(const uint16_t*, const float*, const float*, float, uint16_t*, float*,
                                            float*, const cf_dims&, void*, hipStream_t);
template hipError_t launch_bn_bwd<float>(const float*, const float*, const float*, const float*, const float*, float*,
                                         float*, float*, const cf_dims&, void*, hipStream_t);
template hipError_t launch_bn_bwd<uint16_t>(const uint16_t*, const uint16_t*, const float*, const float*,
                                            const float*, uint16_t*, float*, float*, const cf_dims&, void*,
                                            hipStream_t);

}  // namespace cf
