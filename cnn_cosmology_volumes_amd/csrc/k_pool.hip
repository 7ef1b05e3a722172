// Leaky ReLU + 2^3 stride-2 max pooling, forward and backward, and the
// elementwise leaky ReLU.  Bandwidth-bound kernels over NDHWC tensors.
//
// Forward (CosmoFlow, Sec. III-A: leaky ReLU after every conv; pooling 2^3
// with stride 2 as in Oyama et al., Table I, taken as max pooling):
//   P = max over the 2^3 window of lrelu(Z), idx = window position a*4+b*2+e
//   of the first strict maximum in (a,b,e) lexicographic order.
// lrelu is strictly increasing, so the maximum is found on Z and lrelu is
// applied once to it; the comparison is made in fp32 on the stored values.
// Backward: dZ at the recorded position = dP * (P > 0 ? 1 : slope), all
// other seven positions of the window zero (dZ is written densely).
#include "cf_internal.h"

namespace cf {

namespace {

template <typename T> struct Vec;
template <> struct Vec<uint16_t> {   // 8 bf16 = 16 bytes
    static constexpr int W = 8;
    typedef uint4 raw;
    __device__ __forceinline__ static void unpack(const raw& r, float* f) {
        const uint32_t u[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) { f[2 * i] = __uint_as_float(u[i] << 16); f[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u); }
    }
    __device__ __forceinline__ static raw pack(const float* f) {
        return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
    }
};
template <> struct Vec<float> {      // 4 fp32 = 16 bytes
    static constexpr int W = 4;
    typedef float4 raw;
    __device__ __forceinline__ static void unpack(const raw& r, float* f) { f[0] = r.x; f[1] = r.y; f[2] = r.z; f[3] = r.w; }
    __device__ __forceinline__ static raw pack(const float* f) { return make_float4(f[0], f[1], f[2], f[3]); }
};

// Vector path: C % Vec<T>::W == 0.  One thread per (pooled voxel, channel vector).
template <typename T>
__global__ void pool_fwd_vec(const T* __restrict__ Z, T* __restrict__ P, uint8_t* __restrict__ idx, int N, int D,
                             int H, int W, int C, float slope)
{
    constexpr int V = Vec<T>::W;
    typedef typename Vec<T>::raw raw;
    const int Dp = D / 2, Hp = H / 2, Wp = W / 2, cg = C / V;
    const int64_t total = (int64_t)N * Dp * Hp * Wp * cg;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
        const int g = (int)(e % cg);
        int64_t r = e / cg;
        const int k = (int)(r % Wp); r /= Wp;
        const int j = (int)(r % Hp); r /= Hp;
        const int i = (int)(r % Dp);
        const int n = (int)(r / Dp);
        float best[V], cur[V];
        uint8_t bi[V];
        raw win[8];
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int a = p >> 2, b = (p >> 1) & 1, c = p & 1;
            const int64_t vox = (((int64_t)n * D + 2 * i + a) * H + 2 * j + b) * W + 2 * k + c;
            win[p] = *reinterpret_cast<const raw*>(Z + vox * C + g * V);
        }
        Vec<T>::unpack(win[0], best);
#pragma unroll
        for (int c = 0; c < V; ++c) bi[c] = 0;
#pragma unroll
        for (int p = 1; p < 8; ++p) {
            Vec<T>::unpack(win[p], cur);
#pragma unroll
            for (int c = 0; c < V; ++c)
                if (cur[c] > best[c]) { best[c] = cur[c]; bi[c] = (uint8_t)p; }
        }
#pragma unroll
        for (int c = 0; c < V; ++c) best[c] = best[c] > 0.f ? best[c] : slope * best[c];
        const int64_t o = e * V;
        *reinterpret_cast<raw*>(P + o) = Vec<T>::pack(best);
        if (V == 8) {
            uint2 ib;
            ib.x = bi[0] | (bi[1] << 8) | (bi[2] << 16) | ((uint32_t)bi[3] << 24);
            ib.y = bi[4 % V] | (bi[5 % V] << 8) | (bi[6 % V] << 16) | ((uint32_t)bi[7 % V] << 24);
            *reinterpret_cast<uint2*>(idx + o) = ib;
        } else {
            *reinterpret_cast<uint32_t*>(idx + o) = bi[0] | (bi[1] << 8) | (bi[2 % V] << 16) | ((uint32_t)bi[3 % V] << 24);
        }
    }
}

template <typename T>
__global__ void pool_bwd_vec(const T* __restrict__ dP, const T* __restrict__ P, const uint8_t* __restrict__ idx,
                             T* __restrict__ dZ, int N, int D, int H, int W, int C, float slope)
{
    constexpr int V = Vec<T>::W;
    typedef typename Vec<T>::raw raw;
    const int Dp = D / 2, Hp = H / 2, Wp = W / 2, cg = C / V;
    const int64_t total = (int64_t)N * Dp * Hp * Wp * cg;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
        const int g = (int)(e % cg);
        int64_t r = e / cg;
        const int k = (int)(r % Wp); r /= Wp;
        const int j = (int)(r % Hp); r /= Hp;
        const int i = (int)(r % Dp);
        const int n = (int)(r / Dp);
        const int64_t o = e * V;
        float gv[V], pv[V], outv[V];
        Vec<T>::unpack(*reinterpret_cast<const raw*>(dP + o), gv);
        Vec<T>::unpack(*reinterpret_cast<const raw*>(P + o), pv);
        uint8_t bi[V];
        if (V == 8) {
            const uint2 ib = *reinterpret_cast<const uint2*>(idx + o);
#pragma unroll
            for (int c = 0; c < 4; ++c) { bi[c] = (ib.x >> (8 * c)) & 0xff; bi[(c + 4) % V] = (ib.y >> (8 * c)) & 0xff; }
        } else {
            const uint32_t ib = *reinterpret_cast<const uint32_t*>(idx + o);
#pragma unroll
            for (int c = 0; c < V; ++c) bi[c] = (ib >> (8 * c)) & 0xff;
        }
#pragma unroll
        for (int c = 0; c < V; ++c) gv[c] = pv[c] > 0.f ? gv[c] : slope * gv[c];
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const int a = p >> 2, b = (p >> 1) & 1, c2 = p & 1;
#pragma unroll
            for (int c = 0; c < V; ++c) outv[c] = (bi[c] == p) ? gv[c] : 0.f;
            const int64_t vox = (((int64_t)n * D + 2 * i + a) * H + 2 * j + b) * W + 2 * k + c2;
            *reinterpret_cast<raw*>(dZ + vox * C + g * V) = Vec<T>::pack(outv);
        }
    }
}

// Scalar fallbacks for channel counts that are not a multiple of the vector width.
template <typename T>
__global__ void pool_fwd_scalar(const T* __restrict__ Z, T* __restrict__ P, uint8_t* __restrict__ idx, int N, int D,
                                int H, int W, int C, float slope)
{
    const int Dp = D / 2, Hp = H / 2, Wp = W / 2;
    const int64_t total = (int64_t)N * Dp * Hp * Wp * C;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
        const int c = (int)(e % C);
        int64_t r = e / C;
        const int k = (int)(r % Wp); r /= Wp;
        const int j = (int)(r % Hp); r /= Hp;
        const int i = (int)(r % Dp);
        const int n = (int)(r / Dp);
        float best = 0.f;
        int bi = 0;
        for (int p = 0; p < 8; ++p) {
            const int a = p >> 2, b = (p >> 1) & 1, cc = p & 1;
            const int64_t vox = (((int64_t)n * D + 2 * i + a) * H + 2 * j + b) * W + 2 * k + cc;
            const float v = Elem<T>::load(Z, vox * C + c);
            if (p == 0 || v > best) { best = v; bi = p; }
        }
        Elem<T>::store(P, e, best > 0.f ? best : slope * best);
        idx[e] = (uint8_t)bi;
    }
}

template <typename T>
__global__ void pool_bwd_scalar(const T* __restrict__ dP, const T* __restrict__ P, const uint8_t* __restrict__ idx,
                                T* __restrict__ dZ, int N, int D, int H, int W, int C, float slope)
{
    const int Dp = D / 2, Hp = H / 2, Wp = W / 2;
    const int64_t total = (int64_t)N * Dp * Hp * Wp * C;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
        const int c = (int)(e % C);
        int64_t r = e / C;
        const int k = (int)(r % Wp); r /= Wp;
        const int j = (int)(r % Hp); r /= Hp;
        const int i = (int)(r % Dp);
        const int n = (int)(r / Dp);
        const float pv = Elem<T>::load(P, e);
        float g = Elem<T>::load(dP, e);
        g = pv > 0.f ? g : slope * g;
        const int bi = idx[e];
        for (int p = 0; p < 8; ++p) {
            const int a = p >> 2, b = (p >> 1) & 1, cc = p & 1;
            const int64_t vox = (((int64_t)n * D + 2 * i + a) * H + 2 * j + b) * W + 2 * k + cc;
            Elem<T>::store(dZ, vox * C + c, p == bi ? g : 0.f);
        }
    }
}

template <typename T>
__global__ void lrelu_kernel(const T* __restrict__ x, const T* __restrict__ dy, T* __restrict__ out, int64_t n,
                             float slope)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const float v = Elem<T>::load(x, i);
        if (dy) {
            const float g = Elem<T>::load(dy, i);
            Elem<T>::store(out, i, v > 0.f ? g : slope * g);
        } else {
            Elem<T>::store(out, i, v > 0.f ? v : slope * v);
        }
    }
}

unsigned grid_for(int64_t total) {
    int64_t b = (total + 255) / 256;
    if (b > 262144) b = 262144;
    if (b < 1) b = 1;
    return (unsigned)b;
}

}  // namespace

template <typename T>
hipError_t launch_pool_fwd(const T* Z, T* P, uint8_t* idx, const cf_dims& z, float slope, hipStream_t s)
{
    const int64_t pooled = z.n * (z.d / 2) * (z.h / 2) * (z.w / 2);
    if (z.c % Vec<T>::W == 0) {
        hipLaunchKernelGGL(pool_fwd_vec<T>, dim3(grid_for(pooled * (z.c / Vec<T>::W))), dim3(256), 0, s, Z, P, idx,
                           (int)z.n, (int)z.d, (int)z.h, (int)z.w, (int)z.c, slope);
    } else {
        hipLaunchKernelGGL(pool_fwd_scalar<T>, dim3(grid_for(pooled * z.c)), dim3(256), 0, s, Z, P, idx, (int)z.n,
                           (int)z.d, (int)z.h, (int)z.w, (int)z.c, slope);
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_pool_bwd(const T* dP, const T* P, const uint8_t* idx, T* dZ, const cf_dims& z, float slope,
                           hipStream_t s)
{
    const int64_t pooled = z.n * (z.d / 2) * (z.h / 2) * (z.w / 2);
    if (z.c % Vec<T>::W == 0) {
        hipLaunchKernelGGL(pool_bwd_vec<T>, dim3(grid_for(pooled * (z.c / Vec<T>::W))), dim3(256), 0, s, dP, P, idx,
                           dZ, (int)z.n, (int)z.d, (int)z.h, (int)z.w, (int)z.c, slope);
    } else {
        hipLaunchKernelGGL(pool_bwd_scalar<T>, dim3(grid_for(pooled * z.c)), dim3(256), 0, s, dP, P, idx, dZ,
                           (int)z.n, (int)z.d, (int)z.h, (int)z.w, (int)z.c, slope);
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_lrelu(const T* x, const T* dy, T* out, int64_t n, float slope, hipStream_t s)
{
    hipLaunchKernelGGL(lrelu_kernel<T>, dim3(grid_for(n)), dim3(256), 0, s, x, dy, out, n, slope);
    return hipGetLastError();
}

template hipError_t launch_pool_fwd<float>(const float*, float*, uint8_t*, const cf_dims&, float, hipStream_t);
template hipError_t launch_pool_fwd<uint16_t>(const uint16_t*, uint16_t*, uint8_t*, const cf_dims&, float, hipStream_t);
template hipError_t launch_pool_bwd<float>(const float*, const float*, const uint8_t*, float*, const cf_dims&, float,
                                           hipStream_t);
template hipError_t launch_pool_bwd<uint16_t>(const uint16_t*, const uint16_t*, const uint8_t*, uint16_t*,
                                              const cf_dims&, float, hipStream_t);
template hipError_t launch_lrelu<float>(const float*, const float*, float*, int64_t, float, hipStream_t);
template hipError_t launch_lrelu<uint16_t>(const uint16_t*, const uint16_t*, uint16_t*, int64_t, float, hipStream_t);

}  // namespace cf
