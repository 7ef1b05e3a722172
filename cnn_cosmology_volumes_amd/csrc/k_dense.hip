// Dense head, loss and optimizer kernels (fp32; latency-bound, a few MFLOP).
//
//   forward : pre[b,o] = sum_i X[b,i] W[i,o] + bias[o];  Y = lrelu(pre) or pre
//             (fully connected layers with leaky ReLU except the last one,
//             Oyama et al., Sec. IV; CosmoFlow, Sec. III-A)
//   backward: dpre = dY * lrelu'(pre); dW = X^T dpre; db = sum_b dpre;
//             dX = dpre W^T (chain rule of the forward)
//   MSE     : L = mean (yhat - t)^2 over B*K, dyhat = 2 (yhat - t) / (B*K)
//             (Oyama et al., Sec. IV: mean squared error loss)
//   SGD     : W <- W - lr * dW  (Oyama et al., Sec. II-A)
// Every reduction is split into fixed pieces combined in a fixed order, so
// results are reproducible bit for bit.
#include "cf_internal.h"

namespace cf {

namespace {

constexpr int DB = 8;        // batch rows per block
constexpr int DO = 64;       // output columns per block
constexpr int DI = 4;        // input lanes per block
constexpr int DK = 128;      // input rows per split

__device__ __forceinline__ float xin(const float* X, const uint16_t* Xb, int64_t i) {
    return Xb ? bf2f(Xb[i]) : X[i];
}

__device__ __forceinline__ float gate(float dy, float pre, float slope) {
    return (slope >= 0.f && !(pre > 0.f)) ? slope * dy : dy;
}

// part[ks][b][o] = sum_{i in split ks} X[b,i] W[i,o].  The block's input
// rows (DB x DK values) are staged in LDS once; each thread then streams W
// rows (coalesced over o) and accumulates DB batch rows.
__global__ __launch_bounds__(DO * DI)
void dense_fwd_partial(const float* __restrict__ X, const uint16_t* __restrict__ Xb, const float* __restrict__ W,
                       float* __restrict__ part, int B, int In, int Out)
{
    __shared__ float xs[DB][DK];
    __shared__ float red[DI][DB][DO];
    const int ol = threadIdx.x % DO, il = threadIdx.x / DO;
    const int o = blockIdx.x * DO + ol;
    const int ks = blockIdx.y;
    const int b0 = blockIdx.z * DB;
    const int nb = min(DB, B - b0);
    const int i0 = ks * DK, i1 = min(In, i0 + DK);
    for (int e = threadIdx.x; e < DB * DK; e += DO * DI) {
        const int b = e / DK, i = i0 + e % DK;
        xs[b][e % DK] = (b < nb && i < i1) ? xin(X, Xb, (int64_t)(b0 + b) * In + i) : 0.f;
    }
    __syncthreads();
    float acc[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) acc[b] = 0.f;
    if (o < Out) {
        // rows i0+il, i0+il+DI, ... in increasing order; the weight loads of
        // eight rows are issued together (latency, not bandwidth, bounds this)
        constexpr int U = 8;
        for (int i = i0 + il; i < i1; i += DI * U) {
            float w[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int ii = i + u * DI;
                w[u] = ii < i1 ? W[(int64_t)ii * Out + o] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int ii = i + u * DI;
                if (ii < i1) {
#pragma unroll
                    for (int b = 0; b < DB; ++b) acc[b] = fmaf(xs[b][ii - i0], w[u], acc[b]);
                }
            }
        }
    }
#pragma unroll
    for (int b = 0; b < DB; ++b) red[il][b][ol] = acc[b];
    __syncthreads();
    if (il == 0 && o < Out) {
        for (int b = 0; b < nb; ++b) {
            float s = red[0][b][ol];
#pragma unroll
            for (int k = 1; k < DI; ++k) s += red[k][b][ol];
            part[((int64_t)ks * B + b0 + b) * Out + o] = s;
        }
    }
}

// One wave per output element: lane l sums the splits l, l + 64, ... in
// increasing order, then the 64 lane sums are combined by a fixed butterfly.
__global__ __launch_bounds__(256)
void dense_fwd_finalize(const float* __restrict__ part, const float* __restrict__ bias, float slope,
                        float* __restrict__ pre, float* __restrict__ Y, int B, int Out, int nks)
{
    const int lane = threadIdx.x & 63;
    const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (e >= B * Out) return;
    const int o = e % Out;
    float s = 0.f;
    for (int k = lane; k < nks; k += 64) s += part[(int64_t)k * B * Out + e];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
    if (lane == 0) {
        if (bias) s += bias[o];
        pre[e] = s;
        Y[e] = slope >= 0.f ? (s > 0.f ? s : slope * s) : s;
    }
}

__global__ void dense_bwd_db(const float* __restrict__ pre, const float* __restrict__ dY, float slope,
                             float* __restrict__ db, int B, int Out)
{
    const int o = blockIdx.x * blockDim.x + threadIdx.x;
    if (o >= Out) return;
    float s = 0.f;
    for (int b0 = 0; b0 < B; b0 += DB) {
        float g[DB];
#pragma unroll
        for (int b = 0; b < DB; ++b)
            g[b] = b0 + b < B ? gate(dY[(b0 + b) * Out + o], pre[(b0 + b) * Out + o], slope) : 0.f;
#pragma unroll
        for (int b = 0; b < DB; ++b)
            if (b0 + b < B) s += g[b];
    }
    db[o] = s;
}

__global__ void dense_bwd_dw(const float* __restrict__ X, const uint16_t* __restrict__ Xb,
                             const float* __restrict__ pre, const float* __restrict__ dY, float slope,
                             float* __restrict__ dW, int B, int In, int Out)
{
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= (int64_t)In * Out) return;
    const int o = (int)(e % Out);
    const int64_t i = e / Out;
    float s = 0.f;
    for (int b0 = 0; b0 < B; b0 += DB) {
        float x[DB], g[DB];
#pragma unroll
        for (int b = 0; b < DB; ++b) {
            const bool ok = b0 + b < B;
            x[b] = ok ? xin(X, Xb, (int64_t)(b0 + b) * In + i) : 0.f;
            g[b] = ok ? gate(dY[(b0 + b) * Out + o], pre[(b0 + b) * Out + o], slope) : 0.f;
        }
#pragma unroll
        for (int b = 0; b < DB; ++b)
            if (b0 + b < B) s = fmaf(x[b], g[b], s);
    }
    dW[e] = s;
}

// One wave per input row i: lanes stride over o, then a fixed butterfly sum.
__global__ __launch_bounds__(256)
void dense_bwd_dx(const float* __restrict__ W, const float* __restrict__ pre, const float* __restrict__ dY,
                  float slope, float* __restrict__ dX, uint16_t* __restrict__ dXb, int B, int In, int Out)
{
    const int lane = threadIdx.x & 63;
    const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= In) return;
    for (int b0 = 0; b0 < B; b0 += DB) {
        const int nb = min(DB, B - b0);
        float acc[DB];
#pragma unroll
        for (int b = 0; b < DB; ++b) acc[b] = 0.f;
        for (int o = lane; o < Out; o += 64) {
            const float w = W[i * Out + o];
#pragma unroll
            for (int b = 0; b < DB; ++b)
                if (b < nb) acc[b] = fmaf(gate(dY[(b0 + b) * Out + o], pre[(b0 + b) * Out + o], slope), w, acc[b]);
        }
#pragma unroll
        for (int b = 0; b < DB; ++b) {
            float v = acc[b];
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
            acc[b] = v;
        }
        if (lane == 0) {
            for (int b = 0; b < nb; ++b) {
                const int64_t o2 = (int64_t)(b0 + b) * In + i;
                if (dXb) dXb[o2] = f2bf(acc[b]);
                else dX[o2] = acc[b];
            }
        }
    }
}

__global__ void mse_kernel(const float* __restrict__ yhat, const float* __restrict__ t, float* __restrict__ loss,
                           float* __restrict__ dyhat, int n)
{
    const int lane = threadIdx.x;
    const float inv = 1.0f / (float)n;
    float s = 0.f;
    for (int e = lane; e < n; e += 64) {
        const float r = yhat[e] - t[e];
        s = fmaf(r, r, s);
        if (dyhat) dyhat[e] = 2.0f * r * inv;
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
    if (lane == 0) *loss = s * inv;
}

// One rounding: W - lr * dW as a fused multiply-add (both SGD kernels use this).
__device__ __forceinline__ float sgd_update(float w, float g, float lr) { return fmaf(-lr, g, w); }

__global__ void sgd_kernel(float* __restrict__ W, const float* __restrict__ dW, float lr, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) W[i] = sgd_update(W[i], dW[i], lr);
}

// Several tensors in one launch: blockIdx.y picks the tensor.
__global__ void sgd_multi_kernel(SgdList l, float lr)
{
    const int t = blockIdx.y;
    float* __restrict__ W = l.w[t];
    const float* __restrict__ dW = l.dw[t];
    const int64_t n = l.n[t];
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) W[i] = sgd_update(W[i], dW[i], lr);
}

__global__ void copy_kernel(const float* __restrict__ s, float* __restrict__ d, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) d[i] = s[i];
}

int nsplits(int In) { return (In + DK - 1) / DK; }

}  // namespace

size_t dense_fwd_part_bytes(int B, int in, int out) { return (size_t)nsplits(in) * B * out * sizeof(float); }

hipError_t launch_dense_fwd(int B, int in, int out, const float* X, const uint16_t* Xb, const float* W,
                            const float* b, float slope, float* pre, float* Y, float* part, hipStream_t s)
{
    const int nks = nsplits(in);
    dim3 grid((unsigned)((out + DO - 1) / DO), (unsigned)nks, (unsigned)((B + DB - 1) / DB));
    hipLaunchKernelGGL(dense_fwd_partial, grid, dim3(DO * DI), 0, s, X, Xb, W, part, B, in, out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(dense_fwd_finalize, dim3((unsigned)((B * out + 3) / 4)), dim3(256), 0, s, part, b, slope,
                       pre, Y, B, out, nks);
    return hipGetLastError();
}

hipError_t launch_dense_bwd(int B, int in, int out, const float* X, const uint16_t* Xb, const float* W,
                            const float* pre, const float* dY, float slope, float* dX, uint16_t* dXb, float* dW,
                            float* db, hipStream_t s)
{
    hipLaunchKernelGGL(dense_bwd_db, dim3((unsigned)((out + 255) / 256)), dim3(256), 0, s, pre, dY, slope, db, B, out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t ndw = (int64_t)in * out;
    hipLaunchKernelGGL(dense_bwd_dw, dim3((unsigned)((ndw + 255) / 256)), dim3(256), 0, s, X, Xb, pre, dY, slope, dW,
                       B, in, out);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (dX || dXb) {
        hipLaunchKernelGGL(dense_bwd_dx, dim3((unsigned)((in + 3) / 4)), dim3(256), 0, s, W, pre, dY, slope, dX, dXb, B,
                           in, out);
        e = hipGetLastError();
    }
    return e;
}

hipError_t launch_mse(int B, int K, const float* yhat, const float* t, float* loss, float* dyhat, hipStream_t s)
{
    hipLaunchKernelGGL(mse_kernel, dim3(1), dim3(64), 0, s, yhat, t, loss, dyhat, B * K);
    return hipGetLastError();
}

hipError_t launch_sgd(int64_t n, float lr, float* W, const float* dW, hipStream_t s)
{
    int64_t b = (n + 255) / 256;
    if (b > 8192) b = 8192;
    hipLaunchKernelGGL(sgd_kernel, dim3((unsigned)(b < 1 ? 1 : b)), dim3(256), 0, s, W, dW, lr, n);
    return hipGetLastError();
}

hipError_t launch_sgd_multi(const SgdList& l, float lr, hipStream_t s)
{
    if (l.count <= 0) return hipSuccess;
    int64_t m = 1;
    for (int t = 0; t < l.count; ++t) m = l.n[t] > m ? l.n[t] : m;
    int64_t b = (m + 255) / 256;
    if (b > 2048) b = 2048;
    hipLaunchKernelGGL(sgd_multi_kernel, dim3((unsigned)b, (unsigned)l.count), dim3(256), 0, s, l, lr);
    return hipGetLastError();
}

hipError_t launch_copy_f32(const float* src, float* dst, int64_t n, hipStream_t s)
{
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src, dst, n);
    return hipGetLastError();
}

}  // namespace cf
