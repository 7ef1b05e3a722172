// Adam with LARC's layer-wise rate clipping and a polynomial learning-rate
// decay, over a list of fp32 parameter tensors in two launches.
//
// Launch 1 (larc_norms_kernel): every block owns one OPT_CHUNK-element
// chunk of one tensor and writes that chunk's sums of w^2 and g^2.
// Launch 2 (adam_larc_kernel): every block first adds up its tensor's chunk
// sums in fp64, in chunk order (the same order in every block of the
// tensor, so all of them get the same norms), derives the tensor's rate,
// and then updates its own chunk: the moments, and w by the rate times the
// bias-corrected Adam direction.  No atomics: results are reproducible bit
// for bit.
#include "cf_internal.h"

#include <math.h>

namespace cf {
namespace {

constexpr int OPT_T = 256;                  // threads per block
constexpr int OPT_V = 4;                    // float4 vectors per thread per chunk
constexpr int OPT_CHUNK = OPT_T * OPT_V * 4;

// The tensor whose block range holds this block.
__device__ __forceinline__ int find_tensor(const OptList& l)
{
    int t = 0;
    while (t + 1 < l.count && (int)blockIdx.x >= l.start[t + 1]) ++t;
    return t;
}

// Sum of a and b over the block, returned in every thread: a fixed
// butterfly within each wave, then the four wave sums in wave order.
__device__ __forceinline__ void block_sum2(float& a, float& b, float* lds)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        a += __shfl_xor(a, m, 64);
        b += __shfl_xor(b, m, 64);
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        lds[2 * wave] = a;
        lds[2 * wave + 1] = b;
    }
    __syncthreads();
    a = ((lds[0] + lds[2]) + lds[4]) + lds[6];
    b = ((lds[1] + lds[3]) + lds[5]) + lds[7];
}

__global__ __launch_bounds__(OPT_T) void larc_norms_kernel(OptList l, float2* __restrict__ part)
{
    __shared__ float lds[8];
    const int t = find_tensor(l);
    const int64_t n = l.n[t];
    const int64_t c0 = (int64_t)((int)blockIdx.x - l.start[t]) * OPT_CHUNK;
    const float* __restrict__ w = l.w[t];
    const float* __restrict__ g = l.g[t];
    float sw = 0.f, sg = 0.f;
#pragma unroll
    for (int k = 0; k < OPT_V; ++k) {
        const int64_t i = c0 + ((int64_t)k * OPT_T + threadIdx.x) * 4;
        if (i + 4 <= n) {
            const float4 a = *reinterpret_cast<const float4*>(w + i);
            const float4 b = *reinterpret_cast<const float4*>(g + i);
            sw += a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w;
            sg += b.x * b.x + b.y * b.y + b.z * b.z + b.w * b.w;
        } else {
            for (int e = 0; e < 4; ++e)
                if (i + e < n) {
                    sw += w[i + e] * w[i + e];
                    sg += g[i + e] * g[i + e];
                }
        }
    }
    block_sum2(sw, sg, lds);
    if (threadIdx.x == 0) part[blockIdx.x] = make_float2(sw, sg);
}

__global__ __launch_bounds__(OPT_T) void adam_larc_kernel(OptList l, const float2* __restrict__ part, AdamArgs a,
                                                          float* __restrict__ lr_out)
{
    __shared__ float rate;
    const int t = find_tensor(l);
    if (threadIdx.x < 64) {
        // the tensor's norms from its chunk sums, fp64, fixed order
        double sw = 0.0, sg = 0.0;
        for (int b = l.start[t] + (int)threadIdx.x; b < l.start[t + 1]; b += 64) {
            const float2 p = part[b];
            sw += (double)p.x;
            sg += (double)p.y;
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            sw += __shfl_xor(sw, m, 64);
            sg += __shfl_xor(sg, m, 64);
        }
        if (threadIdx.x == 0) {
            double lr = (double)a.lr;
            if (a.trust > 0.f && sw > 0.0 && sg > 0.0) {
                const double ratio = (double)a.trust * sqrt(sw) / sqrt(sg);
                if (ratio < lr) lr = ratio;
            }
            rate = (float)lr;
            if (lr_out && (int)blockIdx.x == l.start[t]) lr_out[t] = (float)lr;
        }
    }
    __syncthreads();
    const float lr = rate;
    const int64_t n = l.n[t];
    const int64_t c0 = (int64_t)((int)blockIdx.x - l.start[t]) * OPT_CHUNK;
    float* __restrict__ W = l.w[t];
    const float* __restrict__ G = l.g[t];
    float* __restrict__ M = l.m[t];
    float* __restrict__ V = l.v[t];
    auto upd = [&](float& w, float g, float& m, float& v) {
        m = a.beta1 * m + a.omb1 * g;
        v = a.beta2 * v + a.omb2 * (g * g);
        const float mhat = m * a.bc1;
        const float vhat = v * a.bc2;
        w = w - lr * (mhat / (sqrtf(vhat) + a.eps));
    };
#pragma unroll
    for (int k = 0; k < OPT_V; ++k) {
        const int64_t i = c0 + ((int64_t)k * OPT_T + threadIdx.x) * 4;
        if (i + 4 <= n) {
            float4 w = *reinterpret_cast<const float4*>(W + i);
            const float4 g = *reinterpret_cast<const float4*>(G + i);
            float4 m = *reinterpret_cast<const float4*>(M + i);
            float4 v = *reinterpret_cast<const float4*>(V + i);
            upd(w.x, g.x, m.x, v.x);
            upd(w.y, g.y, m.y, v.y);
            upd(w.z, g.z, m.z, v.z);
            upd(w.w, g.w, m.w, v.w);
            *reinterpret_cast<float4*>(W + i) = w;
            *reinterpret_cast<float4*>(M + i) = m;
            *reinterpret_cast<float4*>(V + i) = v;
        } else {
            for (int e = 0; e < 4; ++e)
                if (i + e < n) {
                    float w = W[i + e], m = M[i + e], v = V[i + e];
                    upd(w, G[i + e], m, v);
                    W[i + e] = w;
                    M[i + e] = m;
                    V[i + e] = v;
                }
        }
    }
}

int blocks_for(int64_t n) { return (int)((n + OPT_CHUNK - 1) / OPT_CHUNK); }

}  // namespace

cf_status check_adam(const cf_adam_larc_params* hp, int64_t t, const char* fn)
{
    if (!hp) return report(CF_ERR_INVALID, "%s: null optimizer parameters", fn);
    if (t < 1) return report(CF_ERR_INVALID, "%s: the update count t starts at 1 (got %lld)", fn, (long long)t);
    if (!(hp->lr0 >= 0.f) || !(hp->lr_end >= 0.f) || hp->decay_steps < 1 || !(hp->power > 0.f))
        return report(CF_ERR_INVALID, "%s: decay needs lr0, lr_end >= 0, decay_steps >= 1, power > 0", fn);
    if (!(hp->beta1 >= 0.f && hp->beta1 < 1.f) || !(hp->beta2 >= 0.f && hp->beta2 < 1.f) || !(hp->eps > 0.f))
        return report(CF_ERR_INVALID, "%s: need 0 <= beta1, beta2 < 1 and eps > 0", fn);
    if (!(hp->trust == hp->trust)) return report(CF_ERR_INVALID, "%s: trust is NaN", fn);
    return CF_OK;
}

AdamArgs adam_args(const cf_adam_larc_params* hp, int64_t t)
{
    // the decayed rate after t - 1 completed updates, in fp64
    const double T = (double)hp->decay_steps;
    const double done = t - 1 < hp->decay_steps ? (double)(t - 1) : T;
    AdamArgs a{};
    a.lr = (float)(((double)hp->lr0 - (double)hp->lr_end) * pow(1.0 - done / T, (double)hp->power) +
                   (double)hp->lr_end);
    a.beta1 = hp->beta1;
    a.omb1 = (float)(1.0 - (double)hp->beta1);
    a.beta2 = hp->beta2;
    a.omb2 = (float)(1.0 - (double)hp->beta2);
    a.bc1 = (float)(1.0 / (1.0 - pow((double)hp->beta1, (double)t)));
    a.bc2 = (float)(1.0 / (1.0 - pow((double)hp->beta2, (double)t)));
    a.eps = hp->eps;
    a.trust = hp->trust;
    return a;
}

size_t adam_larc_part_bytes(const OptList& l)
{
    int64_t b = 0;
    for (int t = 0; t < l.count; ++t) b += blocks_for(l.n[t]);
    return (size_t)b * sizeof(float2);
}

hipError_t launch_adam_larc(const OptList& l_in, const AdamArgs& a, float* part, float* lr_out, hipStream_t s)
{
    if (l_in.count <= 0) return hipSuccess;
    OptList l = l_in;
    int total = 0;
    for (int t = 0; t < l.count; ++t) {
        l.start[t] = total;
        total += blocks_for(l.n[t]);
    }
    l.start[l.count] = total;
    hipLaunchKernelGGL(larc_norms_kernel, dim3((unsigned)total), dim3(OPT_T), 0, s, l, (float2*)part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(adam_larc_kernel, dim3((unsigned)total), dim3(OPT_T), 0, s, l, (const float2*)part, a, lr_out);
    return hipGetLastError();
}

}  // namespace cf
