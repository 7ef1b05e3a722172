// Weight re-layouts feeding the conv kernels.  Source weights are DHWIO
// [3][3][3][Cin][Cout] in fp32 (master copy) or bf16; the bf16 copies are
// rounded to nearest even.
//
// Backward-data of a stride-1, pad-1 3^3 correlation is itself a pad-1
// correlation of dY with the weights flipped in all three spatial axes and
// with input/output channels swapped:
//   dX[v, ci] = sum_{t'} sum_co dY[v + off(t'), co] * W[26 - t'][ci][co]
// (substitute t' = 26 - t in the backward-data definition, CosmoFlow
// Sec. III-C's separate backward-data operator), so the forward kernels run
// it unchanged on the re-laid weights below.
#include "cf_internal.h"

namespace cf {

namespace {

__device__ __forceinline__ float wload(const void* W, bool f32, int64_t i) {
    return f32 ? reinterpret_cast<const float*>(W)[i] : bf2f(reinterpret_cast<const uint16_t*>(W)[i]);
}

// Wk[t][co][ci], co < copad (zero rows beyond cout).
__global__ void wprep_fwd_kernel(const void* W, bool f32, int cin, int cout, int copad, uint16_t* Wk)
{
    const int64_t total = (int64_t)27 * copad * cin;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
        const int ci = (int)(e % cin);
        const int co = (int)((e / cin) % copad);
        const int t = (int)(e / ((int64_t)cin * copad));
        Wk[e] = co < cout ? f2bf(wload(W, f32, ((int64_t)t * cin + ci) * cout + co)) : (uint16_t)0;
    }
}

// Wk[t'][ci][co] = W[26 - t'][ci][co], ci < cipad (zero rows beyond cin).
__global__ void wprep_dgrad_kernel(const void* W, bool f32, int cin, int cout, int cipad, uint16_t* Wk)
{
    const int64_t total = (int64_t)27 * cipad * cout;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
        const int co = (int)(e % cout);
        const int ci = (int)((e / cout) % cipad);
        const int t = (int)(e / ((int64_t)cout * cipad));
        Wk[e] = ci < cin ? f2bf(wload(W, f32, ((int64_t)(26 - t) * cin + ci) * cout + co)) : (uint16_t)0;
    }
}

// Wk[co][k], k = t*4 + ci for t < 27, zero for k >= 108 or co >= cout.
__global__ void wprep_c4_kernel(const void* W, bool f32, int cout, int copad, uint16_t* Wk)
{
    const int64_t total = (int64_t)copad * 128;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
        const int k = (int)(e % 128);
        const int co = (int)(e / 128);
        const int t = k / 4, ci = k % 4;
        Wk[e] = (co < cout && t < 27) ? f2bf(wload(W, f32, ((int64_t)t * 4 + ci) * cout + co)) : (uint16_t)0;
    }
}

// Direct-path backward-data weights (same element type as the source):
// Wt[t'][co][ci] = W[26 - t'][ci][co]  (DHWIO with in = cout, out = cin).
template <typename T>
__global__ void wprep_direct_dgrad_kernel(const T* W, int cin, int cout, T* Wt)
{
    const int64_t total = (int64_t)27 * cin * cout;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
        const int ci = (int)(e % cin);
        const int co = (int)((e / cin) % cout);
        const int t = (int)(e / ((int64_t)cin * cout));
        Wt[e] = W[((int64_t)(26 - t) * cin + ci) * cout + co];
    }
}

unsigned blocks_for(int64_t n) {
    int64_t b = (n + 255) / 256;
    if (b > 4096) b = 4096;
    return (unsigned)(b < 1 ? 1 : b);
}

}  // namespace

hipError_t launch_wprep_fwd(const void* W, bool w_is_f32, int cin, int cout, int copad, uint16_t* Wk, hipStream_t s)
{
    hipLaunchKernelGGL(wprep_fwd_kernel, dim3(blocks_for((int64_t)27 * copad * cin)), dim3(256), 0, s, W, w_is_f32,
                       cin, cout, copad, Wk);
    return hipGetLastError();
}

hipError_t launch_wprep_dgrad(const void* W, bool w_is_f32, int cin, int cout, int cipad, uint16_t* Wk, hipStream_t s)
{
    hipLaunchKernelGGL(wprep_dgrad_kernel, dim3(blocks_for((int64_t)27 * cipad * cout)), dim3(256), 0, s, W, w_is_f32,
                       cin, cout, cipad, Wk);
    return hipGetLastError();
}

hipError_t launch_wprep_c4(const void* W, bool w_is_f32, int cout, int copad, uint16_t* Wk, hipStream_t s)
{
    hipLaunchKernelGGL(wprep_c4_kernel, dim3(blocks_for((int64_t)copad * 128)), dim3(256), 0, s, W, w_is_f32, cout,
                       copad, Wk);
    return hipGetLastError();
}

hipError_t launch_wprep_direct_dgrad(const void* W, cf_dtype dt, int cin, int cout, void* Wt, hipStream_t s)
{
    const unsigned g = blocks_for((int64_t)27 * cin * cout);
    if (dt == CF_F32)
        hipLaunchKernelGGL(wprep_direct_dgrad_kernel<float>, dim3(g), dim3(256), 0, s,
                           reinterpret_cast<const float*>(W), cin, cout, reinterpret_cast<float*>(Wt));
    else
        hipLaunchKernelGGL(wprep_direct_dgrad_kernel<uint16_t>, dim3(g), dim3(256), 0, s,
                           reinterpret_cast<const uint16_t*>(W), cin, cout, reinterpret_cast<uint16_t*>(Wt));
    return hipGetLastError();
}

}  // namespace cf
