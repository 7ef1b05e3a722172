// Matrix-core throughput probe (measurement only; not part of libcf.so).
// Every wave runs `iters` rounds of 8 independent MFMA chains on register
// operands (no memory traffic until one store per lane at the end), so the
// kernel's rate is the chip's sustained MFMA rate at its running clock:
//   kind 0: v_mfma_f32_16x16x32_bf16 (16 * 16 * 32 * 2 flop each)
//   kind 1: v_mfma_f32_16x16x4_f32   (16 * 16 * 4 * 2 flop each)
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void mfma_peak_bf16(float* out, int iters)
{
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(float)((threadIdx.x + i) & 7);
        b[i] = (__bf16)(float)((threadIdx.x * 3 + i) & 7);
    }
    f32x4 acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[k], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void mfma_peak_f32(float* out, int iters)
{
    const float a = (float)(threadIdx.x & 7), b = (float)((threadIdx.x * 3) & 7);
    f32x4 acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[k], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
    out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// out: at least blocks * 256 floats.  Returns 0, or -1 for a bad argument,
// or the HIP error code of the launch.
extern "C" int cf_probe_mfma(int kind, int blocks, int iters, float* out, hipStream_t stream)
{
    if (blocks < 1 || iters < 1 || !out || (kind != 0 && kind != 1)) return -1;
    if (kind == 0)
        hipLaunchKernelGGL(mfma_peak_bf16, dim3(blocks), dim3(256), 0, stream, out, iters);
    else
        hipLaunchKernelGGL(mfma_peak_f32, dim3(blocks), dim3(256), 0, stream, out, iters);
    return (int)hipGetLastError();
}
