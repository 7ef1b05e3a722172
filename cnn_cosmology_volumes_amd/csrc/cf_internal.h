// Internal declarations shared by the libcf translation units (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "cf.h"

namespace cf {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;   // bfloat16 storage word

// ---------------------------------------------------------------- bf16 <-> f32
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f2bf(float f) {
    __bf16 h = (__bf16)f;
    return __builtin_bit_cast(uint16_t, h);
}

// Two values rounded as by f2bf, packed low | high << 16.  Written as one
// two-lane conversion so that it is a single v_cvt_pk_bf16_f32 (two scalar
// conversions compile to two of them plus an OR).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2_t r = __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, r);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ __forceinline__ static float load(const float* p, int64_t i) { return p[i]; }
    __device__ __forceinline__ static void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
    __device__ __forceinline__ static float load(const uint16_t* p, int64_t i) { return bf2f(p[i]); }
    __device__ __forceinline__ static void store(uint16_t* p, int64_t i, float v) { p[i] = f2bf(v); }
};

// Spread consecutive logical block ids over the 8 XCDs so that neighbouring
// tiles (which share halo data) run on the same XCD and share its L2.
// Hardware dispatches block b to XCD (b % 8); logical id = xcd * per + b / 8.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t b, uint32_t nblocks) {
    const uint32_t per = nblocks / 8u;
    if (per == 0) return b;
    const uint32_t full = per * 8u;
    if (b >= full) return b;
    return (b % 8u) * per + (b / 8u);
}

// Workgroup barrier for LDS traffic only: waits until this wave's LDS
// accesses are done (lgkmcnt 0) but leaves its global loads in flight,
// which __syncthreads() would drain (its fence waits for vmcnt 0 as well).
// The empty asm statements keep the compiler from moving memory accesses
// across the barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// K order of the Cin = 4 forward: k = slot * 4 + ci, slot 0..31, and
// C4_SLOT_TAP[slot] is the tap (kd * 9 + kh * 3 + kw) of that slot, or -1 for
// a zero slot.  An MFMA lane takes slots 2p and 2p + 1 of a 32-deep step;
// within each step the second tap of every lane lies the same halo offset
// from its first (one voxel along w in steps 0, 1 and 3, one row along h in
// step 2), so the two 8-byte reads share one base and pair into one LDS
// access.  The weight re-layout and the kernel both use this table.
__host__ __device__ constexpr int c4_slot_tap(int slot) {
    constexpr int t[32] = {0,  1,  3,  4,  6,  7,  9,  10, 12, 13, 15, 16, 18, 19, 21, 22,
                           2,  5,  11, 14, 20, 23, 8,  -1, 24, 25, 17, -1, 26, -1, -1, -1};
    return t[slot];
}

// Raw buffer resource over `bytes` bytes from p.  A lane whose offset is
// >= bytes reads zeros and touches no memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

// Sets the calling thread's cf_last_error() text; returns s.
cf_status report(cf_status s, const char* fmt, ...);

// ----------------------------------------------------------------- launchers
// Every launcher enqueues on `s` and returns hipGetLastError() of the launch.

// Weight re-layouts (fp32 or bf16 DHWIO source -> bf16 kernel layouts).
// fwd:   Wk[t][co][ci]            (co padded to copad with zeros)
// dgrad: Wk[t'][ci][co] = W[26-t'][ci][co] (ci padded to cipad with zeros)
// c4:    Wk[co][128] with k = t*4 + ci, zero for t >= 27 (Cin == 4 only)
hipError_t launch_wprep_fwd(const void* W, bool w_is_f32, int cin, int cout, int copad, uint16_t* Wk, hipStream_t s);
hipError_t launch_wprep_dgrad(const void* W, bool w_is_f32, int cin, int cout, int cipad, uint16_t* Wk, hipStream_t s);
// The forward layout with the input channels padded to cinp (zeros beyond cin).
hipError_t launch_wprep_fwd_pad(const void* W, bool w_is_f32, int cin, int cinp, int cout, int copad, uint16_t* Wk,
                                hipStream_t s);
// bf16 activations with cin channels copied into cinp channels, zeros after
// (cin, cinp multiples of 8); the matching backward-weight result [27][cinp]
// [cout] cut back to [27][cin][cout].
hipError_t launch_pad_channels(const uint16_t* X, uint16_t* Y, int64_t nvox, int cin, int cinp, hipStream_t s);
hipError_t launch_unpad_dw(const float* dWp, float* dW, int cin, int cinp, int cout, hipStream_t s);
hipError_t launch_wprep_c4(const void* W, bool w_is_f32, int cout, int copad, uint16_t* Wk, hipStream_t s);
// The same re-layouts, several in one launch (identical results).
struct WprepJob {
    int kind;           // 0: fwd (pad = copad), 1: dgrad (pad = cipad), 2: c4 (pad = copad)
    bool f32;
    int cin, cout, pad;
    const void* src;
    uint16_t* dst;
};
struct WprepList {
    int count;
    WprepJob job[2 * 8];
    int start[2 * 8 + 1];   // first block of each job in the flattened grid (set by the launcher)
};
hipError_t launch_wprep_multi(const WprepList& l, hipStream_t s);
// fp32 dgrad weights for the direct path: Wt[t'][co][ci] = W[26-t'][ci][co] (float or bf16 source kept as-is)
hipError_t launch_wprep_direct_dgrad(const void* W, cf_dtype dt, int cin, int cout, void* Wt, hipStream_t s);

// MFMA implicit-GEMM 3^3 conv (forward orientation), in-channels % 32 == 0.
// Used for the forward pass (Wk from wprep_fwd) and backward-data (Wk from
// wprep_dgrad, in/out channels swapped).
struct ConvPlan {
    int cfg;          // tile configuration id
    int bm;           // out-channels per block
    int splits;       // split over in-channel chunks (fp32 partials when > 1)
    bool ring;        // weights through the block's LDS ring (else per-wave loads)
    size_t part_bytes;
};
ConvPlan plan_conv_mfma(const cf_dims& x, int cout);
hipError_t launch_conv_mfma(const ConvPlan& p, const uint16_t* X, const uint16_t* Wk, uint16_t* Y,
                            float* part, const cf_dims& x, int cout, int coutpad, hipStream_t s);

// Conv + leaky ReLU + 2^3 max pool writing P and idx only (no Z), for plans
// with 4x4x16 tiles and no split (one launch, pooled in the conv epilogue)
// and for split plans (the partials' reduction pools; part as for
// launch_conv_mfma); d, h, w even.
bool conv_mfma_can_pool(const ConvPlan& p, const cf_dims& x);
// A conv (x: its input, cout: its output channels) whose output is the
// pooled gradient dP of a 2^3 max-pool: the pool backward (P, idx: the
// pool's output and window indices, shape of the conv output) is applied in
// the partials' reduction (split plans) or the conv epilogue (weight-ring
// plans), writing dZ (2x the conv output's D, H, W) in place of dP; equal to
// launch_conv_mfma then the pool backward bit for bit.
// Which plans can unpool: split plans (in the partials' reduction).
bool conv_mfma_can_unpool(const ConvPlan& p);
hipError_t launch_conv_mfma_unpool(const ConvPlan& p, const uint16_t* X, const uint16_t* Wk, float* part,
                                   const uint16_t* P, const uint8_t* idx, uint16_t* dZ, float slope, const cf_dims& x,
                                   int cout, int coutpad, hipStream_t s);
hipError_t launch_conv_mfma_pool(const ConvPlan& p, const uint16_t* X, const uint16_t* Wk, uint16_t* P, uint8_t* idx,
                                 float slope, const cf_dims& x, int cout, int coutpad, float* part, hipStream_t s);

// Layer-1 forward (Cin == 4) on MFMA, K = 27*4 padded to 128.
hipError_t launch_conv_c4_fwd(const uint16_t* X, const uint16_t* Wk, uint16_t* Y, const cf_dims& x,
                              int cout, int copad, hipStream_t s);
// Same conv with leaky ReLU + 2^3 max pooling fused into the epilogue: writes
// P [n, d/2, h/2, w/2, cout] and idx only (cout % 32 == 0; d, h, w even).
// Shapes the Cin = 4 forward takes (32-bit offsets within a sample built
// from 24-bit multiplies; pooled: a sample's P below 2^31 bytes).
bool conv_c4_fits(const cf_dims& x);
bool conv_c4_pool_fits(const cf_dims& x, int cout);
hipError_t launch_conv_c4_pool_fwd(const uint16_t* X, const uint16_t* Wk, uint16_t* P, uint8_t* idx, float slope,
                                   const cf_dims& x, int cout, hipStream_t s);

// Backward-weight on MFMA.  Partial sums per voxel split into `part`
// ([splits][27*cin*cout] fp32), then a fixed-order reduction into dW.
struct WgradPlan {
    int kind;         // 0: cin % 32 == 0; 1: cin == 4; 2: fp32
    int splits;
    int64_t vox_per_split;
    size_t part_bytes;
};
WgradPlan plan_wgrad(const cf_dims& x, int cout);
// The general kernel (Cin % 32 == 0) addresses a box's six input planes and
// four output-gradient planes with 32-bit byte offsets.
bool wgrad_mfma_fits(const cf_dims& x, int cout);
// The Cin == 4 kernel addresses each box through 32-bit offsets from the
// box's first (d) plane; that needs H * W <= 2^23.
bool wgrad_c4_fits(const cf_dims& x);
hipError_t launch_wgrad(const WgradPlan& p, const uint16_t* X, const uint16_t* dY, float* part, float* dW,
                        const cf_dims& x, int cout, hipStream_t s);
// Cin == 4, cout == 32 backward-weight with the pool backward fused into the
// operand staging: dY is rebuilt per box from the pooled gradient dP, the
// pooled values P and the window indices (plan from plan_wgrad(x, 32)).
hipError_t launch_wgrad_c4_pool(const WgradPlan& p, const uint16_t* X, const uint16_t* dP, const uint16_t* P,
                                const uint8_t* idx, float slope, float* part, float* dW, const cf_dims& x,
                                hipStream_t s);

// Convolution on the fp32 matrix cores (k_conv_f32.hip); channel counts
// multiples of 4.  Weights re-laid as [27][rup(out,64)][rup(in,16)] fp32
// (backward-data: flipped taps, in = forward cout, out = forward cin).  The
// activations are fp32, or bf16 (widened on load, rounded on store) for bf16
// layers outside the bf16 kernels' channel counts; the weight source is fp32
// as is, fp32 rounded to bf16, or bf16.
enum class F32WSrc : int { F32 = 0, F32RoundBf16 = 1, Bf16 = 2 };
bool conv_f32_mfma_ok(const cf_dims& x, int cout);
size_t conv_f32_wk_bytes(int in, int out);
hipError_t launch_wprep_f32(const void* W, F32WSrc src, int cin, int cout, bool dgrad, float* Wk, hipStream_t s);
hipError_t launch_conv_f32_mfma(const float* X, const float* Wk, float* Y, const cf_dims& x, int cout, hipStream_t s);
hipError_t launch_conv_f32_mfma(const uint16_t* X, const float* Wk, uint16_t* Y, const cf_dims& x, int cout,
                                hipStream_t s);
WgradPlan plan_wgrad_f32(const cf_dims& x, int cout);
hipError_t launch_wgrad_f32_mfma(const WgradPlan& p, const float* X, const float* dY, float* part, float* dW,
                                 const cf_dims& x, int cout, hipStream_t s);
hipError_t launch_wgrad_f32_mfma(const WgradPlan& p, const uint16_t* X, const uint16_t* dY, float* part, float* dW,
                                 const cf_dims& x, int cout, hipStream_t s);

// Direct (non-MFMA) conv kernels for fp32 and for shapes outside the MFMA
// paths.  T = float or uint16_t (bf16).  Wt layout is DHWIO for the forward;
// for backward-data the caller passes the flipped/transposed weights.
template <typename T>
hipError_t launch_conv_direct(const T* X, const T* W, T* Y, const cf_dims& x, int cout, hipStream_t s);
template <typename T>
size_t wgrad_direct_part_bytes(const cf_dims& x, int cout);
template <typename T>
hipError_t launch_wgrad_direct(const T* X, const T* dY, float* part, float* dW, const cf_dims& x, int cout,
                               hipStream_t s);

// Pooling / activations.
template <typename T>
hipError_t launch_pool_fwd(const T* Z, T* P, uint8_t* idx, const cf_dims& z, float slope, hipStream_t s);
template <typename T>
hipError_t launch_pool_bwd(const T* dP, const T* P, const uint8_t* idx, T* dZ, const cf_dims& z, float slope,
                           hipStream_t s);
template <typename T>
hipError_t launch_lrelu(const T* x, const T* dy, T* out, int64_t n, float slope, hipStream_t s);

// Dense head and loss (fp32).  Xb: optional bf16 input (used instead of X).
size_t dense_fwd_part_bytes(int B, int in, int out);
hipError_t launch_dense_fwd(int B, int in, int out, const float* X, const uint16_t* Xb, const float* W,
                            const float* b, float slope, float* pre, float* Y, float* part, hipStream_t s);
// Pool backward applied to a dense layer's bf16 input gradient (the pooled
// gradient of the last conv block, flattened NDHWC [B][Dp][Hp][Wp][C]): P and
// idx of that pool, slope, and the full-resolution output dZ.
struct DenseUnpool {
    const uint16_t* P;
    const uint8_t* idx;
    uint16_t* dZ;
    int Dp, Hp, Wp, C;
    float slope;
};
hipError_t launch_dense_bwd(int B, int in, int out, const float* X, const uint16_t* Xb, const float* W,
                            const float* pre, const float* dY, float slope, float* dX, uint16_t* dXb,
                            float* dW, float* db, hipStream_t s, const DenseUnpool* up = nullptr);
// Layers 2 and 3 of the head, MSE, their backward and layer 1's gated
// gradient and bias gradient in one launch (same arithmetic as the
// standalone kernels).  Fits when the two small layers have In <= 128.
struct DenseHead {
    int B, d0, d1, d2;
    float slope;
    const float *y1, *pre1, *W2, *b2, *W3, *b3, *t;
    float *pre2, *y2, *pre3, *y3, *dy3, *loss, *pred;
    float *dy2, *dW3, *db3, *dy1, *dW2, *db2, *g1, *db1;
};
bool dense_head_fits(int B, int d0, int d1, int d2);
hipError_t launch_dense_head(const DenseHead& h, hipStream_t s);
hipError_t launch_mse(int B, int K, const float* yhat, const float* t, float* loss, float* dyhat, hipStream_t s);
hipError_t launch_sgd(int64_t n, float lr, float* W, const float* dW, hipStream_t s);
// The same update for up to 16 tensors in one launch (identical arithmetic).
struct SgdList {
    int count;
    float* w[16];
    const float* dw[16];
    int64_t n[16];
    int start[17];      // first block of each tensor in the flattened grid (set by the launcher)
};
hipError_t launch_sgd_multi(const SgdList& l, float lr, hipStream_t s);
hipError_t launch_copy_f32(const float* src, float* dst, int64_t n, hipStream_t s);

// Adam + LARC over up to CF_MAX_OPT_TENSORS fp32 tensors (k_optim.hip).
struct OptList {
    int count;
    float* w[CF_MAX_OPT_TENSORS];
    const float* g[CF_MAX_OPT_TENSORS];
    float* m[CF_MAX_OPT_TENSORS];
    float* v[CF_MAX_OPT_TENSORS];
    int64_t n[CF_MAX_OPT_TENSORS];
    int start[CF_MAX_OPT_TENSORS + 1];   // first block of each tensor (set by the launcher)
};
// Per-update scalars, computed on the host in fp64 and rounded to fp32.
struct AdamArgs {
    float lr;               // decayed nominal rate of this update
    float beta1, omb1;      // beta1 and 1 - beta1
    float beta2, omb2;      // beta2 and 1 - beta2
    float bc1, bc2;         // 1 / (1 - beta1^t), 1 / (1 - beta2^t)
    float eps, trust;
};
// The per-update scalars of update t (>= 1): decayed rate, bias corrections.
AdamArgs adam_args(const cf_adam_larc_params* hp, int64_t t);
// Validates hp and t (error text through report()).
cf_status check_adam(const cf_adam_larc_params* hp, int64_t t, const char* fn);
size_t adam_larc_part_bytes(const OptList& l);
hipError_t launch_adam_larc(const OptList& l, const AdamArgs& a, float* part, float* lr_out, hipStream_t s);

// Stride-2 resampling and 2^3 average pooling with leaky ReLU
// (k_resample.hip); channel counts multiple of 4.
template <typename T>
hipError_t launch_subsample(const T* Z, T* Y, const cf_dims& z, int Do, int Ho, int Wo, int q, hipStream_t s);
template <typename T>
hipError_t launch_upsample(const T* dY, T* U, const cf_dims& z, int Do, int Ho, int Wo, int q, hipStream_t s);
template <typename T>
hipError_t launch_avgpool_fwd(const T* Z, T* P, const cf_dims& z, float slope, hipStream_t s);
template <typename T>
hipError_t launch_avgpool_bwd(const T* dP, const T* Z, T* dZ, const cf_dims& z, float slope, hipStream_t s);

// Training-mode batch normalisation over (N, D, H, W) per channel of an
// NDHWC tensor, C % 4 == 0 (k_bn.hip).  T = float or uint16_t (bf16).
size_t bn_ws_bytes(const cf_dims& x);
template <typename T>
hipError_t launch_bn_fwd(const T* X, const float* gamma, const float* beta, float eps, T* Y, float* mean,
                         float* invstd, const cf_dims& x, void* ws, hipStream_t s);
template <typename T>
hipError_t launch_bn_bwd(const T* X, const T* dY, const float* gamma, const float* mean, const float* invstd, T* dX,
                         float* dgamma, float* dbeta, const cf_dims& x, void* ws, hipStream_t s);

}  // namespace cf
