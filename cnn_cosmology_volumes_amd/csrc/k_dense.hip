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
constexpr int HEAD_RED = 8192;   // LDS partials of the fused head kernel (floats)

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
    {
        constexpr int KX = DB * DK / (DO * DI);    // staging loads per thread, issued before the stores
        float xv[KX];
#pragma unroll
        for (int k = 0; k < KX; ++k) {
            const int e = threadIdx.x + k * DO * DI, b = e / DK, i = i0 + e % DK;
            xv[k] = (b < nb && i < i1) ? xin(X, Xb, (int64_t)(b0 + b) * In + i) : 0.f;
        }
#pragma unroll
        for (int k = 0; k < KX; ++k) {
            const int e = threadIdx.x + k * DO * DI;
            xs[e / DK][e % DK] = xv[k];
        }
    }
    __syncthreads();
    float acc[DB];
#pragma unroll
    for (int b = 0; b < DB; ++b) acc[b] = 0.f;
    if (o < Out) {
        // rows i0+il, i0+il+DI, ... in increasing order; all of a thread's
        // weight loads (DK / DI rows) are issued together: latency, not
        // bandwidth, bounds this kernel
        constexpr int U = DK / DI;
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

// dW[i][o] = sum over b of X[b][i] * g[b][o] (fmaf chain in b order).  A
// block owns DW_RI input rows x DW_OC output columns.  Per chunk of up to
// DW_BC batch rows it stages the gated gradient g (DW_BC x DW_OC) and the
// input rows (DW_BC x DW_RI) in LDS, so every operand is loaded from global
// memory once per block (loading them per output element made this kernel
// bound by the load-instruction rate).  A thread owns 4 rows x 4 consecutive
// columns; results go out with 16-byte stores when Out % 4 == 0.
constexpr int DW_OC = 128, DW_RI = 32, DW_BC = 32;
__global__ __launch_bounds__(256)
void dense_bwd_dw(const float* __restrict__ X, const uint16_t* __restrict__ Xb,
                  const float* __restrict__ pre, const float* __restrict__ dY, float slope,
                  float* __restrict__ dW, int B, int In, int Out)
{
    __shared__ __attribute__((aligned(16))) float gs[DW_BC][DW_OC];
    __shared__ float xs[DW_BC][DW_RI];
    const int64_t i_blk = (int64_t)blockIdx.x * DW_RI;
    const int tcol = threadIdx.x % (DW_OC / 4), trow = threadIdx.x / (DW_OC / 4);   // 32 column quads x 8 rows
    constexpr int NR = DW_RI / 8;
    const int nch = (Out + DW_OC - 1) / DW_OC;
    for (int ch = blockIdx.y; ch < nch; ch += gridDim.y) {
    const int o_blk = ch * DW_OC;
    float sum[NR][4];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int v = 0; v < 4; ++v) sum[r][v] = 0.f;
    for (int b0 = 0; b0 < B; b0 += DW_BC) {
        const int nb = min(DW_BC, B - b0);
        __syncthreads();
        for (int e = threadIdx.x; e < nb * DW_OC; e += blockDim.x) {
            const int b = e / DW_OC, oo = e % DW_OC, og = o_blk + oo;
            const int64_t r = (int64_t)(b0 + b) * Out + og;
            gs[b][oo] = og < Out ? gate(dY[r], pre[r], slope) : 0.f;
        }
        for (int e = threadIdx.x; e < nb * DW_RI; e += blockDim.x) {
            const int b = e / DW_RI, ii = e % DW_RI;
            const int64_t i = i_blk + ii;
            xs[b][ii] = i < In ? xin(X, Xb, (int64_t)(b0 + b) * In + i) : 0.f;
        }
        __syncthreads();
        for (int b = 0; b < nb; ++b) {
            const float4 g = *reinterpret_cast<const float4*>(&gs[b][tcol * 4]);
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                const float x = xs[b][trow + 8 * r];
                sum[r][0] = fmaf(x, g.x, sum[r][0]);
                sum[r][1] = fmaf(x, g.y, sum[r][1]);
                sum[r][2] = fmaf(x, g.z, sum[r][2]);
                sum[r][3] = fmaf(x, g.w, sum[r][3]);
            }
        }
    }
    const int o = o_blk + tcol * 4;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int64_t i = i_blk + trow + 8 * r;
        if (i >= In) continue;
        float* d = dW + i * Out + o;
        if (Out % 4 == 0) {
            if (o < Out) *reinterpret_cast<float4*>(d) = make_float4(sum[r][0], sum[r][1], sum[r][2], sum[r][3]);
        } else {
#pragma unroll
            for (int v = 0; v < 4; ++v)
                if (o + v < Out) d[v] = sum[r][v];
        }
    }
    }
}

// dX[b][i] = sum over o of g[b][o] * W[i][o], g the gated output gradient:
// one sequential fmaf chain in o order per output element.  The standalone
// kernel and the fused head kernel both use this order, so the training
// step equals the composed entry points bit for bit.
__device__ __forceinline__ float dx_dot(float acc, const float* __restrict__ g, const float* __restrict__ w, int n)
{
    for (int o = 0; o < n; ++o) acc = fmaf(g[o], w[o], acc);
    return acc;
}

// A block owns DX_RI input rows x DB batch rows (one output per thread).
// Per chunk of DX_OC output columns it stages those rows of W and the gated
// gradient in LDS (each loaded once per block); every thread sums the chunk
// in a chain of its own and adds the chunk sums in chunk order (blocked
// summation: the fp32 chains stay DX_OC long whatever Out is; with Out <=
// DX_OC it is the single chain of the fused head kernel).
constexpr int DX_RI = 32, DX_OC = 128;
// With up.dZ set, the bf16 input gradient is the pooled gradient dP of a
// 2^3 max pool whose output is the (flattened NDHWC) input X: dP is rounded to
// bf16 as dXb would hold it, then the pool backward is applied as the pool
// backward kernel does it (times the slope where the pooled value is not
// positive, at the recorded window position; zero at the other seven), and
// the full-resolution gradient dZ is written instead of dP.
__global__ __launch_bounds__(256)
void dense_bwd_dx(const float* __restrict__ W, const float* __restrict__ pre, const float* __restrict__ dY,
                  float slope, float* __restrict__ dX, uint16_t* __restrict__ dXb, int B, int In, int Out,
                  DenseUnpool up)
{
    static_assert(DX_RI * DB == 256, "one output per thread");
    __shared__ float ws[DX_RI][DX_OC + 1];      // +1: the threads of a wave read 8 rows at one column
    __shared__ float gs[DB][DX_OC + 1];
    const int64_t i_blk = (int64_t)blockIdx.x * DX_RI;
    const int bl = threadIdx.x % DB, r = threadIdx.x / DB;
    const int64_t i = i_blk + r;
    for (int b0 = 0; b0 < B; b0 += DB) {
        const int nb = min(DB, B - b0);
        float acc = 0.f;
        for (int oc = 0; oc < Out; oc += DX_OC) {
            const int no = min(DX_OC, Out - oc);
            // every thread issues all of its staging loads before its LDS stores
            constexpr int KW = DX_RI * DX_OC / 256, KG = DB * DX_OC / 256;
            float wv[KW], gv[KG];
#pragma unroll
            for (int k = 0; k < KW; ++k) {
                const int e = threadIdx.x + 256 * k, rr = e / DX_OC, oo = e % DX_OC;
                const int64_t ii = i_blk + rr;
                wv[k] = (ii < In && oo < no) ? W[ii * Out + oc + oo] : 0.f;
            }
#pragma unroll
            for (int k = 0; k < KG; ++k) {
                const int e = threadIdx.x + 256 * k, bb = e / DX_OC, oo = e % DX_OC;
                const int64_t q = (int64_t)(b0 + bb) * Out + oc + oo;
                gv[k] = (bb < nb && oo < no) ? gate(dY[q], pre[q], slope) : 0.f;
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < KW; ++k) {
                const int e = threadIdx.x + 256 * k;
                ws[e / DX_OC][e % DX_OC] = wv[k];
            }
#pragma unroll
            for (int k = 0; k < KG; ++k) {
                const int e = threadIdx.x + 256 * k;
                gs[e / DX_OC][e % DX_OC] = gv[k];
            }
            __syncthreads();
            if (oc == 0) acc = dx_dot(0.f, gs[bl], ws[r], no);
            else acc += dx_dot(0.f, gs[bl], ws[r], no);
        }
        if (i < In && bl < nb) {
            const int64_t q = (int64_t)(b0 + bl) * In + i;
            if (up.dZ) {
                float g = bf2f(f2bf(acc));
                if (!(bf2f(up.P[q]) > 0.f)) g = up.slope * g;
                const uint16_t gb = f2bf(g);
                const int c = (int)(i % up.C);
                int r = (int)(i / up.C);
                const int pw = r % up.Wp; r /= up.Wp;
                const int ph = r % up.Hp;
                const int pd = r / up.Hp;
                const int sel = up.idx[q];
                const int D2 = 2 * up.Dp, H2 = 2 * up.Hp, W2 = 2 * up.Wp;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const int64_t vox = (((int64_t)(b0 + bl) * D2 + 2 * pd + (k >> 2)) * H2 + 2 * ph + ((k >> 1) & 1)) *
                                            W2 + 2 * pw + (k & 1);
                    up.dZ[vox * up.C + c] = k == sel ? gb : (uint16_t)0;
                }
            } else if (dXb) {
                dXb[q] = f2bf(acc);
            } else {
                dX[q] = acc;
            }
        }
    }
}

// The small layers of the head in one block (In <= 128 for layers 2 and 3,
// so each has a single K split): layer 2 and 3 forward, MSE, layer 3 and 2
// backward, and layer 1's gated output gradient and bias gradient.  Every
// value is computed with the same operations in the same order as the
// standalone kernels (partial fmaf chains over i = il mod 4, their sum in il
// order, the split finalize, the MSE and backward reductions), so the fused
// step matches the entry points bit for bit.
__device__ __forceinline__ void head_fwd_layer(const float* __restrict__ X, const float* __restrict__ W, int ldw,
                                               const float* __restrict__ bias, float slope, float* __restrict__ pre,
                                               float* __restrict__ Y, float* red, int B, int In, int Out)
{
    const int n = B * Out;
    for (int task = threadIdx.x; task < n * DI; task += blockDim.x) {
        const int il = task / n, e = task % n, b = e / Out, o = e % Out;
        float acc = 0.f;
        for (int i = il; i < In; i += DI) acc = fmaf(X[b * In + i], W[i * ldw + o], acc);
        red[task] = acc;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < n; e += blockDim.x) {
        float p = red[e];
#pragma unroll
        for (int k = 1; k < DI; ++k) p += red[k * n + e];
        float sum = 0.f;
        sum += p;                       // the finalize's single-split lane sum
        if (bias) sum += bias[e % Out];
        pre[e] = sum;
        Y[e] = slope >= 0.f ? (sum > 0.f ? sum : slope * sum) : sum;
    }
    __syncthreads();
}

// g (B x Out, LDS scratch) receives the gated output gradient once; the bias,
// weight and data gradients then read it (the gate is exact, so this is the
// same arithmetic as gating inside each sum, as the standalone kernels do).
// g: LDS scratch for the gated gradient, rows of Out + 1 floats; W (LDS)
// has rows of ldw floats.  Both strides are odd multiples of 4 bytes apart
// from a power of two, so the 8 rows a wave reads in the dX dots fall on
// distinct banks.
__device__ __forceinline__ void head_bwd_layer(const float* __restrict__ X, const float* __restrict__ W, int ldw,
                                               const float* __restrict__ pre, const float* __restrict__ dY,
                                               float slope, float* __restrict__ dX, float* __restrict__ dW,
                                               float* __restrict__ db, float* __restrict__ g, int B, int In, int Out)
{
    const int ldg = Out + 1;
    for (int e = threadIdx.x; e < B * Out; e += blockDim.x) g[(e / Out) * ldg + e % Out] = gate(dY[e], pre[e], slope);
    __syncthreads();
    for (int o = threadIdx.x; o < Out; o += blockDim.x) {
        float sum = 0.f;
        for (int b = 0; b < B; ++b) sum += g[b * ldg + o];
        db[o] = sum;
    }
    for (int e = threadIdx.x; e < In * Out; e += blockDim.x) {
        const int i = e / Out, o = e % Out;
        float sum = 0.f;
        for (int b = 0; b < B; ++b) sum = fmaf(X[b * In + i], g[b * ldg + o], sum);
        dW[e] = sum;
    }
    if (dX)
        for (int e = threadIdx.x; e < B * In; e += blockDim.x) {
            const int b = e % B, i = e / B;
            dX[b * In + i] = dx_dot(0.f, g + b * ldg, W + i * ldw, Out);
        }
    __syncthreads();
}

// dst (rows of ldd floats) = src (rows x cols, dense) by the whole block,
// every thread issuing its loads before its stores.
__device__ __forceinline__ void block_copy_rows(float* __restrict__ dst, int ldd, const float* __restrict__ src,
                                                int rows, int cols)
{
    constexpr int U = 8;
    const int n = rows * cols;
    for (int e0 = threadIdx.x; e0 < n; e0 += U * blockDim.x) {
        float v[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int e = e0 + k * blockDim.x;
            v[k] = e < n ? src[e] : 0.f;
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int e = e0 + k * blockDim.x;
            if (e < n) dst[(e / cols) * ldd + e % cols] = v[k];
        }
    }
}

// dst[e] = src[e] for e < n by the whole block, every thread issuing its
// loads before its stores (a load-store loop would wait on each load in turn).
__device__ __forceinline__ void block_copy(float* __restrict__ dst, const float* __restrict__ src, int n)
{
    constexpr int U = 8;
    for (int e0 = threadIdx.x; e0 < n; e0 += U * blockDim.x) {
        float v[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int e = e0 + k * blockDim.x;
            v[k] = e < n ? src[e] : 0.f;
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int e = e0 + k * blockDim.x;
            if (e < n) dst[e] = v[k];
        }
    }
}

__global__ __launch_bounds__(1024)
void dense_head_kernel(DenseHead h)
{
    // Every operand and intermediate lives in LDS (tens of KB): the
    // reductions are short dependent chains, so LDS latency instead of L2
    // latency is what makes one block fast enough.
    extern __shared__ float lds[];
    const int B = h.B, d0 = h.d0, d1 = h.d1, d2 = h.d2;
    float* red = lds;                      // HEAD_RED
    float* y1 = red + HEAD_RED;            // B*d0
    float* pre1 = y1 + B * d0;             // B*d0
    const int ld2 = d1 + 1, ld3 = d2 + 1;  // padded rows (see head_bwd_layer)
    float* W2 = pre1 + B * d0;             // d0 x ld2
    float* W3 = W2 + d0 * ld2;             // d1 x ld3
    float* pre2 = W3 + d1 * ld3;           // B*d1
    float* y2 = pre2 + B * d1;             // B*d1
    float* pre3 = y2 + B * d1;             // B*d2
    float* y3 = pre3 + B * d2;             // B*d2
    float* dy3 = y3 + B * d2;              // B*d2
    float* dy2 = dy3 + B * d2;             // B*d1
    float* dy1 = dy2 + B * d1;             // B*d0
    block_copy(y1, h.y1, B * d0);
    block_copy(pre1, h.pre1, B * d0);
    block_copy_rows(W2, ld2, h.W2, d0, d1);
    block_copy_rows(W3, ld3, h.W3, d1, d2);
    __syncthreads();
    head_fwd_layer(y1, W2, ld2, h.b2, h.slope, pre2, y2, red, B, d0, d1);
    head_fwd_layer(y2, W3, ld3, h.b3, -1.f, pre3, y3, red, B, d1, d2);
    const int n = B * d2;
    if (threadIdx.x < 64) {
        // mean squared error, as mse_kernel
        const int lane = threadIdx.x;
        const float inv = 1.0f / (float)n;
        float sum = 0.f;
        for (int e = lane; e < n; e += 64) {
            const float r = y3[e] - h.t[e];
            sum = fmaf(r, r, sum);
            dy3[e] = 2.0f * r * inv;
            if (h.pred) h.pred[e] = y3[e];
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) sum += __shfl_xor(sum, m, 64);
        if (lane == 0) *h.loss = sum * inv;
    }
    __syncthreads();
    // red (free after the forward layers) holds each layer's gated gradient
    head_bwd_layer(y2, W3, ld3, pre3, dy3, -1.f, dy2, h.dW3, h.db3, red, B, d1, d2);
    head_bwd_layer(y1, W2, ld2, pre2, dy2, h.slope, dy1, h.dW2, h.db2, red, B, d0, d1);
    // layer 1: gated output gradient (consumed by its weight / data gradient
    // kernels with the gate switched off) and the bias gradient
    for (int e = threadIdx.x; e < B * d0; e += blockDim.x) h.g1[e] = gate(dy1[e], pre1[e], h.slope);
    for (int o = threadIdx.x; o < d0; o += blockDim.x) {
        float sum = 0.f;
        for (int b = 0; b < B; ++b) sum += gate(dy1[b * d0 + o], pre1[b * d0 + o], h.slope);
        h.db1[o] = sum;
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

// Several tensors in one launch: the grid is the tensors' block ranges laid
// end to end, and a block finds its tensor in the list's start table.
// A thread updates SGD_E consecutive elements, issuing all of its loads
// (16-byte when both tensors are 16-byte aligned) before any update, so one
// memory latency is paid per thread instead of one per element.
constexpr int SGD_E = 4;
__global__ __launch_bounds__(256)
void sgd_multi_kernel(SgdList l, float lr)
{
    int t = 0;
    while (t + 1 < l.count && (int)blockIdx.x >= l.start[t + 1]) ++t;
    const int bid = (int)blockIdx.x - l.start[t], nblk = l.start[t + 1] - l.start[t];
    float* __restrict__ W = l.w[t];
    const float* __restrict__ dW = l.dw[t];
    const int64_t n = l.n[t];
    const int64_t stride = (int64_t)nblk * blockDim.x * SGD_E;
    const bool vec = (((uintptr_t)W | (uintptr_t)dW) & 15u) == 0;
    for (int64_t i0 = ((int64_t)bid * blockDim.x + threadIdx.x) * SGD_E; i0 < n; i0 += stride) {
        if (vec && i0 + SGD_E <= n) {
            float4 w[SGD_E / 4], g[SGD_E / 4];
#pragma unroll
            for (int k = 0; k < SGD_E / 4; ++k) {
                w[k] = reinterpret_cast<const float4*>(W + i0)[k];
                g[k] = reinterpret_cast<const float4*>(dW + i0)[k];
            }
#pragma unroll
            for (int k = 0; k < SGD_E / 4; ++k)
                reinterpret_cast<float4*>(W + i0)[k] =
                    make_float4(sgd_update(w[k].x, g[k].x, lr), sgd_update(w[k].y, g[k].y, lr),
                                sgd_update(w[k].z, g[k].z, lr), sgd_update(w[k].w, g[k].w, lr));
        } else {
            float w[SGD_E], g[SGD_E];
#pragma unroll
            for (int k = 0; k < SGD_E; ++k) {
                w[k] = i0 + k < n ? W[i0 + k] : 0.f;
                g[k] = i0 + k < n ? dW[i0 + k] : 0.f;
            }
#pragma unroll
            for (int k = 0; k < SGD_E; ++k)
                if (i0 + k < n) W[i0 + k] = sgd_update(w[k], g[k], lr);
        }
    }
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
                            float* db, hipStream_t s, const DenseUnpool* up)
{
    const DenseUnpool nu{};
    hipError_t e;
    if (db) {
        hipLaunchKernelGGL(dense_bwd_db, dim3((unsigned)((out + 255) / 256)), dim3(256), 0, s, pre, dY, slope, db, B,
                           out);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int nch = (out + DW_OC - 1) / DW_OC;
    hipLaunchKernelGGL(dense_bwd_dw, dim3((unsigned)((in + DW_RI - 1) / DW_RI), (unsigned)(nch < 65535 ? nch : 65535)),
                       dim3(256), 0, s, X, Xb, pre, dY, slope, dW, B, in, out);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (dX || dXb || (up && up->dZ)) {
        hipLaunchKernelGGL(dense_bwd_dx, dim3((unsigned)((in + DX_RI - 1) / DX_RI)), dim3(256), 0, s, W, pre, dY, slope, dX, dXb, B,
                           in, out, up ? *up : nu);
        e = hipGetLastError();
    }
    return e;
}

size_t head_lds_bytes(int B, int d0, int d1, int d2)
{
    return sizeof(float) * ((size_t)HEAD_RED + 3 * (size_t)B * d0 + (size_t)d0 * (d1 + 1) + (size_t)d1 * (d2 + 1) +
                            3 * (size_t)B * d1 + 3 * (size_t)B * d2);
}

bool dense_head_fits(int B, int d0, int d1, int d2)
{
    return d0 <= DK && d1 <= DK && (int64_t)B * d1 * DI <= HEAD_RED && (int64_t)B * d2 * DI <= HEAD_RED &&
           B * d2 <= 64 && head_lds_bytes(B, d0, d1, d2) <= 96 * 1024;
}

hipError_t launch_dense_head(const DenseHead& h, hipStream_t s)
{
    if (!dense_head_fits(h.B, h.d0, h.d1, h.d2)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(dense_head_kernel, dim3(1), dim3(1024), head_lds_bytes(h.B, h.d0, h.d1, h.d2), s, h);
    return hipGetLastError();
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

hipError_t launch_sgd_multi(const SgdList& l_in, float lr, hipStream_t s)
{
    if (l_in.count <= 0) return hipSuccess;
    // each tensor gets the blocks it needs (capped), laid end to end in one
    // grid, instead of every tensor getting the largest tensor's count
    SgdList l = l_in;
    int total = 0;
    for (int t = 0; t < l.count; ++t) {
        int64_t b = (l.n[t] + 256 * SGD_E - 1) / (256 * SGD_E);
        if (b < 1) b = 1;
        if (b > 2048) b = 2048;
        l.start[t] = total;
        total += (int)b;
    }
    l.start[l.count] = total;
    hipLaunchKernelGGL(sgd_multi_kernel, dim3((unsigned)total), dim3(256), 0, s, l, lr);
    return hipGetLastError();
}

hipError_t launch_copy_f32(const float* src, float* dst, int64_t n, hipStream_t s)
{
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, src, dst, n);
    return hipGetLastError();
}

}  // namespace cf
