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

// Element e of the dgrad and c4 layouts (their element-wise paths in the
// batched kernel below).  The fwd layout, Wk[t][co][ci] with zero rows for
// co >= cout, goes through that kernel's transposing tiles.
// Element indices stay far below 2^31 (27 taps x padded channels), so the
// index arithmetic is 32-bit.
// dgrad: Wk[t'][ci][co] = W[26 - t'][ci][co], ci < cipad (zero rows beyond cin).
__device__ __forceinline__ uint16_t wk_dgrad_elem(const void* W, bool f32, int cin, int cout, int cipad, int64_t e64)
{
    const uint32_t e = (uint32_t)e64;
    const int co = (int)(e % (uint32_t)cout);
    const int ci = (int)((e / (uint32_t)cout) % (uint32_t)cipad);
    const int t = (int)(e / ((uint32_t)cout * (uint32_t)cipad));
    return ci < cin ? f2bf(wload(W, f32, ((int64_t)(26 - t) * cin + ci) * cout + co)) : (uint16_t)0;
}
// c4:    Wk[co][k], k = slot*4 + ci with the tap of each slot from
//        c4_slot_tap (zero for empty slots and for co >= cout).
__device__ __forceinline__ uint16_t wk_c4_elem(const void* W, bool f32, int cout, int64_t e64)
{
    const uint32_t e = (uint32_t)e64;
    const int k = (int)(e % 128u);
    const int co = (int)(e / 128u);
    const int t = c4_slot_tap(k / 4), ci = k % 4;
    return (co < cout && t >= 0) ? f2bf(wload(W, f32, ((int64_t)t * 4 + ci) * cout + co)) : (uint16_t)0;
}


// fwd with the input channels padded to cinp (zero columns for ci >= cin):
// Wk[t][co][ci], ci < cinp.
__global__ void wprep_fwd_pad_kernel(const void* W, bool f32, int cin, int cinp, int cout, int copad, uint16_t* Wk)
{
    const int64_t total = (int64_t)27 * copad * cinp;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < total; e += (int64_t)gridDim.x * blockDim.x) {
        const uint32_t u = (uint32_t)e;
        const int ci = (int)(u % (uint32_t)cinp);
        const int co = (int)((u / (uint32_t)cinp) % (uint32_t)copad);
        const int t = (int)(u / ((uint32_t)cinp * (uint32_t)copad));
        Wk[e] = (ci < cin && co < cout) ? f2bf(wload(W, f32, ((int64_t)t * cin + ci) * cout + co)) : (uint16_t)0;
    }
}

// Several re-layouts in one launch: blockIdx.y picks the job.  The fwd
// layout transposes (input channel) x (output channel) matrices, so those
// jobs go through 32 x 32 LDS tiles: the fp32 source is read along its
// contiguous output channels and the bf16 copy written along its contiguous
// rows.  The dgrad layout keeps the source's channel order and the c4 layout
// is a small permutation; both are copied element by element.  Values are
// the same f2bf roundings either way.
constexpr int WT = 32;

__global__ __launch_bounds__(256)
void wprep_multi_kernel(WprepList l)
{
    __shared__ float tile[WT][WT + 1];
    // the grid is the jobs' block ranges laid end to end: find this block's job
    int ji = 0;
    while (ji + 1 < l.count && (int)blockIdx.x >= l.start[ji + 1]) ++ji;
    const WprepJob& j = l.job[ji];
    const int bid = (int)blockIdx.x - l.start[ji], nblk = l.start[ji + 1] - l.start[ji];
    if (j.kind == 1 && j.cout % 8 == 0) {
        // 8 consecutive output channels per thread: the tap flip keeps the
        // channel order, so both sides are contiguous (16-byte-aligned
        // sources; the same f2bf roundings as wk_dgrad_elem)
        const uint32_t total8 = (uint32_t)(27 * j.pad * j.cout / 8);
        const uint32_t c8 = (uint32_t)(j.cout / 8);
        for (uint32_t e = (uint32_t)bid * blockDim.x + threadIdx.x; e < total8; e += (uint32_t)nblk * blockDim.x) {
            const uint32_t co = (e % c8) * 8u, ci = (e / c8) % (uint32_t)j.pad, t = e / (c8 * (uint32_t)j.pad);
            uint4 o = make_uint4(0u, 0u, 0u, 0u);
            if (ci < (uint32_t)j.cin) {
                const int64_t si = ((int64_t)(26 - t) * j.cin + ci) * j.cout + co;
                float v[8];
                if (j.f32) {
                    const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(j.src) + si);
                    const float4 b = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(j.src) + si + 4);
                    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
                } else {
                    const uint4 a = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(j.src) + si);
                    const uint32_t w4[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        v[2 * k] = __uint_as_float(w4[k] << 16);
                        v[2 * k + 1] = __uint_as_float(w4[k] & 0xffff0000u);
                    }
                }
                o = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                               pack_bf16x2(v[6], v[7]));
            }
            reinterpret_cast<uint4*>(j.dst)[e] = o;
        }
        return;
    }
    if (j.kind == 1) {
        const int64_t total = (int64_t)27 * j.pad * j.cout;
        for (int64_t e = (int64_t)bid * blockDim.x + threadIdx.x; e < total; e += (int64_t)nblk * blockDim.x)
            j.dst[e] = wk_dgrad_elem(j.src, j.f32, j.cin, j.cout, j.pad, e);
        return;
    }
    if (j.kind == 2) {            // c4: a permutation of taps, tiny (copad x 128)
        const int64_t total = (int64_t)j.pad * 128;
        for (int64_t e = (int64_t)bid * blockDim.x + threadIdx.x; e < total; e += (int64_t)nblk * blockDim.x)
            j.dst[e] = wk_c4_elem(j.src, j.f32, j.cout, e);
        return;
    }
    // source S[r][c] (c = output channel, contiguous), R rows per matrix;
    // destination D[c][r] with row length Rpad, c < pad (zero beyond cout),
    // r < Rpad (zero beyond R)
    const int R = j.cin, Rpad = j.cin, C = j.cout, Cpad = j.pad;
    const int nmat = 27;
    const int tr = (Rpad + WT - 1) / WT, tc = (Cpad + WT - 1) / WT;
    const int ntiles = nmat * tr * tc;
    const int lx = threadIdx.x % WT, ly = threadIdx.x / WT;     // 32 x 8
    for (int tile_id = bid; tile_id < ntiles; tile_id += nblk) {
        const int m = tile_id / (tr * tc), rt = (tile_id / tc) % tr, ct = tile_id % tc;
        const int r0 = rt * WT, c0 = ct * WT;
        const int64_t sbase = (int64_t)m * R * C, dbase = (int64_t)m * Cpad * Rpad;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < WT / 8; ++k) {
            const int r = r0 + ly + 8 * k, c = c0 + lx;
            tile[ly + 8 * k][lx] = (r < R && c < C) ? wload(j.src, j.f32, sbase + (int64_t)r * C + c) : 0.f;
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < WT / 8; ++k) {
            const int c = c0 + ly + 8 * k, r = r0 + lx;
            if (c < Cpad && r < Rpad)
                j.dst[dbase + (int64_t)c * Rpad + r] = (r < R && c < C) ? f2bf(tile[lx][ly + 8 * k]) : (uint16_t)0;
        }
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

// The single re-layouts are one-job launches of the batched kernel (its
// transposing and 16-byte paths; the values are the same roundings).
static hipError_t launch_wprep_one(int kind, const void* W, bool w_is_f32, int cin, int cout, int pad, uint16_t* Wk,
                            hipStream_t s)
{
    WprepList l{};
    l.count = 1;
    l.job[0] = WprepJob{kind, w_is_f32, cin, cout, pad, W, Wk};
    return launch_wprep_multi(l, s);
}

hipError_t launch_wprep_fwd(const void* W, bool w_is_f32, int cin, int cout, int copad, uint16_t* Wk, hipStream_t s)
{
    return launch_wprep_one(0, W, w_is_f32, cin, cout, copad, Wk, s);
}

hipError_t launch_wprep_fwd_pad(const void* W, bool w_is_f32, int cin, int cinp, int cout, int copad, uint16_t* Wk,
                                hipStream_t s)
{
    hipLaunchKernelGGL(wprep_fwd_pad_kernel, dim3(blocks_for((int64_t)27 * copad * cinp)), dim3(256), 0, s, W, w_is_f32,
                       cin, cinp, cout, copad, Wk);
    return hipGetLastError();
}

hipError_t launch_wprep_dgrad(const void* W, bool w_is_f32, int cin, int cout, int cipad, uint16_t* Wk, hipStream_t s)
{
    return launch_wprep_one(1, W, w_is_f32, cin, cout, cipad, Wk, s);
}

hipError_t launch_wprep_c4(const void* W, bool w_is_f32, int cout, int copad, uint16_t* Wk, hipStream_t s)
{
    return launch_wprep_one(2, W, w_is_f32, 4, cout, copad, Wk, s);
}

hipError_t launch_wprep_multi(const WprepList& l_in, hipStream_t s)
{
    if (l_in.count <= 0) return hipSuccess;
    // each job gets the blocks it needs (capped), laid end to end in one grid,
    // instead of every job getting the largest job's count
    WprepList l = l_in;
    int total = 0;
    for (int i = 0; i < l.count; ++i) {
        const WprepJob& j = l.job[i];
        int64_t b;
        if (j.kind == 1) b = blocks_for((int64_t)27 * j.pad * j.cout / (j.cout % 8 == 0 ? 8 : 1));
        else if (j.kind == 0) b = (int64_t)27 * ((j.cin + WT - 1) / WT) * ((j.pad + WT - 1) / WT);
        else b = blocks_for((int64_t)j.pad * 128);
        if (b < 1) b = 1;
        if (b > 4096) b = 4096;
        l.start[i] = total;
        total += (int)b;
    }
    l.start[l.count] = total;
    hipLaunchKernelGGL(wprep_multi_kernel, dim3((unsigned)total), dim3(256), 0, s, l);
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
