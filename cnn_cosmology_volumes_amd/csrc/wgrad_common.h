// Internal helpers shared by the backward-weight translation units
// (k_wgrad.hip: Cin % 32 == 0 and the split reduction; k_wgrad_c4.hip: the
// 4-channel first layer, compiled on its own with other scheduler options).
#pragma once

#include "cf_internal.h"

namespace cf {

// Tile of the 4-channel backward-weight (its plan lives with the others).
constexpr int C4_TD = 4, C4_TH = 4, C4_TW = 16;

namespace {

// Box coordinates (sample, box d, box h, box w) in row-major box order.
// Decoded once per block, then advanced one box at a time in 32-bit
// arithmetic (a 64-bit divide per box costs hundreds of VALU instructions).
struct BoxPos {
    int n, bd, bh, bw;
};

__device__ __forceinline__ BoxPos box_decode(int64_t box, int bD, int bH, int bW)
{
    BoxPos p;
    p.bw = (int)(box % bW); box /= bW;
    p.bh = (int)(box % bH); box /= bH;
    p.bd = (int)(box % bD);
    p.n = (int)(box / bD);
    return p;
}

__device__ __forceinline__ BoxPos box_next(BoxPos p, int bD, int bH, int bW)
{
    if (++p.bw == bW) {
        p.bw = 0;
        if (++p.bh == bH) {
            p.bh = 0;
            if (++p.bd == bD) { p.bd = 0; ++p.n; }
        }
    }
    return p;
}

// The same position, marked wave-uniform (scalar registers), so that
// buffer resources built from it need no per-lane handling.
__device__ __forceinline__ BoxPos box_uniform(BoxPos p)
{
    p.n = __builtin_amdgcn_readfirstlane(p.n);
    p.bd = __builtin_amdgcn_readfirstlane(p.bd);
    p.bh = __builtin_amdgcn_readfirstlane(p.bh);
    p.bw = __builtin_amdgcn_readfirstlane(p.bw);
    return p;
}

}  // namespace

// dW[e] = sum over splits of part[s][e] in a fixed order (deterministic).
hipError_t launch_wgrad_reduce(const float* part, float* dW, int64_t n, int splits, hipStream_t s);
// The 4-channel backward-weight's fp32 partials ([splits][27*4*cout]), cout
// 32 or 16; with dP, P and idx non-null (fused, cout 32) the conv-output
// gradient is rebuilt from the pooled gradient, else it is read from dY.
hipError_t launch_wgrad_c4_partials(const WgradPlan& p, const uint16_t* X, const uint16_t* dY, const uint16_t* dP,
                                    const uint16_t* P, const uint8_t* idx, float slope, float* part, const cf_dims& x,
                                    int cout, hipStream_t s);

}  // namespace cf
