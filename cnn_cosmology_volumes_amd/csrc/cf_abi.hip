// C ABI of libcf.so: argument validation, path selection and the training
// step.  Every entry point validates before enqueuing anything, enqueues on
// the caller's stream, and never synchronises or allocates device memory.
// The library keeps no host state between calls besides the thread-local
// error text: the training step's second stream and its events, when used,
// are the caller's (cf_step_aux).
#include "cf_internal.h"

#include <atomic>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

namespace cf {
namespace {

thread_local char g_err[512] = "";

cf_status fail(cf_status s, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

}  // namespace

cf_status report(cf_status s, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

namespace {

cf_status check_hip(hipError_t e, const char* what)
{
    if (e == hipSuccess) return CF_OK;
    return fail(CF_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define CF_TRY_HIP(expr, what)                                   \
    do {                                                         \
        cf_status st_ = check_hip((expr), (what));               \
        if (st_ != CF_OK) return st_;                            \
    } while (0)

bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
size_t up256(size_t b) { return (b + 255) & ~(size_t)255; }
int roundup(int v, int m) { return (v + m - 1) / m * m; }

constexpr int64_t kMaxDim = (int64_t)1 << 30;
constexpr int64_t kMaxElems = (int64_t)1 << 40;

cf_status check_dims(const cf_dims& x, const char* name)
{
    if (x.n <= 0 || x.d <= 0 || x.h <= 0 || x.w <= 0 || x.c <= 0)
        return fail(CF_ERR_INVALID, "%s: every dimension must be positive", name);
    if (x.n > kMaxDim || x.d > kMaxDim || x.h > kMaxDim || x.w > kMaxDim || x.c > 65536)
        return fail(CF_ERR_INVALID, "%s: dimension too large", name);
    const double el = (double)x.n * (double)x.d * (double)x.h * (double)x.w * (double)x.c;
    if (el > (double)kMaxElems) return fail(CF_ERR_INVALID, "%s: tensor too large", name);
    return CF_OK;
}

cf_status check_dtype(cf_dtype dt)
{
    if (dt != CF_F32 && dt != CF_BF16) return fail(CF_ERR_INVALID, "unknown dtype %d", (int)dt);
    return CF_OK;
}

cf_status check_conv(cf_dtype dt, const cf_dims& x, int32_t cout, const cf_conv& cv)
{
    cf_status s = check_dtype(dt);
    if (s != CF_OK) return s;
    if ((s = check_dims(x, "x")) != CF_OK) return s;
    if (cout <= 0 || cout > 65536) return fail(CF_ERR_INVALID, "cout must be in 1..65536");
    const bool s1 = cv.k == 3 && cv.stride == 1 && cv.pad == 1;
    const bool s2 = cv.k == 3 && cv.stride == 2 && cv.pad == (int)(x.d & 1) && (x.d & 1) == (x.h & 1) &&
                    (x.d & 1) == (x.w & 1);
    if (!s1 && !s2)
        return fail(CF_ERR_UNSUPPORTED,
                    "only k=3 with stride 1, pad 1, or stride 2 with \"same\" padding (pad = 1 for odd sizes, 0 for "
                    "even, all three sizes of one parity) is implemented (got k=%d stride=%d pad=%d)", cv.k,
                    cv.stride, cv.pad);
    const double el = (double)x.n * x.d * x.h * x.w * (double)cout;
    if (el > (double)kMaxElems) return fail(CF_ERR_INVALID, "output tensor too large");
    return CF_OK;
}

// ------------------------------------------------------------ path choice
cf_dims with_c(const cf_dims& x, int64_t c) { cf_dims y = x; y.c = c; return y; }

enum class Fwd { Mfma, C4, F32Mfma, MfmaPad, Direct };
enum class Wg { Mfma, C4, F32Mfma, MfmaPad, Direct };

// The MFMA conv kernels address a tile's six input planes (of `cin`
// channels) and the weight copy with 32-bit byte offsets; a shape beyond
// that takes the direct kernel.
bool mfma_offsets_fit(const cf_dims& x, int64_t cin, int64_t cout)
{
    const int64_t lim = (int64_t)1 << 31;
    return 6 * x.h * x.w * cin * 2 < lim && 27 * roundup((int)cout, 128) * cin * 2 < lim;
}


// bf16 layers whose input channels are a multiple of 8 but not of 32 (and
// more than 4) run the bf16 MFMA kernels on a copy of the input padded with
// zero channels to the next multiple of 32 (MfmaPad): the zero channels add
// exact zeros to every sum, at twice the MFMA work for 16 channels, where the
// fp32 matrix cores would run at a sixteenth of the rate.
int64_t pad32(int64_t c) { return (c + 31) / 32 * 32; }
bool pad_path_ok(cf_dtype dt, const cf_dims& x, int cout)
{
    return dt == CF_BF16 && x.c > 4 && x.c % 8 == 0 && x.c % 32 != 0 && cout % 4 == 0 &&
           mfma_offsets_fit(x, pad32(x.c), cout);
}
size_t xpad_bytes(const cf_dims& x) { return (size_t)(x.n * x.d * x.h * x.w) * (size_t)pad32(x.c) * 2; }

Fwd fwd_path(cf_dtype dt, const cf_dims& x, int cout)
{
    const int64_t cin = x.c;
    if (dt == CF_BF16 && cout % 4 == 0) {
        if (cin % 32 == 0 && mfma_offsets_fit(x, cin, cout)) return Fwd::Mfma;
        if (cin == 4 && conv_c4_fits(x)) return Fwd::C4;
        if (pad_path_ok(dt, x, cout)) return Fwd::MfmaPad;
    }
    // fp32 layers, and bf16 layers of other channel counts (multiples of 4)
    if (conv_f32_mfma_ok(x, cout)) return Fwd::F32Mfma;
    return Fwd::Direct;
}

// backward-data runs the forward kernels with in = cout, out = cin
Fwd dgrad_path(cf_dtype dt, const cf_dims& x, int cout)
{
    const int64_t cin = x.c;
    if (dt == CF_BF16 && cout % 32 == 0 && cin % 4 == 0 && mfma_offsets_fit(x, cout, cin)) return Fwd::Mfma;
    if (conv_f32_mfma_ok(with_c(x, cout), (int)cin)) return Fwd::F32Mfma;
    return Fwd::Direct;
}

Wg wgrad_path(cf_dtype dt, const cf_dims& x, int cout)
{
    if (dt == CF_BF16) {
        if (x.c % 32 == 0 && cout % 32 == 0 && wgrad_mfma_fits(x, cout)) return Wg::Mfma;
        if (x.c == 4 && (cout == 32 || cout == 16) && wgrad_c4_fits(x)) return Wg::C4;
        if (cout % 32 == 0 && pad_path_ok(dt, x, cout) && wgrad_mfma_fits(with_c(x, pad32(x.c)), cout))
            return Wg::MfmaPad;
    }
    if (x.c % 4 == 0 && cout % 4 == 0) return Wg::F32Mfma;
    return Wg::Direct;
}

size_t esize(cf_dtype dt) { return dt == CF_F32 ? 4 : 2; }

// Fused block kernels exist for the 4-channel first layer in bf16.
bool fused_pool_fwd_c4(cf_dtype dt, const cf_dims& x, int cout)
{
    return dt == CF_BF16 && x.c == 4 && cout % 32 == 0 && conv_c4_pool_fits(x, cout);
}
// The conv + pool forward is fused for Cin = 4 (one launch), and on the
// MFMA path for plans with 4x4x16 tiles and no channel split (one launch) or
// with a channel split (the partials' reduction pools).
bool fused_pool_fwd_mfma(cf_dtype dt, const cf_dims& x, int cout)
{
    return fwd_path(dt, x, cout) == Fwd::Mfma && conv_mfma_can_pool(plan_conv_mfma(x, cout), x);
}
bool fused_pool_fwd(cf_dtype dt, const cf_dims& x, int cout)
{
    return fused_pool_fwd_c4(dt, x, cout) || fused_pool_fwd_mfma(dt, x, cout);
}
// (the fused kernel takes 32 output channels)
bool fused_pool_wgrad(cf_dtype dt, const cf_dims& x, int cout)
{
    return cout == 32 && wgrad_path(dt, x, cout) == Wg::C4;
}

// Bytes of re-laid weights each path uses.
size_t fwd_wk_bytes(Fwd p, int64_t cin, int cout)
{
    switch (p) {
    case Fwd::Mfma: return (size_t)27 * roundup(cout, 128) * (size_t)cin * 2;
    case Fwd::C4: return (size_t)roundup(cout, 128) * 128 * 2;
    case Fwd::F32Mfma: return conv_f32_wk_bytes((int)cin, cout);
    case Fwd::MfmaPad: return (size_t)27 * roundup(cout, 128) * (size_t)pad32(cin) * 2;
    default: return 0;
    }
}

size_t dgrad_wk_bytes(Fwd p, cf_dtype dt, int64_t cin, int cout)
{
    if (p == Fwd::Mfma) return (size_t)27 * roundup((int)cin, 128) * (size_t)cout * 2;
    if (p == Fwd::F32Mfma) return conv_f32_wk_bytes(cout, (int)cin);
    return (size_t)27 * (size_t)cin * cout * esize(dt);
}

// Stride 2 runs as the stride-1 convolution sampled at 2o + q (q = 1 - pad)
// (k_resample.hip).  Output size ceil(size / 2).
const cf_conv kConv1 = {3, 1, 1};
int s2_q(const cf_conv& cv) { return 1 - cv.pad; }
cf_dims s2_out(const cf_dims& x, int64_t c) { return cf_dims{x.n, (x.d + 1) / 2, (x.h + 1) / 2, (x.w + 1) / 2, c}; }
size_t full_bytes(const cf_dims& x, int64_t c, cf_dtype dt) { return (size_t)(x.n * x.d * x.h * x.w) * c * esize(dt); }

// Enqueue the forward conv given prepared weights `wk` (layout per path; for
// the direct path `wk` is DHWIO in the data type).
hipError_t run_fwd(Fwd p, cf_dtype dt, const cf_dims& x, const void* X, const void* wk, int cout, void* Y, float* part,
                   hipStream_t s)
{
    switch (p) {
    case Fwd::Mfma: {
        const ConvPlan plan = plan_conv_mfma(x, cout);
        return launch_conv_mfma(plan, (const uint16_t*)X, (const uint16_t*)wk, (uint16_t*)Y, part, x, cout,
                                roundup(cout, 128), s);
    }
    case Fwd::C4:
        return launch_conv_c4_fwd((const uint16_t*)X, (const uint16_t*)wk, (uint16_t*)Y, x, cout, roundup(cout, 128), s);
    case Fwd::F32Mfma:
        if (dt == CF_F32) return launch_conv_f32_mfma((const float*)X, (const float*)wk, (float*)Y, x, cout, s);
        return launch_conv_f32_mfma((const uint16_t*)X, (const float*)wk, (uint16_t*)Y, x, cout, s);
    case Fwd::MfmaPad: {
        // scratch: the padded input, then the plan's partials
        const cf_dims xp = with_c(x, pad32(x.c));
        uint16_t* xpad = reinterpret_cast<uint16_t*>(part);
        float* part2 = reinterpret_cast<float*>(reinterpret_cast<char*>(part) + up256(xpad_bytes(x)));
        const hipError_t e = launch_pad_channels((const uint16_t*)X, xpad, x.n * x.d * x.h * x.w, (int)x.c, (int)xp.c, s);
        if (e != hipSuccess) return e;
        return launch_conv_mfma(plan_conv_mfma(xp, cout), xpad, (const uint16_t*)wk, (uint16_t*)Y, part2, xp, cout,
                                roundup(cout, 128), s);
    }
    default:
        if (dt == CF_F32) return launch_conv_direct<float>((const float*)X, (const float*)wk, (float*)Y, x, cout, s);
        return launch_conv_direct<uint16_t>((const uint16_t*)X, (const uint16_t*)wk, (uint16_t*)Y, x, cout, s);
    }
}

size_t fwd_part_bytes(Fwd p, const cf_dims& x, int cout)
{
    if (p == Fwd::MfmaPad) return up256(xpad_bytes(x)) + plan_conv_mfma(with_c(x, pad32(x.c)), cout).part_bytes;
    return p == Fwd::Mfma ? plan_conv_mfma(x, cout).part_bytes : 0;
}

// Backward-data with prepared weights: x is the forward input shape.
hipError_t run_dgrad(Fwd p, cf_dtype dt, const cf_dims& x, const void* dY, const void* wk, int cout, void* dX,
                     float* part, hipStream_t s)
{
    const cf_dims y = with_c(x, cout);          // dY shape: forward output
    if (p == Fwd::Mfma) {
        const ConvPlan plan = plan_conv_mfma(y, (int)x.c);
        return launch_conv_mfma(plan, (const uint16_t*)dY, (const uint16_t*)wk, (uint16_t*)dX, part, y, (int)x.c,
                                roundup((int)x.c, 128), s);
    }
    if (p == Fwd::F32Mfma && dt == CF_F32)
        return launch_conv_f32_mfma((const float*)dY, (const float*)wk, (float*)dX, y, (int)x.c, s);
    if (p == Fwd::F32Mfma)
        return launch_conv_f32_mfma((const uint16_t*)dY, (const float*)wk, (uint16_t*)dX, y, (int)x.c, s);
    if (dt == CF_F32) return launch_conv_direct<float>((const float*)dY, (const float*)wk, (float*)dX, y, (int)x.c, s);
    return launch_conv_direct<uint16_t>((const uint16_t*)dY, (const uint16_t*)wk, (uint16_t*)dX, y, (int)x.c, s);
}

size_t dgrad_part_bytes(Fwd p, const cf_dims& x, int cout)
{
    return p == Fwd::Mfma ? plan_conv_mfma(with_c(x, cout), (int)x.c).part_bytes : 0;
}

size_t wgrad_part_bytes(Wg p, cf_dtype dt, const cf_dims& x, int cout)
{
    if (p == Wg::F32Mfma) return plan_wgrad_f32(x, cout).part_bytes;
    if (p == Wg::MfmaPad) {
        // the padded input, the padded gradient [27][pad32(cin)][cout], the partials
        const cf_dims xp = with_c(x, pad32(x.c));
        return up256(xpad_bytes(x)) + up256((size_t)27 * xp.c * cout * 4) + plan_wgrad(xp, cout).part_bytes;
    }
    if (p != Wg::Direct) return plan_wgrad(x, cout).part_bytes;
    return dt == CF_F32 ? wgrad_direct_part_bytes<float>(x, cout) : wgrad_direct_part_bytes<uint16_t>(x, cout);
}

hipError_t run_wgrad(Wg p, cf_dtype dt, const cf_dims& x, const void* X, const void* dY, int cout, float* dW,
                     float* part, hipStream_t s)
{
    if (p == Wg::F32Mfma && dt == CF_F32)
        return launch_wgrad_f32_mfma(plan_wgrad_f32(x, cout), (const float*)X, (const float*)dY, part, dW, x, cout, s);
    if (p == Wg::F32Mfma)
        return launch_wgrad_f32_mfma(plan_wgrad_f32(x, cout), (const uint16_t*)X, (const uint16_t*)dY, part, dW, x,
                                     cout, s);
    if (p == Wg::MfmaPad) {
        const cf_dims xp = with_c(x, pad32(x.c));
        char* c8 = reinterpret_cast<char*>(part);
        uint16_t* xpad = reinterpret_cast<uint16_t*>(c8);
        float* dwp = reinterpret_cast<float*>(c8 + up256(xpad_bytes(x)));
        float* part2 = reinterpret_cast<float*>(c8 + up256(xpad_bytes(x)) + up256((size_t)27 * xp.c * cout * 4));
        hipError_t e = launch_pad_channels((const uint16_t*)X, xpad, x.n * x.d * x.h * x.w, (int)x.c, (int)xp.c, s);
        if (e != hipSuccess) return e;
        e = launch_wgrad(plan_wgrad(xp, cout), xpad, (const uint16_t*)dY, part2, dwp, xp, cout, s);
        if (e != hipSuccess) return e;
        return launch_unpad_dw(dwp, dW, (int)x.c, (int)xp.c, cout, s);
    }
    if (p != Wg::Direct) {
        const WgradPlan plan = plan_wgrad(x, cout);
        return launch_wgrad(plan, (const uint16_t*)X, (const uint16_t*)dY, part, dW, x, cout, s);
    }
    if (dt == CF_F32) return launch_wgrad_direct<float>((const float*)X, (const float*)dY, part, dW, x, cout, s);
    return launch_wgrad_direct<uint16_t>((const uint16_t*)X, (const uint16_t*)dY, part, dW, x, cout, s);
}

// The weight source of the fp32 matrix-core kernels: fp32 layers take fp32
// weights as they are; bf16 layers take bf16 weights, or round fp32 masters.
F32WSrc f32_wsrc(cf_dtype dt, bool src_f32)
{
    return dt == CF_F32 ? F32WSrc::F32 : src_f32 ? F32WSrc::F32RoundBf16 : F32WSrc::Bf16;
}

// Prepare forward weights from a DHWIO source (fp32 master or bf16).
hipError_t prep_fwd(Fwd p, cf_dtype dt, const void* W, bool src_f32, int64_t cin, int cout, void* wk, hipStream_t s)
{
    switch (p) {
    case Fwd::Mfma: return launch_wprep_fwd(W, src_f32, (int)cin, cout, roundup(cout, 128), (uint16_t*)wk, s);
    case Fwd::C4: return launch_wprep_c4(W, src_f32, cout, roundup(cout, 128), (uint16_t*)wk, s);
    case Fwd::F32Mfma: return launch_wprep_f32(W, f32_wsrc(dt, src_f32), (int)cin, cout, false, (float*)wk, s);
    case Fwd::MfmaPad:
        return launch_wprep_fwd_pad(W, src_f32, (int)cin, (int)pad32(cin), cout, roundup(cout, 128), (uint16_t*)wk, s);
    default: return hipSuccess;
    }
}

hipError_t prep_dgrad(Fwd p, cf_dtype dt, const void* W, bool src_f32, int64_t cin, int cout, void* wk, hipStream_t s)
{
    if (p == Fwd::Mfma) return launch_wprep_dgrad(W, src_f32, (int)cin, cout, roundup((int)cin, 128), (uint16_t*)wk, s);
    if (p == Fwd::F32Mfma) return launch_wprep_f32(W, f32_wsrc(dt, src_f32), (int)cin, cout, true, (float*)wk, s);
    return launch_wprep_direct_dgrad(W, dt, (int)cin, cout, wk, s);
}

}  // namespace
}  // namespace cf

using namespace cf;

extern "C" {

int32_t cf_abi_version(void) { return CF_ABI_VERSION; }

const char* cf_status_string(cf_status s)
{
    switch (s) {
    case CF_OK: return "ok";
    case CF_ERR_INVALID: return "invalid argument";
    case CF_ERR_UNSUPPORTED: return "unsupported configuration";
    case CF_ERR_WORKSPACE: return "workspace too small";
    case CF_ERR_HIP: return "HIP error";
    default: return "unknown status";
    }
}

const char* cf_last_error(void) { return g_err; }

size_t cf_conv3d_workspace_size(cf_dtype dtype, cf_dims x, int32_t cout, cf_conv conv, cf_conv_pass pass)
{
    if (check_conv(dtype, x, cout, conv) != CF_OK) return 0;
    if (conv.stride == 2) {
        if (pass != CF_CONV_FWD && pass != CF_CONV_BWD_DATA && pass != CF_CONV_BWD_WEIGHT) return 0;
        if (cout % 4) return 0;
        return cf_conv3d_workspace_size(dtype, x, cout, kConv1, pass) + up256(full_bytes(x, cout, dtype));
    }
    switch (pass) {
    case CF_CONV_FWD: {
        const Fwd p = fwd_path(dtype, x, cout);
        return up256(fwd_wk_bytes(p, x.c, cout)) + up256(fwd_part_bytes(p, x, cout));
    }
    case CF_CONV_BWD_DATA: {
        const Fwd p = dgrad_path(dtype, x, cout);
        return up256(dgrad_wk_bytes(p, dtype, x.c, cout)) + up256(dgrad_part_bytes(p, x, cout));
    }
    case CF_CONV_BWD_WEIGHT:
        return up256(wgrad_part_bytes(wgrad_path(dtype, x, cout), dtype, x, cout));
    case CF_CONV_POOL_FWD: {
        if ((x.d & 1) || (x.h & 1) || (x.w & 1)) return 0;
        const Fwd p = fwd_path(dtype, x, cout);
        const size_t z = fused_pool_fwd(dtype, x, cout) ? 0 : (size_t)(x.n * x.d * x.h * x.w) * cout * esize(dtype);
        return up256(fwd_wk_bytes(p, x.c, cout)) + up256(fwd_part_bytes(p, x, cout)) + up256(z);
    }
    case CF_POOL_CONV_BWD_WEIGHT: {
        if ((x.d & 1) || (x.h & 1) || (x.w & 1)) return 0;
        const size_t z = fused_pool_wgrad(dtype, x, cout) ? 0 : (size_t)(x.n * x.d * x.h * x.w) * cout * esize(dtype);
        return up256(wgrad_part_bytes(wgrad_path(dtype, x, cout), dtype, x, cout)) + up256(z);
    }
    default:
        return 0;
    }
}

cf_status cf_conv3d_pool_fwd(cf_dtype dtype, cf_dims x, const void* X, const void* W, int32_t cout, cf_conv conv,
                             float slope, void* P, uint8_t* idx, void* ws, size_t ws_bytes, hipStream_t stream)
{
    cf_status st = check_conv(dtype, x, cout, conv);
    if (st != CF_OK) return st;
    if (conv.stride != 1) return fail(CF_ERR_UNSUPPORTED, "cf_conv3d_pool_fwd: stride 1 only");
    if ((x.d & 1) || (x.h & 1) || (x.w & 1))
        return fail(CF_ERR_UNSUPPORTED, "cf_conv3d_pool_fwd: 2^3 stride-2 pooling needs even D, H, W");
    if (!X || !W || !P || !idx) return fail(CF_ERR_INVALID, "cf_conv3d_pool_fwd: null tensor pointer");
    if (!al16(X) || !al16(W) || !al16(P) || !al16(idx))
        return fail(CF_ERR_INVALID, "cf_conv3d_pool_fwd: pointers must be 16-byte aligned");
    if (!(slope >= 0.f)) return fail(CF_ERR_INVALID, "cf_conv3d_pool_fwd: slope must be >= 0 (got %g)", (double)slope);
    const Fwd p = fwd_path(dtype, x, cout);
    const bool fused = fused_pool_fwd(dtype, x, cout);
    const size_t wkb = up256(fwd_wk_bytes(p, x.c, cout)), pb = up256(fwd_part_bytes(p, x, cout));
    const size_t zb = fused ? 0 : up256((size_t)(x.n * x.d * x.h * x.w) * cout * esize(dtype));
    if (ws_bytes < wkb + pb + zb)
        return fail(CF_ERR_WORKSPACE, "cf_conv3d_pool_fwd: workspace %zu < %zu bytes", ws_bytes, wkb + pb + zb);
    if (wkb + pb + zb && (!ws || !al16(ws))) return fail(CF_ERR_INVALID, "cf_conv3d_pool_fwd: workspace null or misaligned");
    char* w8 = (char*)ws;
    const void* wk = W;
    if (p != Fwd::Direct) {
        CF_TRY_HIP(prep_fwd(p, dtype, W, false, x.c, cout, w8, stream), "weight re-layout");
        wk = w8;
    }
    if (fused) {
        if (p == Fwd::Mfma)
            CF_TRY_HIP(launch_conv_mfma_pool(plan_conv_mfma(x, cout), (const uint16_t*)X, (const uint16_t*)wk,
                                             (uint16_t*)P, idx, slope, x, cout, roundup(cout, 128),
                                             pb ? (float*)(w8 + wkb) : nullptr, stream),
                       "fused conv3d + pool forward");
        else
            CF_TRY_HIP(launch_conv_c4_pool_fwd((const uint16_t*)X, (const uint16_t*)wk, (uint16_t*)P, idx, slope, x,
                                               cout, stream), "fused conv3d + pool forward");
        return CF_OK;
    }
    void* Z = w8 + wkb + pb;
    CF_TRY_HIP(run_fwd(p, dtype, x, X, wk, cout, Z, (float*)(w8 ? w8 + wkb : nullptr), stream), "conv3d forward");
    const cf_dims z = with_c(x, cout);
    hipError_t e = dtype == CF_F32 ? launch_pool_fwd<float>((const float*)Z, (float*)P, idx, z, slope, stream)
                                   : launch_pool_fwd<uint16_t>((const uint16_t*)Z, (uint16_t*)P, idx, z, slope, stream);
    CF_TRY_HIP(e, "pool forward");
    return CF_OK;
}

cf_status cf_pool_conv3d_bwd_weight(cf_dtype dtype, cf_dims x, const void* X, const void* dP, const void* P,
                                    const uint8_t* idx, int32_t cout, cf_conv conv, float slope, float* dW, void* ws,
                                    size_t ws_bytes, hipStream_t stream)
{
    cf_status st = check_conv(dtype, x, cout, conv);
    if (st != CF_OK) return st;
    if (conv.stride != 1) return fail(CF_ERR_UNSUPPORTED, "cf_pool_conv3d_bwd_weight: stride 1 only");
    if ((x.d & 1) || (x.h & 1) || (x.w & 1))
        return fail(CF_ERR_UNSUPPORTED, "cf_pool_conv3d_bwd_weight: 2^3 stride-2 pooling needs even D, H, W");
    if (!X || !dP || !P || !idx || !dW) return fail(CF_ERR_INVALID, "cf_pool_conv3d_bwd_weight: null tensor pointer");
    if (!al16(X) || !al16(dP) || !al16(P) || !al16(idx) || !al16(dW))
        return fail(CF_ERR_INVALID, "cf_pool_conv3d_bwd_weight: pointers must be 16-byte aligned");
    if (!(slope >= 0.f)) return fail(CF_ERR_INVALID, "cf_pool_conv3d_bwd_weight: slope must be >= 0 (got %g)", (double)slope);
    const Wg p = wgrad_path(dtype, x, cout);
    const bool fused = fused_pool_wgrad(dtype, x, cout);
    const size_t pb = up256(wgrad_part_bytes(p, dtype, x, cout));
    const size_t zb = fused ? 0 : up256((size_t)(x.n * x.d * x.h * x.w) * cout * esize(dtype));
    if (ws_bytes < pb + zb)
        return fail(CF_ERR_WORKSPACE, "cf_pool_conv3d_bwd_weight: workspace %zu < %zu bytes", ws_bytes, pb + zb);
    if (!ws || !al16(ws)) return fail(CF_ERR_INVALID, "cf_pool_conv3d_bwd_weight: workspace null or misaligned");
    char* w8 = (char*)ws;
    if (fused) {
        CF_TRY_HIP(launch_wgrad_c4_pool(plan_wgrad(x, cout), (const uint16_t*)X, (const uint16_t*)dP,
                                        (const uint16_t*)P, idx, slope, (float*)w8, dW, x, stream),
                   "fused pool backward + conv3d backward-weight");
        return CF_OK;
    }
    void* dZ = w8 + pb;
    const cf_dims z = with_c(x, cout);
    hipError_t e = dtype == CF_F32
                       ? launch_pool_bwd<float>((const float*)dP, (const float*)P, idx, (float*)dZ, z, slope, stream)
                       : launch_pool_bwd<uint16_t>((const uint16_t*)dP, (const uint16_t*)P, idx, (uint16_t*)dZ, z, slope,
                                                   stream);
    CF_TRY_HIP(e, "pool backward");
    CF_TRY_HIP(run_wgrad(p, dtype, x, X, dZ, cout, dW, (float*)w8, stream), "conv3d backward-weight");
    return CF_OK;
}

static cf_status conv_fwd_s1(cf_dtype dtype, cf_dims x, const void* X, const void* W, int32_t cout, cf_conv conv,
                             void* Y, void* ws, size_t ws_bytes, hipStream_t stream)
{
    cf_status st = check_conv(dtype, x, cout, conv);
    if (st != CF_OK) return st;
    if (!X || !W || !Y) return fail(CF_ERR_INVALID, "cf_conv3d_fwd: null tensor pointer");
    if (!al16(X) || !al16(W) || !al16(Y)) return fail(CF_ERR_INVALID, "cf_conv3d_fwd: pointers must be 16-byte aligned");
    const Fwd p = fwd_path(dtype, x, cout);
    const size_t wkb = up256(fwd_wk_bytes(p, x.c, cout));
    const size_t need = wkb + up256(fwd_part_bytes(p, x, cout));
    if (ws_bytes < need) return fail(CF_ERR_WORKSPACE, "cf_conv3d_fwd: workspace %zu < %zu bytes", ws_bytes, need);
    if (need && (!ws || !al16(ws))) return fail(CF_ERR_INVALID, "cf_conv3d_fwd: workspace null or misaligned");
    char* w8 = (char*)ws;
    const void* wk = W;
    if (p != Fwd::Direct) {
        CF_TRY_HIP(prep_fwd(p, dtype, W, false, x.c, cout, w8, stream), "weight re-layout");
        wk = w8;
    }
    CF_TRY_HIP(run_fwd(p, dtype, x, X, wk, cout, Y, (float*)(w8 ? w8 + wkb : nullptr), stream), "conv3d forward");
    return CF_OK;
}

static cf_status conv_bwd_data_s1(cf_dtype dtype, cf_dims x, const void* dY, const void* W, int32_t cout,
                                  cf_conv conv, void* dX, void* ws, size_t ws_bytes, hipStream_t stream)
{
    cf_status st = check_conv(dtype, x, cout, conv);
    if (st != CF_OK) return st;
    if (!dY || !W || !dX) return fail(CF_ERR_INVALID, "cf_conv3d_bwd_data: null tensor pointer");
    if (!al16(dY) || !al16(W) || !al16(dX)) return fail(CF_ERR_INVALID, "cf_conv3d_bwd_data: pointers must be 16-byte aligned");
    const Fwd p = dgrad_path(dtype, x, cout);
    const size_t wkb = up256(dgrad_wk_bytes(p, dtype, x.c, cout));
    const size_t need = wkb + up256(dgrad_part_bytes(p, x, cout));
    if (ws_bytes < need) return fail(CF_ERR_WORKSPACE, "cf_conv3d_bwd_data: workspace %zu < %zu bytes", ws_bytes, need);
    if (!ws || !al16(ws)) return fail(CF_ERR_INVALID, "cf_conv3d_bwd_data: workspace null or misaligned");
    char* w8 = (char*)ws;
    CF_TRY_HIP(prep_dgrad(p, dtype, W, false, x.c, cout, w8, stream), "weight re-layout");
    CF_TRY_HIP(run_dgrad(p, dtype, x, dY, w8, cout, dX, (float*)(w8 + wkb), stream), "conv3d backward-data");
    return CF_OK;
}

static cf_status conv_bwd_weight_s1(cf_dtype dtype, cf_dims x, const void* X, const void* dY, int32_t cout,
                                    cf_conv conv, float* dW, void* ws, size_t ws_bytes, hipStream_t stream)
{
    cf_status st = check_conv(dtype, x, cout, conv);
    if (st != CF_OK) return st;
    if (!X || !dY || !dW) return fail(CF_ERR_INVALID, "cf_conv3d_bwd_weight: null tensor pointer");
    if (!al16(X) || !al16(dY) || !al16(dW)) return fail(CF_ERR_INVALID, "cf_conv3d_bwd_weight: pointers must be 16-byte aligned");
    const Wg p = wgrad_path(dtype, x, cout);
    const size_t need = up256(wgrad_part_bytes(p, dtype, x, cout));
    if (ws_bytes < need) return fail(CF_ERR_WORKSPACE, "cf_conv3d_bwd_weight: workspace %zu < %zu bytes", ws_bytes, need);
    if (!ws || !al16(ws)) return fail(CF_ERR_INVALID, "cf_conv3d_bwd_weight: workspace null or misaligned");
    CF_TRY_HIP(run_wgrad(p, dtype, x, X, dY, cout, dW, (float*)ws, stream), "conv3d backward-weight");
    return CF_OK;
}

// Stride-2 checks shared by the three passes: 4-channel groups for the
// resampling kernels and a workspace for the stride-1 pass plus one
// full-resolution tensor of `cout` channels.
static cf_status s2_prepare(cf_dtype dtype, const cf_dims& x, int32_t cout, cf_conv_pass pass, void* ws,
                            size_t ws_bytes, const char* fn, size_t* s1_bytes)
{
    if (cout % 4) return fail(CF_ERR_UNSUPPORTED, "%s: stride 2 needs a multiple of 4 output channels", fn);
    const size_t s1 = cf_conv3d_workspace_size(dtype, x, cout, kConv1, pass);
    const size_t need = s1 + up256(full_bytes(x, cout, dtype));
    if (ws_bytes < need) return fail(CF_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
    if (!ws || !al16(ws)) return fail(CF_ERR_INVALID, "%s: workspace null or misaligned", fn);
    *s1_bytes = s1;
    return CF_OK;
}

cf_status cf_conv3d_fwd(cf_dtype dtype, cf_dims x, const void* X, const void* W, int32_t cout, cf_conv conv, void* Y,
                        void* ws, size_t ws_bytes, hipStream_t stream)
{
    cf_status st = check_conv(dtype, x, cout, conv);
    if (st != CF_OK) return st;
    if (conv.stride == 1) return conv_fwd_s1(dtype, x, X, W, cout, conv, Y, ws, ws_bytes, stream);
    if (!X || !W || !Y) return fail(CF_ERR_INVALID, "cf_conv3d_fwd: null tensor pointer");
    if (!al16(X) || !al16(W) || !al16(Y)) return fail(CF_ERR_INVALID, "cf_conv3d_fwd: pointers must be 16-byte aligned");
    size_t s1 = 0;
    if ((st = s2_prepare(dtype, x, cout, CF_CONV_FWD, ws, ws_bytes, "cf_conv3d_fwd", &s1)) != CF_OK) return st;
    void* Z = (char*)ws + s1;
    if ((st = conv_fwd_s1(dtype, x, X, W, cout, kConv1, Z, ws, s1, stream)) != CF_OK) return st;
    const cf_dims o = s2_out(x, cout);
    const cf_dims z = with_c(x, cout);
    hipError_t e = dtype == CF_F32
                       ? launch_subsample<float>((const float*)Z, (float*)Y, z, (int)o.d, (int)o.h, (int)o.w, s2_q(conv),
                                                 stream)
                       : launch_subsample<uint16_t>((const uint16_t*)Z, (uint16_t*)Y, z, (int)o.d, (int)o.h, (int)o.w,
                                                    s2_q(conv), stream);
    CF_TRY_HIP(e, "stride-2 subsample");
    return CF_OK;
}

cf_status cf_conv3d_bwd_data(cf_dtype dtype, cf_dims x, const void* dY, const void* W, int32_t cout, cf_conv conv,
                             void* dX, void* ws, size_t ws_bytes, hipStream_t stream)
{
    cf_status st = check_conv(dtype, x, cout, conv);
    if (st != CF_OK) return st;
    if (conv.stride == 1) return conv_bwd_data_s1(dtype, x, dY, W, cout, conv, dX, ws, ws_bytes, stream);
    if (!dY || !W || !dX) return fail(CF_ERR_INVALID, "cf_conv3d_bwd_data: null tensor pointer");
    if (!al16(dY) || !al16(W) || !al16(dX))
        return fail(CF_ERR_INVALID, "cf_conv3d_bwd_data: pointers must be 16-byte aligned");
    size_t s1 = 0;
    if ((st = s2_prepare(dtype, x, cout, CF_CONV_BWD_DATA, ws, ws_bytes, "cf_conv3d_bwd_data", &s1)) != CF_OK) return st;
    void* U = (char*)ws + s1;
    const cf_dims o = s2_out(x, cout);
    const cf_dims z = with_c(x, cout);
    hipError_t e = dtype == CF_F32
                       ? launch_upsample<float>((const float*)dY, (float*)U, z, (int)o.d, (int)o.h, (int)o.w,
                                                s2_q(conv), stream)
                       : launch_upsample<uint16_t>((const uint16_t*)dY, (uint16_t*)U, z, (int)o.d, (int)o.h, (int)o.w,
                                                   s2_q(conv), stream);
    CF_TRY_HIP(e, "stride-2 upsample");
    return conv_bwd_data_s1(dtype, x, U, W, cout, kConv1, dX, ws, s1, stream);
}

cf_status cf_conv3d_bwd_weight(cf_dtype dtype, cf_dims x, const void* X, const void* dY, int32_t cout, cf_conv conv,
                               float* dW, void* ws, size_t ws_bytes, hipStream_t stream)
{
    cf_status st = check_conv(dtype, x, cout, conv);
    if (st != CF_OK) return st;
    if (conv.stride == 1) return conv_bwd_weight_s1(dtype, x, X, dY, cout, conv, dW, ws, ws_bytes, stream);
    if (!X || !dY || !dW) return fail(CF_ERR_INVALID, "cf_conv3d_bwd_weight: null tensor pointer");
    if (!al16(X) || !al16(dY) || !al16(dW))
        return fail(CF_ERR_INVALID, "cf_conv3d_bwd_weight: pointers must be 16-byte aligned");
    size_t s1 = 0;
    if ((st = s2_prepare(dtype, x, cout, CF_CONV_BWD_WEIGHT, ws, ws_bytes, "cf_conv3d_bwd_weight", &s1)) != CF_OK)
        return st;
    void* U = (char*)ws + s1;
    const cf_dims o = s2_out(x, cout);
    const cf_dims z = with_c(x, cout);
    hipError_t e = dtype == CF_F32
                       ? launch_upsample<float>((const float*)dY, (float*)U, z, (int)o.d, (int)o.h, (int)o.w,
                                                s2_q(conv), stream)
                       : launch_upsample<uint16_t>((const uint16_t*)dY, (uint16_t*)U, z, (int)o.d, (int)o.h, (int)o.w,
                                                   s2_q(conv), stream);
    CF_TRY_HIP(e, "stride-2 upsample");
    return conv_bwd_weight_s1(dtype, x, X, U, cout, kConv1, dW, ws, s1, stream);
}

// ------------------------------------------- backward-weight, no allocation
// Scratch of cf_conv3d_bwd_weight_noalloc: the fp32 split partial sums that
// cf_conv3d_bwd_weight keeps in its workspace.  One copy per device, held
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not the device array: kernels get the device address that
// hipGetSymbolAddress returns for the current device, looked up on the first
// call there and kept in g_scratch_dev.
static __device__ __align__(256) unsigned char scratch[CF_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_dev[kMaxScratchDevices];

cf_status scratch_address(void** out)
{
    int dev = -1;
    CF_TRY_HIP(hipGetDevice(&dev), "hipGetDevice");
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(CF_ERR_UNSUPPORTED, "cf_conv3d_bwd_weight_noalloc: device %d beyond the %d this build tracks", dev,
                    kMaxScratchDevices);
    void* p = g_scratch_dev[dev].load(std::memory_order_acquire);
    if (!p) {
        // the same address on every call for this device, so racing first
        // calls store the same value
        CF_TRY_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "scratch address");
        if (!p) return fail(CF_ERR_HIP, "cf_conv3d_bwd_weight_noalloc: scratch address is null");
        g_scratch_dev[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return CF_OK;
}
}  // namespace

cf_status cf_conv3d_bwd_weight_noalloc(cf_dtype dtype, cf_dims x, const void* X, const void* dY, int32_t cout,
                                       cf_conv conv, float* dW, hipStream_t stream)
{
    cf_status st = check_conv(dtype, x, cout, conv);
    if (st != CF_OK) return st;
    if (conv.stride != 1) return fail(CF_ERR_UNSUPPORTED, "cf_conv3d_bwd_weight_noalloc: stride 1 only");
    if (!X || !dY || !dW) return fail(CF_ERR_INVALID, "cf_conv3d_bwd_weight_noalloc: null tensor pointer");
    if (!al16(X) || !al16(dY) || !al16(dW))
        return fail(CF_ERR_INVALID, "cf_conv3d_bwd_weight_noalloc: pointers must be 16-byte aligned");
    const Wg p = wgrad_path(dtype, x, cout);
    const size_t need = up256(wgrad_part_bytes(p, dtype, x, cout));
    if (need > (size_t)CF_NOALLOC_SCRATCH_BYTES)
        return fail(CF_ERR_WORKSPACE,
                    "cf_conv3d_bwd_weight_noalloc: this shape needs %zu bytes of partial sums, more than the %zu-byte "
                    "static scratch; use cf_conv3d_bwd_weight with a workspace", need,
                    (size_t)CF_NOALLOC_SCRATCH_BYTES);
    void* part = nullptr;
    if ((st = scratch_address(&part)) != CF_OK) return st;
    CF_TRY_HIP(run_wgrad(p, dtype, x, X, dY, cout, dW, (float*)part, stream), "conv3d backward-weight");
    return CF_OK;
}

static cf_status check_pool(cf_dtype dtype, const cf_dims& z)
{
    cf_status st = check_dtype(dtype);
    if (st != CF_OK) return st;
    if ((st = check_dims(z, "z")) != CF_OK) return st;
    if ((z.d & 1) || (z.h & 1) || (z.w & 1))
        return fail(CF_ERR_UNSUPPORTED, "2^3 stride-2 pooling needs even D, H, W (got %lld, %lld, %lld)",
                    (long long)z.d, (long long)z.h, (long long)z.w);
    return CF_OK;
}

cf_status cf_pool3d_fwd(cf_dtype dtype, cf_dims z, const void* Z, float slope, void* P, uint8_t* idx,
                        hipStream_t stream)
{
    cf_status st = check_pool(dtype, z);
    if (st != CF_OK) return st;
    if (!Z || !P || !idx) return fail(CF_ERR_INVALID, "cf_pool3d_fwd: null pointer");
    if (!al16(Z) || !al16(P) || !al16(idx)) return fail(CF_ERR_INVALID, "cf_pool3d_fwd: pointers must be 16-byte aligned");
    if (!(slope >= 0.f)) return fail(CF_ERR_INVALID, "cf_pool3d_fwd: slope must be >= 0 (got %g)", (double)slope);
    hipError_t e = dtype == CF_F32 ? launch_pool_fwd<float>((const float*)Z, (float*)P, idx, z, slope, stream)
                                   : launch_pool_fwd<uint16_t>((const uint16_t*)Z, (uint16_t*)P, idx, z, slope, stream);
    CF_TRY_HIP(e, "pool forward");
    return CF_OK;
}

cf_status cf_pool3d_bwd(cf_dtype dtype, cf_dims z, const void* dP, const void* P, const uint8_t* idx, float slope,
                        void* dZ, hipStream_t stream)
{
    cf_status st = check_pool(dtype, z);
    if (st != CF_OK) return st;
    if (!dP || !P || !idx || !dZ) return fail(CF_ERR_INVALID, "cf_pool3d_bwd: null pointer");
    if (!al16(dP) || !al16(P) || !al16(idx) || !al16(dZ))
        return fail(CF_ERR_INVALID, "cf_pool3d_bwd: pointers must be 16-byte aligned");
    if (!(slope >= 0.f)) return fail(CF_ERR_INVALID, "cf_pool3d_bwd: slope must be >= 0 (got %g)", (double)slope);
    hipError_t e = dtype == CF_F32
                       ? launch_pool_bwd<float>((const float*)dP, (const float*)P, idx, (float*)dZ, z, slope, stream)
                       : launch_pool_bwd<uint16_t>((const uint16_t*)dP, (const uint16_t*)P, idx, (uint16_t*)dZ, z, slope,
                                                   stream);
    CF_TRY_HIP(e, "pool backward");
    return CF_OK;
}

cf_status cf_avgpool3d_fwd(cf_dtype dtype, cf_dims z, const void* Z, float slope, void* P, hipStream_t stream)
{
    cf_status st = check_pool(dtype, z);
    if (st != CF_OK) return st;
    if (z.c % 4) return fail(CF_ERR_UNSUPPORTED, "cf_avgpool3d_fwd: channels must be a multiple of 4");
    if (!Z || !P) return fail(CF_ERR_INVALID, "cf_avgpool3d_fwd: null pointer");
    if (!al16(Z) || !al16(P)) return fail(CF_ERR_INVALID, "cf_avgpool3d_fwd: pointers must be 16-byte aligned");
    if (!(slope >= 0.f)) return fail(CF_ERR_INVALID, "cf_avgpool3d_fwd: slope must be >= 0 (got %g)", (double)slope);
    hipError_t e = dtype == CF_F32 ? launch_avgpool_fwd<float>((const float*)Z, (float*)P, z, slope, stream)
                                   : launch_avgpool_fwd<uint16_t>((const uint16_t*)Z, (uint16_t*)P, z, slope, stream);
    CF_TRY_HIP(e, "average pool forward");
    return CF_OK;
}

cf_status cf_avgpool3d_bwd(cf_dtype dtype, cf_dims z, const void* dP, const void* Z, float slope, void* dZ,
                           hipStream_t stream)
{
    cf_status st = check_pool(dtype, z);
    if (st != CF_OK) return st;
    if (z.c % 4) return fail(CF_ERR_UNSUPPORTED, "cf_avgpool3d_bwd: channels must be a multiple of 4");
    if (!dP || !Z || !dZ) return fail(CF_ERR_INVALID, "cf_avgpool3d_bwd: null pointer");
    if (!al16(dP) || !al16(Z) || !al16(dZ))
        return fail(CF_ERR_INVALID, "cf_avgpool3d_bwd: pointers must be 16-byte aligned");
    if (!(slope >= 0.f)) return fail(CF_ERR_INVALID, "cf_avgpool3d_bwd: slope must be >= 0 (got %g)", (double)slope);
    hipError_t e = dtype == CF_F32
                       ? launch_avgpool_bwd<float>((const float*)dP, (const float*)Z, (float*)dZ, z, slope, stream)
                       : launch_avgpool_bwd<uint16_t>((const uint16_t*)dP, (const uint16_t*)Z, (uint16_t*)dZ, z, slope,
                                                      stream);
    CF_TRY_HIP(e, "average pool backward");
    return CF_OK;
}

cf_status cf_lrelu(cf_dtype dtype, int64_t n, const void* x, const void* dy, float slope, void* out,
                   hipStream_t stream)
{
    cf_status st = check_dtype(dtype);
    if (st != CF_OK) return st;
    if (n <= 0 || n > kMaxElems) return fail(CF_ERR_INVALID, "cf_lrelu: n out of range");
    if (!x || !out) return fail(CF_ERR_INVALID, "cf_lrelu: null pointer");
    if (!al16(x) || !al16(out) || (dy && !al16(dy))) return fail(CF_ERR_INVALID, "cf_lrelu: pointers must be 16-byte aligned");
    hipError_t e = dtype == CF_F32
                       ? launch_lrelu<float>((const float*)x, (const float*)dy, (float*)out, n, slope, stream)
                       : launch_lrelu<uint16_t>((const uint16_t*)x, (const uint16_t*)dy, (uint16_t*)out, n, slope, stream);
    CF_TRY_HIP(e, "leaky relu");
    return CF_OK;
}

static cf_status check_dense(int32_t B, int32_t in, int32_t out)
{
    if (B <= 0 || in <= 0 || out <= 0) return fail(CF_ERR_INVALID, "dense: sizes must be positive");
    if ((int64_t)in * out > ((int64_t)1 << 31) || (int64_t)B * in > ((int64_t)1 << 31))
        return fail(CF_ERR_INVALID, "dense: sizes too large");
    return CF_OK;
}

size_t cf_dense_workspace_size(int32_t B, int32_t in, int32_t out)
{
    if (check_dense(B, in, out) != CF_OK) return 0;
    return up256(dense_fwd_part_bytes(B, in, out));
}

cf_status cf_dense_fwd(int32_t B, int32_t in, int32_t out, const float* X, const float* W, const float* bias,
                       float slope, float* pre, float* Y, void* ws, size_t ws_bytes, hipStream_t stream)
{
    cf_status st = check_dense(B, in, out);
    if (st != CF_OK) return st;
    if (!X || !W || !pre || !Y) return fail(CF_ERR_INVALID, "cf_dense_fwd: null pointer");
    if (!al16(X) || !al16(W) || !al16(pre) || !al16(Y) || (bias && !al16(bias)))
        return fail(CF_ERR_INVALID, "cf_dense_fwd: pointers must be 16-byte aligned");
    const size_t need = up256(dense_fwd_part_bytes(B, in, out));
    if (ws_bytes < need) return fail(CF_ERR_WORKSPACE, "cf_dense_fwd: workspace %zu < %zu bytes", ws_bytes, need);
    if (!ws || !al16(ws)) return fail(CF_ERR_INVALID, "cf_dense_fwd: workspace null or misaligned");
    CF_TRY_HIP(launch_dense_fwd(B, in, out, X, nullptr, W, bias, slope, pre, Y, (float*)ws, stream), "dense forward");
    return CF_OK;
}

cf_status cf_dense_bwd(int32_t B, int32_t in, int32_t out, const float* X, const float* W, const float* pre,
                       const float* dY, float slope, float* dX, float* dW, float* db, hipStream_t stream)
{
    cf_status st = check_dense(B, in, out);
    if (st != CF_OK) return st;
    if (!X || !W || !pre || !dY || !dW || !db) return fail(CF_ERR_INVALID, "cf_dense_bwd: null pointer");
    if (!al16(X) || !al16(W) || !al16(pre) || !al16(dY) || !al16(dW) || !al16(db) || (dX && !al16(dX)))
        return fail(CF_ERR_INVALID, "cf_dense_bwd: pointers must be 16-byte aligned");
    CF_TRY_HIP(launch_dense_bwd(B, in, out, X, nullptr, W, pre, dY, slope, dX, nullptr, dW, db, stream), "dense backward");
    return CF_OK;
}

cf_status cf_mse(int32_t B, int32_t K, const float* yhat, const float* t, float* loss, float* dyhat,
                 hipStream_t stream)
{
    if (B <= 0 || K <= 0 || (int64_t)B * K > (1 << 24)) return fail(CF_ERR_INVALID, "cf_mse: sizes out of range");
    if (!yhat || !t || !loss) return fail(CF_ERR_INVALID, "cf_mse: null pointer");
    CF_TRY_HIP(launch_mse(B, K, yhat, t, loss, dyhat, stream), "mse");
    return CF_OK;
}

cf_status cf_sgd(int64_t n, float lr, float* W, const float* dW, hipStream_t stream)
{
    if (n <= 0 || n > kMaxElems) return fail(CF_ERR_INVALID, "cf_sgd: n out of range");
    if (!W || !dW) return fail(CF_ERR_INVALID, "cf_sgd: null pointer");
    CF_TRY_HIP(launch_sgd(n, lr, W, dW, stream), "sgd");
    return CF_OK;
}

// ----------------------------------------------------- Adam + LARC + decay
static cf_status check_opt(const cf_adam_larc_params* hp, int64_t t, int32_t nt, const int64_t* n,
                           const char* fn)
{
    if (!hp || !n) return fail(CF_ERR_INVALID, "%s: null host argument", fn);
    if (nt < 1 || nt > CF_MAX_OPT_TENSORS)
        return fail(CF_ERR_INVALID, "%s: ntensors must be 1..%d (got %d)", fn, CF_MAX_OPT_TENSORS, nt);
    cf_status st = check_adam(hp, t, fn);
    if (st != CF_OK) return st;
    for (int i = 0; i < nt; ++i)
        if (n[i] <= 0 || n[i] > ((int64_t)1 << 36)) return fail(CF_ERR_INVALID, "%s: n[%d] out of range", fn, i);
    return CF_OK;
}

static OptList opt_list(int32_t nt, const int64_t* n, float* const* w, const float* const* g, float* const* m,
                        float* const* v)
{
    OptList l{};
    l.count = nt;
    for (int i = 0; i < nt; ++i) {
        l.n[i] = n[i];
        if (w) { l.w[i] = w[i]; l.g[i] = g[i]; l.m[i] = m[i]; l.v[i] = v[i]; }
    }
    return l;
}

size_t cf_adam_larc_workspace_size(int32_t ntensors, const int64_t* n)
{
    if (ntensors < 1 || ntensors > CF_MAX_OPT_TENSORS || !n) return 0;
    for (int i = 0; i < ntensors; ++i)
        if (n[i] <= 0 || n[i] > ((int64_t)1 << 36)) return 0;
    return up256(adam_larc_part_bytes(opt_list(ntensors, n, nullptr, nullptr, nullptr, nullptr)));
}

cf_status cf_adam_larc(const cf_adam_larc_params* hp, int64_t t, int32_t ntensors, const int64_t* n, float* const* w,
                       const float* const* g, float* const* m, float* const* v, float* lr_out, void* ws,
                       size_t ws_bytes, hipStream_t stream)
{
    cf_status st = check_opt(hp, t, ntensors, n, "cf_adam_larc");
    if (st != CF_OK) return st;
    if (!w || !g || !m || !v) return fail(CF_ERR_INVALID, "cf_adam_larc: null tensor array");
    for (int i = 0; i < ntensors; ++i)
        if (!w[i] || !g[i] || !m[i] || !v[i] || !al16(w[i]) || !al16(g[i]) || !al16(m[i]) || !al16(v[i]))
            return fail(CF_ERR_INVALID, "cf_adam_larc: tensor %d has a null or misaligned pointer", i);
    if (lr_out && !al16(lr_out)) return fail(CF_ERR_INVALID, "cf_adam_larc: lr_out must be 16-byte aligned");
    const OptList l = opt_list(ntensors, n, w, g, m, v);
    const size_t need = up256(adam_larc_part_bytes(l));
    if (ws_bytes < need) return fail(CF_ERR_WORKSPACE, "cf_adam_larc: workspace %zu < %zu bytes", ws_bytes, need);
    if (!ws || !al16(ws)) return fail(CF_ERR_INVALID, "cf_adam_larc: workspace null or misaligned");
    CF_TRY_HIP(launch_adam_larc(l, adam_args(hp, t), (float*)ws, lr_out, stream), "adam + larc");
    return CF_OK;
}

// ------------------------------------------------------------- batch norm
static cf_status check_bn(cf_dtype dtype, const cf_dims& x, const char* fn)
{
    cf_status st = check_dtype(dtype);
    if (st != CF_OK) return st;
    if ((st = check_dims(x, "x")) != CF_OK) return st;
    if (x.c % 4 || x.c > 1024) return fail(CF_ERR_UNSUPPORTED, "%s: channels must be a multiple of 4, at most 1024", fn);
    return CF_OK;
}

size_t cf_batchnorm_workspace_size(cf_dtype dtype, cf_dims x)
{
    if (check_bn(dtype, x, "cf_batchnorm_workspace_size") != CF_OK) return 0;
    return bn_ws_bytes(x);
}

cf_status cf_batchnorm_fwd(cf_dtype dtype, cf_dims x, const void* X, const float* gamma, const float* beta, float eps,
                           void* Y, float* mean, float* invstd, void* ws, size_t ws_bytes, hipStream_t stream)
{
    cf_status st = check_bn(dtype, x, "cf_batchnorm_fwd");
    if (st != CF_OK) return st;
    if (!X || !gamma || !beta || !Y || !mean || !invstd) return fail(CF_ERR_INVALID, "cf_batchnorm_fwd: null pointer");
    if (!al16(X) || !al16(gamma) || !al16(beta) || !al16(Y) || !al16(mean) || !al16(invstd))
        return fail(CF_ERR_INVALID, "cf_batchnorm_fwd: pointers must be 16-byte aligned");
    if (!(eps > 0.f) || !(eps < INFINITY)) return fail(CF_ERR_INVALID, "cf_batchnorm_fwd: eps must be positive and finite");
    const size_t need = bn_ws_bytes(x);
    if (ws_bytes < need) return fail(CF_ERR_WORKSPACE, "cf_batchnorm_fwd: workspace %zu < %zu bytes", ws_bytes, need);
    if (!ws || !al16(ws)) return fail(CF_ERR_INVALID, "cf_batchnorm_fwd: workspace null or misaligned");
    hipError_t e = dtype == CF_F32
                       ? launch_bn_fwd<float>((const float*)X, gamma, beta, eps, (float*)Y, mean, invstd, x, ws, stream)
                       : launch_bn_fwd<uint16_t>((const uint16_t*)X, gamma, beta, eps, (uint16_t*)Y, mean, invstd, x,
                                                 ws, stream);
    CF_TRY_HIP(e, "batch norm forward");
    return CF_OK;
}

cf_status cf_batchnorm_bwd(cf_dtype dtype, cf_dims x, const void* X, const void* dY, const float* gamma,
                           const float* mean, const float* invstd, void* dX, float* dgamma, float* dbeta, void* ws,
                           size_t ws_bytes, hipStream_t stream)
{
    cf_status st = check_bn(dtype, x, "cf_batchnorm_bwd");
    if (st != CF_OK) return st;
    if (!X || !dY || !gamma || !mean || !invstd || !dX || !dgamma || !dbeta)
        return fail(CF_ERR_INVALID, "cf_batchnorm_bwd: null pointer");
    if (!al16(X) || !al16(dY) || !al16(gamma) || !al16(mean) || !al16(invstd) || !al16(dX) || !al16(dgamma) ||
        !al16(dbeta))
        return fail(CF_ERR_INVALID, "cf_batchnorm_bwd: pointers must be 16-byte aligned");
    const size_t need = bn_ws_bytes(x);
    if (ws_bytes < need) return fail(CF_ERR_WORKSPACE, "cf_batchnorm_bwd: workspace %zu < %zu bytes", ws_bytes, need);
    if (!ws || !al16(ws)) return fail(CF_ERR_INVALID, "cf_batchnorm_bwd: workspace null or misaligned");
    hipError_t e = dtype == CF_F32
                       ? launch_bn_bwd<float>((const float*)X, (const float*)dY, gamma, mean, invstd, (float*)dX,
                                              dgamma, dbeta, x, ws, stream)
                       : launch_bn_bwd<uint16_t>((const uint16_t*)X, (const uint16_t*)dY, gamma, mean, invstd,
                                                 (uint16_t*)dX, dgamma, dbeta, x, ws, stream);
    CF_TRY_HIP(e, "batch norm backward");
    return CF_OK;
}

// ------------------------------------------------------------ training step
namespace {

struct LayerPlan {
    cf_dims x;          // block input
    int cout;
    Fwd fwd;
    Fwd dg;
    Wg wg;
    bool fused;         // conv + pool forward and pool backward + wgrad fused (first block)
    bool pool_fused;    // conv + pool forward fused (MFMA path); backward unfused
    size_t wk_fwd, wk_dg, z, p, idx, dp, dw;   // offsets into the workspace
};

struct StepPlan {
    int L;
    LayerPlan layer[CF_MAX_BLOCKS];
    int flat, d0, d1, d2;
    size_t part;        // split-K buffer of the main stream (conv fwd, dgrad, fused block-1 wgrad, dense)
    size_t part_w;      // partial sums of the weight gradients run on the auxiliary stream
    size_t pre1, y1, pre2, y2, pre3, y3, dy3, dy2, dy1, g1;
    size_t dW1, db1, dW2, db2, dW3, db3;
    size_t cast;        // bf16 DHWIO weight copy for direct bf16 fallbacks
    size_t total;
};

cf_status check_model(const cf_model_desc* m, cf_dtype dt, int32_t B)
{
    cf_status st = check_dtype(dt);
    if (st != CF_OK) return st;
    if (!m) return fail(CF_ERR_INVALID, "model description is null");
    if (B <= 0) return fail(CF_ERR_INVALID, "batch must be positive");
    if (m->nblocks < 1 || m->nblocks > CF_MAX_BLOCKS) return fail(CF_ERR_INVALID, "nblocks must be 1..%d", CF_MAX_BLOCKS);
    if (m->cin <= 0 || m->d <= 0 || m->h <= 0 || m->w <= 0) return fail(CF_ERR_INVALID, "input shape must be positive");
    const int div = 1 << m->nblocks;
    if (m->d % div || m->h % div || m->w % div)
        return fail(CF_ERR_UNSUPPORTED, "input D, H, W must be divisible by 2^nblocks");
    for (int l = 0; l < m->nblocks; ++l)
        if (m->filters[l] <= 0 || m->filters[l] > 65536) return fail(CF_ERR_INVALID, "filters[%d] out of range", l);
    for (int k = 0; k < 3; ++k)
        if (m->dense[k] <= 0 || m->dense[k] > 65536) return fail(CF_ERR_INVALID, "dense[%d] out of range", k);
    if (!(m->slope >= 0.f)) return fail(CF_ERR_INVALID, "slope must be >= 0 (got %g)", (double)m->slope);
    cf_dims x{B, m->d, m->h, m->w, m->cin};
    if ((st = check_dims(x, "input")) != CF_OK) return st;
    return CF_OK;
}

StepPlan plan_step(const cf_model_desc* m, cf_dtype dt, int32_t B)
{
    StepPlan P{};
    P.L = m->nblocks;
    size_t off = 0;
    auto take = [&](size_t bytes) { const size_t o = off; off += up256(bytes); return o; };
    const size_t es = esize(dt);
    size_t part = 0, part_w = 0, cast = 0;
    cf_dims x{B, m->d, m->h, m->w, m->cin};
    for (int l = 0; l < P.L; ++l) {
        LayerPlan& Lp = P.layer[l];
        Lp.x = x;
        Lp.cout = m->filters[l];
        Lp.fwd = fwd_path(dt, x, Lp.cout);
        Lp.dg = dgrad_path(dt, x, Lp.cout);
        Lp.wg = wgrad_path(dt, x, Lp.cout);
        const int64_t nvox = x.n * x.d * x.h * x.w;
        const int64_t npool = nvox / 8;
        Lp.wk_fwd = take(Lp.fwd == Fwd::Direct ? 0 : fwd_wk_bytes(Lp.fwd, x.c, Lp.cout));
        Lp.wk_dg = take(l > 0 ? dgrad_wk_bytes(Lp.dg, dt, x.c, Lp.cout) : 0);
        Lp.fused = l == 0 && fused_pool_fwd_c4(dt, x, Lp.cout) && fused_pool_wgrad(dt, x, Lp.cout);
        Lp.pool_fused = !Lp.fused && fused_pool_fwd_mfma(dt, x, Lp.cout);
        Lp.z = take(Lp.fused ? 0 : (size_t)nvox * Lp.cout * es);
        Lp.p = take((size_t)npool * Lp.cout * es);
        Lp.idx = take((size_t)npool * Lp.cout);
        Lp.dp = take((size_t)npool * Lp.cout * es);
        Lp.dw = take((size_t)27 * x.c * Lp.cout * 4);
        size_t pb = fwd_part_bytes(Lp.fwd, x, Lp.cout);
        if (l > 0 && dgrad_part_bytes(Lp.dg, x, Lp.cout) > pb) pb = dgrad_part_bytes(Lp.dg, x, Lp.cout);
        if (Lp.fused) {
            if (wgrad_part_bytes(Lp.wg, dt, x, Lp.cout) > pb) pb = wgrad_part_bytes(Lp.wg, dt, x, Lp.cout);
        } else if (wgrad_part_bytes(Lp.wg, dt, x, Lp.cout) > part_w) {
            part_w = wgrad_part_bytes(Lp.wg, dt, x, Lp.cout);
        }
        if (pb > part) part = pb;
        if (dt == CF_BF16 && Lp.fwd == Fwd::Direct) {
            const size_t c = (size_t)27 * x.c * Lp.cout * 2;
            if (c > cast) cast = c;
        }
        x = cf_dims{B, x.d / 2, x.h / 2, x.w / 2, Lp.cout};
    }
    P.flat = (int)(x.d * x.h * x.w * x.c);
    P.d0 = m->dense[0]; P.d1 = m->dense[1]; P.d2 = m->dense[2];
    size_t dp = dense_fwd_part_bytes(B, P.flat, P.d0);
    if (dense_fwd_part_bytes(B, P.d0, P.d1) > dp) dp = dense_fwd_part_bytes(B, P.d0, P.d1);
    if (dense_fwd_part_bytes(B, P.d1, P.d2) > dp) dp = dense_fwd_part_bytes(B, P.d1, P.d2);
    if (dp > part) part = dp;
    P.part = take(part);
    P.part_w = take(part_w);
    P.cast = take(cast);
    const size_t f = 4;
    P.pre1 = take((size_t)B * P.d0 * f); P.y1 = take((size_t)B * P.d0 * f);
    P.pre2 = take((size_t)B * P.d1 * f); P.y2 = take((size_t)B * P.d1 * f);
    P.pre3 = take((size_t)B * P.d2 * f); P.y3 = take((size_t)B * P.d2 * f);
    P.dy3 = take((size_t)B * P.d2 * f); P.dy2 = take((size_t)B * P.d1 * f); P.dy1 = take((size_t)B * P.d0 * f);
    P.g1 = take((size_t)B * P.d0 * f);
    P.dW1 = take((size_t)P.flat * P.d0 * f); P.db1 = take((size_t)P.d0 * f);
    P.dW2 = take((size_t)P.d0 * P.d1 * f); P.db2 = take((size_t)P.d1 * f);
    P.dW3 = take((size_t)P.d1 * P.d2 * f); P.db3 = take((size_t)P.d2 * f);
    P.total = off;
    return P;
}

__global__ void cast_bf16_kernel(const float* __restrict__ s, uint16_t* __restrict__ d, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) d[i] = f2bf(s[i]);
}

}  // namespace

cf_status cf_step_aux_create(cf_step_aux* aux)
{
    if (!aux) return fail(CF_ERR_INVALID, "cf_step_aux_create: aux is null");
    memset(aux, 0, sizeof(*aux));
    cf_status st = check_hip(hipStreamCreateWithFlags(&aux->stream, hipStreamNonBlocking), "auxiliary stream");
    for (int i = 0; i < CF_MAX_BLOCKS && st == CF_OK; ++i)
        st = check_hip(hipEventCreateWithFlags(&aux->fork[i], hipEventDisableTiming), "fork event");
    if (st == CF_OK) st = check_hip(hipEventCreateWithFlags(&aux->join, hipEventDisableTiming), "join event");
    if (st != CF_OK) {
        char keep[sizeof(g_err)];
        memcpy(keep, g_err, sizeof(keep));
        cf_step_aux_destroy(aux);
        memcpy(g_err, keep, sizeof(keep));
    }
    return st;
}

cf_status cf_step_aux_destroy(cf_step_aux* aux)
{
    if (!aux) return CF_OK;
    cf_status st = CF_OK;
    for (int i = 0; i < CF_MAX_BLOCKS; ++i)
        if (aux->fork[i]) {
            const cf_status e = check_hip(hipEventDestroy(aux->fork[i]), "fork event");
            if (st == CF_OK) st = e;
        }
    if (aux->join) {
        const cf_status e = check_hip(hipEventDestroy(aux->join), "join event");
        if (st == CF_OK) st = e;
    }
    if (aux->stream) {
        const cf_status e = check_hip(hipStreamDestroy(aux->stream), "auxiliary stream");
        if (st == CF_OK) st = e;
    }
    memset(aux, 0, sizeof(*aux));
    return st;
}

size_t cf_train_step_workspace_size(const cf_model_desc* m, cf_dtype dtype, int32_t B)
{
    if (check_model(m, dtype, B) != CF_OK) return 0;
    return plan_step(m, dtype, B).total;
}

cf_status cf_train_step(const cf_model_desc* m, cf_dtype dtype, int32_t B, const void* X, const float* targets,
                        float* const* params, float lr, float* loss_out, float* pred_out, void* ws, size_t ws_bytes,
                        hipStream_t stream, const cf_step_aux* aux)
{
    cf_status st = check_model(m, dtype, B);
    if (st != CF_OK) return st;
    if (!X || !targets || !params || !loss_out) return fail(CF_ERR_INVALID, "cf_train_step: null pointer");
    const int L = m->nblocks;
    for (int i = 0; i < L + 6; ++i)
        if (!params[i] || !al16(params[i])) return fail(CF_ERR_INVALID, "cf_train_step: params[%d] null or misaligned", i);
    if (!al16(X)) return fail(CF_ERR_INVALID, "cf_train_step: X must be 16-byte aligned");
    const StepPlan P = plan_step(m, dtype, B);
    if (ws_bytes < P.total) return fail(CF_ERR_WORKSPACE, "cf_train_step: workspace %zu < %zu bytes", ws_bytes, P.total);
    if (!ws || !al16(ws)) return fail(CF_ERR_INVALID, "cf_train_step: workspace null or misaligned");
    if (aux) {
        if (!aux->stream || !aux->join) return fail(CF_ERR_INVALID, "cf_train_step: aux stream or join event is null");
        if (aux->stream == stream) return fail(CF_ERR_INVALID, "cf_train_step: aux->stream must differ from stream");
        for (int i = 0; i < CF_MAX_BLOCKS; ++i)
            if (!aux->fork[i]) return fail(CF_ERR_INVALID, "cf_train_step: aux->fork[%d] is null", i);
    }
    // weight gradients go to the caller's second stream when one is given
    const bool two = aux != nullptr;
    hipStream_t as = two ? aux->stream : stream;
    char* w = (char*)ws;
    auto F = [&](size_t o) { return (float*)(w + o); };
    float* part = F(P.part);
    const float slope = m->slope;
    const bool bf = dtype == CF_BF16;

    // 1. weight copies for this step (bf16 rounding of the fp32 masters); the
    //    MFMA-path re-layouts of all blocks go in one launch
    static_assert(CF_MAX_BLOCKS <= 8, "WprepList capacity");
    WprepList wl{};
    for (int l = 0; l < L; ++l) {
        const LayerPlan& Lp = P.layer[l];
        if (Lp.fwd == Fwd::Mfma)
            wl.job[wl.count++] = WprepJob{0, true, (int)Lp.x.c, Lp.cout, roundup(Lp.cout, 128), params[l],
                                          (uint16_t*)(w + Lp.wk_fwd)};
        else if (Lp.fwd == Fwd::C4)
            wl.job[wl.count++] = WprepJob{2, true, (int)Lp.x.c, Lp.cout, roundup(Lp.cout, 128), params[l],
                                          (uint16_t*)(w + Lp.wk_fwd)};
        else if (Lp.fwd == Fwd::F32Mfma)
            CF_TRY_HIP(launch_wprep_f32(params[l], f32_wsrc(dtype, true), (int)Lp.x.c, Lp.cout, false,
                                        (float*)(w + Lp.wk_fwd), stream),
                       "weight re-layout");
        else if (Lp.fwd == Fwd::MfmaPad)
            CF_TRY_HIP(launch_wprep_fwd_pad(params[l], true, (int)Lp.x.c, (int)pad32(Lp.x.c), Lp.cout,
                                            roundup(Lp.cout, 128), (uint16_t*)(w + Lp.wk_fwd), stream),
                       "weight re-layout");
        if (l > 0) {
            if (Lp.dg == Fwd::Mfma) {
                wl.job[wl.count++] = WprepJob{1, true, (int)Lp.x.c, Lp.cout, roundup((int)Lp.x.c, 128), params[l],
                                              (uint16_t*)(w + Lp.wk_dg)};
            } else if (Lp.dg == Fwd::F32Mfma) {
                CF_TRY_HIP(launch_wprep_f32(params[l], f32_wsrc(dtype, true), (int)Lp.x.c, Lp.cout, true,
                                            (float*)(w + Lp.wk_dg), stream),
                           "weight re-layout");
            } else if (bf) {
                const int64_t n = (int64_t)27 * Lp.x.c * Lp.cout;
                hipLaunchKernelGGL(cast_bf16_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                                   params[l], (uint16_t*)(w + P.cast), n);
                CF_TRY_HIP(hipGetLastError(), "weight cast");
                CF_TRY_HIP(launch_wprep_direct_dgrad(w + P.cast, dtype, (int)Lp.x.c, Lp.cout, w + Lp.wk_dg, stream),
                           "weight re-layout");
            } else {
                CF_TRY_HIP(launch_wprep_direct_dgrad(params[l], dtype, (int)Lp.x.c, Lp.cout, w + Lp.wk_dg, stream),
                           "weight re-layout");
            }
        }
    }
    CF_TRY_HIP(launch_wprep_multi(wl, stream), "weight re-layout");

    // 2. forward through the blocks
    const void* a = X;
    for (int l = 0; l < L; ++l) {
        const LayerPlan& Lp = P.layer[l];
        const void* wk = w + Lp.wk_fwd;
        if (Lp.fwd == Fwd::Direct) {
            if (bf) {
                const int64_t n = (int64_t)27 * Lp.x.c * Lp.cout;
                hipLaunchKernelGGL(cast_bf16_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                                   params[l], (uint16_t*)(w + P.cast), n);
                CF_TRY_HIP(hipGetLastError(), "weight cast");
                wk = w + P.cast;
            } else {
                wk = params[l];
            }
        }
        if (Lp.fused) {
            CF_TRY_HIP(launch_conv_c4_pool_fwd((const uint16_t*)a, (const uint16_t*)wk, (uint16_t*)(w + Lp.p),
                                               (uint8_t*)(w + Lp.idx), slope, Lp.x, Lp.cout, stream),
                       "fused conv3d + pool forward");
            a = w + Lp.p;
            continue;
        }
        if (Lp.pool_fused) {
            CF_TRY_HIP(launch_conv_mfma_pool(plan_conv_mfma(Lp.x, Lp.cout), (const uint16_t*)a, (const uint16_t*)wk,
                                             (uint16_t*)(w + Lp.p), (uint8_t*)(w + Lp.idx), slope, Lp.x, Lp.cout,
                                             roundup(Lp.cout, 128), part, stream),
                       "fused conv3d + pool forward");
            a = w + Lp.p;
            continue;
        }
        CF_TRY_HIP(run_fwd(Lp.fwd, dtype, Lp.x, a, wk, Lp.cout, w + Lp.z, part, stream), "conv3d forward");
        const cf_dims z = with_c(Lp.x, Lp.cout);
        hipError_t e = bf ? launch_pool_fwd<uint16_t>((const uint16_t*)(w + Lp.z), (uint16_t*)(w + Lp.p),
                                                      (uint8_t*)(w + Lp.idx), z, slope, stream)
                          : launch_pool_fwd<float>((const float*)(w + Lp.z), (float*)(w + Lp.p), (uint8_t*)(w + Lp.idx),
                                                   z, slope, stream);
        CF_TRY_HIP(e, "pool forward");
        a = w + Lp.p;
    }

    // 3. dense head (the flattened NDHWC pooled volume is the dense input)
    const LayerPlan& last = P.layer[L - 1];
    const float* hX = bf ? nullptr : (const float*)(w + last.p);
    const uint16_t* hXb = bf ? (const uint16_t*)(w + last.p) : nullptr;
    const float* W1 = params[L], *b1 = params[L + 1], *W2 = params[L + 2], *b2 = params[L + 3], *W3 = params[L + 4],
                *b3 = params[L + 5];
    CF_TRY_HIP(launch_dense_fwd(B, P.flat, P.d0, hX, hXb, W1, b1, slope, F(P.pre1), F(P.y1), part, stream), "dense1");
    // bf16: the dense input gradient goes through the last block's pool
    // backward inside the dense backward-data kernel, which writes that
    // block's full-resolution conv-output gradient (dP is never stored)
    const bool head_unpool = bf && !last.fused;
    const DenseUnpool dup{(const uint16_t*)(w + last.p), (const uint8_t*)(w + last.idx), (uint16_t*)(w + last.z),
                          (int)(last.x.d / 2), (int)(last.x.h / 2), (int)(last.x.w / 2), last.cout, slope};
    if (dense_head_fits(B, P.d0, P.d1, P.d2)) {
        // layers 2-3, the loss and their backward in one launch; layer 1's
        // gated output gradient g1 then feeds its weight and data gradients
        // with the gate switched off (slope < 0), which gives the same values
        DenseHead h{};
        h.B = B; h.d0 = P.d0; h.d1 = P.d1; h.d2 = P.d2; h.slope = slope;
        h.y1 = F(P.y1); h.pre1 = F(P.pre1); h.W2 = W2; h.b2 = b2; h.W3 = W3; h.b3 = b3; h.t = targets;
        h.pre2 = F(P.pre2); h.y2 = F(P.y2); h.pre3 = F(P.pre3); h.y3 = F(P.y3); h.dy3 = F(P.dy3);
        h.loss = loss_out; h.pred = pred_out;
        h.dy2 = F(P.dy2); h.dW3 = F(P.dW3); h.db3 = F(P.db3);
        h.dy1 = F(P.dy1); h.dW2 = F(P.dW2); h.db2 = F(P.db2);
        h.g1 = F(P.g1); h.db1 = F(P.db1);
        CF_TRY_HIP(launch_dense_head(h, stream), "dense head");
        CF_TRY_HIP(launch_dense_bwd(B, P.flat, P.d0, hX, hXb, W1, F(P.g1), F(P.g1), -1.f,
                                    bf ? nullptr : (float*)(w + last.dp),
                                    bf && !head_unpool ? (uint16_t*)(w + last.dp) : nullptr, F(P.dW1), nullptr, stream,
                                    head_unpool ? &dup : nullptr), "dense1 backward");
    } else {
        CF_TRY_HIP(launch_dense_fwd(B, P.d0, P.d1, F(P.y1), nullptr, W2, b2, slope, F(P.pre2), F(P.y2), part, stream),
                   "dense2");
        CF_TRY_HIP(launch_dense_fwd(B, P.d1, P.d2, F(P.y2), nullptr, W3, b3, -1.f, F(P.pre3), F(P.y3), part, stream),
                   "dense3");
        CF_TRY_HIP(launch_mse(B, P.d2, F(P.y3), targets, loss_out, F(P.dy3), stream), "mse");
        if (pred_out) CF_TRY_HIP(launch_copy_f32(F(P.y3), pred_out, (int64_t)B * P.d2, stream), "copy predictions");
        CF_TRY_HIP(launch_dense_bwd(B, P.d1, P.d2, F(P.y2), nullptr, W3, F(P.pre3), F(P.dy3), -1.f, F(P.dy2), nullptr,
                                    F(P.dW3), F(P.db3), stream), "dense3 backward");
        CF_TRY_HIP(launch_dense_bwd(B, P.d0, P.d1, F(P.y1), nullptr, W2, F(P.pre2), F(P.dy2), slope, F(P.dy1), nullptr,
                                    F(P.dW2), F(P.db2), stream), "dense2 backward");
        CF_TRY_HIP(launch_dense_bwd(B, P.flat, P.d0, hX, hXb, W1, F(P.pre1), F(P.dy1), slope,
                                    bf ? nullptr : (float*)(w + last.dp),
                                    bf && !head_unpool ? (uint16_t*)(w + last.dp) : nullptr, F(P.dW1), F(P.db1), stream,
                                    head_unpool ? &dup : nullptr), "dense1 backward");
    }

    // 5. conv blocks backward: pool backward -> data gradient on the caller's
    //    stream; each block's weight gradient (with its split reduction) on
    //    the auxiliary stream once its conv-output gradient exists, so it
    //    overlaps the rest of the backward chain.
    // 6. SGD.  The fp32 masters are read only by the weight copies, the
    //    forward and the dense backward, all enqueued on the caller's stream
    //    before the first fork, so the masters whose gradients the auxiliary
    //    stream holds (the dense head's, and those of the blocks whose weight
    //    gradient runs there) are updated there in one launch, overlapping the
    //    end of the backward chain; the rest are updated after the join.
    static_assert(CF_MAX_BLOCKS + 6 <= 16, "SgdList capacity");
    SgdList sl_aux{}, sl_main{};
    auto add = [](SgdList& sl, float* wp, const float* g, int64_t n) {
        sl.w[sl.count] = wp;
        sl.dw[sl.count] = g;
        sl.n[sl.count] = n;
        ++sl.count;
    };
    {
        float* part_w = F(P.part_w);
        bool forked = false;
        int deferred = -1;    // a block whose weight gradient waits for the next fork
        // this block's dz was already written by the kernel that produced its
        // pooled gradient (the dense backward for the last block, the next
        // block's backward-data otherwise)
        bool unpooled = head_unpool;
        cf_status bst = CF_OK;
        for (int l = L - 1; l >= 0 && bst == CF_OK; --l) {
            const LayerPlan& Lp = P.layer[l];
            if (Lp.fused) {
                bst = check_hip(launch_wgrad_c4_pool(plan_wgrad(Lp.x, Lp.cout),
                                                     (const uint16_t*)(l == 0 ? X : w + P.layer[l - 1].p),
                                                     (const uint16_t*)(w + Lp.dp), (const uint16_t*)(w + Lp.p),
                                                     (const uint8_t*)(w + Lp.idx), slope, part, F(Lp.dw), Lp.x,
                                                     stream),
                                "fused pool backward + conv3d backward-weight");
                continue;
            }
            const cf_dims z = with_c(Lp.x, Lp.cout);
            void* dz = w + Lp.z;    // the conv output buffer is reused for its gradient
            if (!unpooled) {
                hipError_t e = bf ? launch_pool_bwd<uint16_t>((const uint16_t*)(w + Lp.dp), (const uint16_t*)(w + Lp.p),
                                                              (const uint8_t*)(w + Lp.idx), (uint16_t*)dz, z, slope,
                                                              stream)
                                  : launch_pool_bwd<float>((const float*)(w + Lp.dp), (const float*)(w + Lp.p),
                                                           (const uint8_t*)(w + Lp.idx), (float*)dz, z, slope, stream);
                if ((bst = check_hip(e, "pool backward")) != CF_OK) break;
            }
            unpooled = false;
            // The deepest block's weight gradient is the smallest, and the
            // auxiliary stream has nothing else to do yet: it waits for the
            // next block's fork (block l - 1 >= 1, never fused, so it forks),
            // which saves one fork on the caller's stream.  Its dz and input
            // are not written before the join.
            if (l == L - 1 && l >= 2) {
                deferred = l;
            } else {
                // fork: the weight gradients read dz and the block inputs,
                // which nothing on the caller's stream writes until the join
                if (two) {
                    if ((bst = check_hip(hipEventRecord(aux->fork[l], stream), "fork event")) != CF_OK) break;
                    if ((bst = check_hip(hipStreamWaitEvent(as, aux->fork[l], 0), "fork wait")) != CF_OK) break;
                    forked = true;
                }
                for (const int q : {deferred, l}) {
                    if (q < 0) continue;
                    const LayerPlan& Lq = P.layer[q];
                    const void* xin = q == 0 ? X : (const void*)(w + P.layer[q - 1].p);
                    if ((bst = check_hip(run_wgrad(Lq.wg, dtype, Lq.x, xin, w + Lq.z, Lq.cout, F(Lq.dw), part_w, as),
                                         "conv3d backward-weight")) != CF_OK)
                        break;
                }
                deferred = -1;
                if (bst != CF_OK) break;
            }
            if (l > 0) {
                // A backward-data whose output is a non-fused block's pooled
                // gradient applies that block's pool backward itself (in the
                // reduction of split partials, or in the epilogue of the
                // weight-ring kernel) and writes the block's dz directly; the
                // pooled gradient dp is read by nothing else.
                const LayerPlan& Lm = P.layer[l - 1];
                const cf_dims y = with_c(Lp.x, Lp.cout);
                const bool can = Lp.dg == Fwd::Mfma && conv_mfma_can_unpool(plan_conv_mfma(y, (int)Lp.x.c));
                if (can && bf && !Lm.fused) {
                    bst = check_hip(launch_conv_mfma_unpool(plan_conv_mfma(y, (int)Lp.x.c), (const uint16_t*)dz,
                                                            (const uint16_t*)(w + Lp.wk_dg), part,
                                                            (const uint16_t*)(w + Lm.p), (const uint8_t*)(w + Lm.idx),
                                                            (uint16_t*)(w + Lm.z), slope, y, (int)Lp.x.c,
                                                            roundup((int)Lp.x.c, 128), stream),
                                    "conv3d backward-data + pool backward");
                    unpooled = true;
                } else {
                    bst = check_hip(run_dgrad(Lp.dg, dtype, Lp.x, dz, w + Lp.wk_dg, Lp.cout, w + Lm.dp, part, stream),
                                    "conv3d backward-data");
                }
            }
        }
        SgdList& dense_sl = forked ? sl_aux : sl_main;
        add(dense_sl, params[L], F(P.dW1), (int64_t)P.flat * P.d0);
        add(dense_sl, params[L + 1], F(P.db1), P.d0);
        add(dense_sl, params[L + 2], F(P.dW2), (int64_t)P.d0 * P.d1);
        add(dense_sl, params[L + 3], F(P.db2), P.d1);
        add(dense_sl, params[L + 4], F(P.dW3), (int64_t)P.d1 * P.d2);
        add(dense_sl, params[L + 5], F(P.db3), P.d2);
        for (int l = 0; l < L; ++l)    // a fused block's weight gradient is made on the caller's stream
            add(forked && !P.layer[l].fused ? sl_aux : sl_main, params[l], F(P.layer[l].dw),
                (int64_t)27 * P.layer[l].x.c * P.layer[l].cout);
        if (forked && bst == CF_OK) bst = check_hip(launch_sgd_multi(sl_aux, lr, as), "sgd");
        if (forked) {
            // join even after an error, so no work of this call outlives it on the auxiliary stream
            const cf_status j1 = check_hip(hipEventRecord(aux->join, as), "join event");
            const cf_status j2 = j1 == CF_OK ? check_hip(hipStreamWaitEvent(stream, aux->join, 0), "join wait")
                                             : j1;
            if (bst == CF_OK) bst = j2;
        }
        if (bst != CF_OK) return bst;
    }

    CF_TRY_HIP(launch_sgd_multi(sl_main, lr, stream), "sgd");
    return CF_OK;
}

}  // extern "C"
