// cf_net_train_step: one training step of a general conv network (per
// layer: 3^3 conv of stride 1 or 2, optional batch normalisation, leaky
// ReLU, max / average / no pooling; then a dense head with or without
// biases, MSE, and SGD or Adam + LARC).  It composes the library's entry
// points and launchers in the order the method runs a step ([CF] Sec. III;
// [OY] Sec. II-A and IV): forward layer by layer, dense head, loss,
// backward in reverse, one update.  Everything runs on the caller's stream;
// the intermediate tensors live in the caller's workspace.
//
// bf16 storage points (as the oracle models them): each layer's conv output
// Z, batch-norm output Y, layer output A (pooled or activated), and the
// gradients dA, dY and dZ; conv weights are rounded from the fp32 masters at
// the start of the step.  Weight gradients, BN and dense parameters and the
// dense head are fp32.
#include "cf_internal.h"

namespace cf {
namespace {

size_t up256n(size_t b) { return (b + 255) & ~(size_t)255; }
size_t es_of(cf_dtype dt) { return dt == CF_F32 ? 4 : 2; }
int64_t vox(const cf_dims& d) { return d.n * d.d * d.h * d.w; }

struct NetLayer {
    cf_dims x, z, a;          // input, conv output, layer output
    int f, pool;
    cf_conv geom;
    size_t wb, zb, yb, ab, idx, mean, invstd, da, dw, dgam, dbet;   // workspace offsets
    int pw, pg, pb;           // parameter indices (conv W; gamma, beta or -1)
};

struct NetPlan {
    int L, K, np;
    bool bn, bias;
    NetLayer l[CF_MAX_BLOCKS];
    int din[CF_MAX_DENSE], dout[CF_MAX_DENSE], pwd[CF_MAX_DENSE], pbd[CF_MAX_DENSE];
    size_t pre[CF_MAX_DENSE], y[CF_MAX_DENSE], dx[CF_MAX_DENSE], dwd[CF_MAX_DENSE], dbd[CF_MAX_DENSE];
    size_t dyhat, g1, g2, cws, bws, dws, ows;
    size_t cws_bytes, bws_bytes, dws_bytes, ows_bytes;
    int64_t n[CF_MAX_OPT_TENSORS];
    size_t total;
};

cf_status check_net(const cf_net_desc* m, cf_dtype dt, int32_t B)
{
    if (dt != CF_F32 && dt != CF_BF16) return report(CF_ERR_INVALID, "unknown dtype %d", (int)dt);
    if (!m) return report(CF_ERR_INVALID, "network description is null");
    if (B <= 0) return report(CF_ERR_INVALID, "batch must be positive");
    if (m->nlayers < 1 || m->nlayers > CF_MAX_BLOCKS)
        return report(CF_ERR_INVALID, "nlayers must be 1..%d", CF_MAX_BLOCKS);
    if (m->cin <= 0 || m->d <= 0 || m->h <= 0 || m->w <= 0) return report(CF_ERR_INVALID, "input shape must be positive");
    if (m->ndense < 1 || m->ndense > CF_MAX_DENSE) return report(CF_ERR_INVALID, "ndense must be 1..%d", CF_MAX_DENSE);
    if (!(m->slope >= 0.f)) return report(CF_ERR_INVALID, "slope must be >= 0");
    if (m->batch_norm && !(m->bn_eps > 0.f && m->bn_eps < INFINITY)) return report(CF_ERR_INVALID, "bn_eps must be positive and finite");
    int64_t d = m->d, h = m->h, w = m->w;
    for (int l = 0; l < m->nlayers; ++l) {
        const int f = m->filters[l], s = m->stride[l], p = m->pool[l];
        if (f <= 0 || f > 65536) return report(CF_ERR_INVALID, "filters[%d] out of range", l);
        if (s != 1 && s != 2) return report(CF_ERR_UNSUPPORTED, "stride[%d] must be 1 or 2", l);
        if (p < CF_POOL_MAX || p > CF_POOL_NONE) return report(CF_ERR_INVALID, "pool[%d] is not a cf_pool_kind", l);
        if (s == 2) {
            if ((d & 1) != (h & 1) || (d & 1) != (w & 1))
                return report(CF_ERR_UNSUPPORTED, "layer %d: stride 2 needs d, h, w of one parity", l);
            if (f % 4) return report(CF_ERR_UNSUPPORTED, "layer %d: stride 2 needs filters %% 4 == 0", l);
            d = (d + 1) / 2; h = (h + 1) / 2; w = (w + 1) / 2;
        }
        if (m->batch_norm && (f % 4 || f > 1024))
            return report(CF_ERR_UNSUPPORTED, "layer %d: batch norm needs filters %% 4 == 0 and <= 1024", l);
        if (p == CF_POOL_AVG && f % 4) return report(CF_ERR_UNSUPPORTED, "layer %d: average pool needs filters %% 4 == 0", l);
        if (p != CF_POOL_NONE) {
            if ((d & 1) || (h & 1) || (w & 1))
                return report(CF_ERR_UNSUPPORTED, "layer %d: pooling needs even conv output sizes", l);
            d /= 2; h /= 2; w /= 2;
        }
    }
    for (int k = 0; k < m->ndense; ++k)
        if (m->dense[k] <= 0 || m->dense[k] > 65536) return report(CF_ERR_INVALID, "dense[%d] out of range", k);
    const int np = m->nlayers * (m->batch_norm ? 3 : 1) + m->ndense * (m->dense_bias ? 2 : 1);
    if (np > CF_MAX_OPT_TENSORS) return report(CF_ERR_UNSUPPORTED, "%d parameter tensors, at most %d", np, CF_MAX_OPT_TENSORS);
    const double el = (double)B * m->d * m->h * m->w * (double)m->cin;
    if (el > (double)((int64_t)1 << 40)) return report(CF_ERR_INVALID, "input too large");
    const int64_t flat = d * h * w * m->filters[m->nlayers - 1];
    if (flat > ((int64_t)1 << 31) / 4) return report(CF_ERR_INVALID, "flattened features too many");
    return CF_OK;
}

NetPlan plan_net(const cf_net_desc* m, cf_dtype dt, int32_t B)
{
    NetPlan P{};
    P.L = m->nlayers;
    P.K = m->ndense;
    P.bn = m->batch_norm != 0;
    P.bias = m->dense_bias != 0;
    const size_t es = es_of(dt);
    size_t off = 0;
    auto take = [&](size_t bytes) { const size_t o = off; off += up256n(bytes); return o; };
    cf_dims x{B, m->d, m->h, m->w, m->cin};
    int pi = 0;
    size_t gmax = 0;
    for (int i = 0; i < P.L; ++i) {
        NetLayer& L = P.l[i];
        L.f = m->filters[i];
        L.pool = m->pool[i];
        L.x = x;
        L.geom = m->stride[i] == 1 ? cf_conv{3, 1, 1} : cf_conv{3, 2, (int32_t)(x.d & 1)};
        L.z = m->stride[i] == 1 ? cf_dims{B, x.d, x.h, x.w, L.f}
                                : cf_dims{B, (x.d + 1) / 2, (x.h + 1) / 2, (x.w + 1) / 2, L.f};
        L.a = L.pool == CF_POOL_NONE ? L.z : cf_dims{B, L.z.d / 2, L.z.h / 2, L.z.w / 2, L.f};
        const size_t zbytes = (size_t)vox(L.z) * L.f * es;
        L.wb = take(dt == CF_BF16 ? (size_t)27 * x.c * L.f * 2 : 0);
        L.zb = take(zbytes);
        L.yb = take(P.bn ? zbytes : 0);
        L.ab = take((size_t)vox(L.a) * L.f * es);
        L.idx = take(L.pool == CF_POOL_MAX ? (size_t)vox(L.a) * L.f : 0);
        L.mean = take(P.bn ? (size_t)L.f * 4 : 0);
        L.invstd = take(P.bn ? (size_t)L.f * 4 : 0);
        L.da = take((size_t)vox(L.a) * L.f * es);
        L.dw = take((size_t)27 * x.c * L.f * 4);
        L.dgam = take(P.bn ? (size_t)L.f * 4 : 0);
        L.dbet = take(P.bn ? (size_t)L.f * 4 : 0);
        L.pw = pi++;
        P.n[L.pw] = (int64_t)27 * x.c * L.f;
        L.pg = L.pb = -1;
        if (P.bn) {
            L.pg = pi++;
            L.pb = pi++;
            P.n[L.pg] = P.n[L.pb] = L.f;
        }
        if (zbytes > gmax) gmax = zbytes;
        size_t c = cf_conv3d_workspace_size(dt, x, L.f, L.geom, CF_CONV_FWD);
        if (cf_conv3d_workspace_size(dt, x, L.f, L.geom, CF_CONV_BWD_WEIGHT) > c)
            c = cf_conv3d_workspace_size(dt, x, L.f, L.geom, CF_CONV_BWD_WEIGHT);
        if (i > 0 && cf_conv3d_workspace_size(dt, x, L.f, L.geom, CF_CONV_BWD_DATA) > c)
            c = cf_conv3d_workspace_size(dt, x, L.f, L.geom, CF_CONV_BWD_DATA);
        if (c > P.cws_bytes) P.cws_bytes = c;
        if (P.bn && bn_ws_bytes(L.z) > P.bws_bytes) P.bws_bytes = bn_ws_bytes(L.z);
        x = L.a;
    }
    int fan = (int)(vox(x) / B * x.c);
    for (int k = 0; k < P.K; ++k) {
        P.din[k] = fan;
        P.dout[k] = m->dense[k];
        P.pre[k] = take((size_t)B * P.dout[k] * 4);
        P.y[k] = take((size_t)B * P.dout[k] * 4);
        P.dx[k] = take(k > 0 ? (size_t)B * P.din[k] * 4 : 0);
        P.dwd[k] = take((size_t)P.din[k] * P.dout[k] * 4);
        P.dbd[k] = take((size_t)P.dout[k] * 4);
        P.pwd[k] = pi++;
        P.n[P.pwd[k]] = (int64_t)P.din[k] * P.dout[k];
        P.pbd[k] = -1;
        if (P.bias) {
            P.pbd[k] = pi++;
            P.n[P.pbd[k]] = P.dout[k];
        }
        const size_t d = dense_fwd_part_bytes(B, P.din[k], P.dout[k]);
        if (d > P.dws_bytes) P.dws_bytes = d;
        fan = P.dout[k];
    }
    P.np = pi;
    P.dyhat = take((size_t)B * P.dout[P.K - 1] * 4);
    P.g1 = take(gmax);
    P.g2 = take(P.bn ? gmax : 0);
    P.cws = take(P.cws_bytes);
    P.bws = take(P.bws_bytes);
    P.dws = take(P.dws_bytes);
    OptList ol{};
    ol.count = P.np;
    for (int i = 0; i < P.np; ++i) ol.n[i] = P.n[i];
    P.ows_bytes = adam_larc_part_bytes(ol);
    P.ows = take(P.ows_bytes);
    P.total = off;
    return P;
}

__global__ void cast_f32_bf16_kernel(const float* __restrict__ s, uint16_t* __restrict__ d, int64_t n)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) d[i] = f2bf(s[i]);
}

#define NET_TRY(expr)                        \
    do {                                     \
        const cf_status st_ = (expr);        \
        if (st_ != CF_OK) return st_;        \
    } while (0)
#define NET_HIP(expr, what)                                                                   \
    do {                                                                                      \
        const hipError_t e_ = (expr);                                                         \
        if (e_ != hipSuccess) return report(CF_ERR_HIP, "%s: %s", what, hipGetErrorString(e_)); \
    } while (0)

}  // namespace
}  // namespace cf

using namespace cf;

extern "C" {

int32_t cf_net_param_count(const cf_net_desc* net, int64_t* n)
{
    if (check_net(net, CF_F32, 1) != CF_OK) return -1;
    const NetPlan P = plan_net(net, CF_F32, 1);
    if (n)
        for (int i = 0; i < P.np; ++i) n[i] = P.n[i];
    return P.np;
}

size_t cf_net_train_step_workspace_size(const cf_net_desc* net, cf_dtype dtype, int32_t B)
{
    if (check_net(net, dtype, B) != CF_OK) return 0;
    return plan_net(net, dtype, B).total;
}

cf_status cf_net_train_step(const cf_net_desc* net, cf_dtype dtype, int32_t B, const void* X, const float* targets,
                            float* const* params, const cf_optimizer* opt, float* const* m, float* const* v,
                            float* loss_out, float* pred_out, void* ws, size_t ws_bytes, hipStream_t stream)
{
    NET_TRY(check_net(net, dtype, B));
    if (!X || !targets || !params || !opt || !loss_out)
        return report(CF_ERR_INVALID, "cf_net_train_step: null pointer");
    if (opt->kind != CF_OPT_SGD && opt->kind != CF_OPT_ADAM_LARC)
        return report(CF_ERR_INVALID, "cf_net_train_step: unknown optimizer kind %d", opt->kind);
    if (opt->kind == CF_OPT_ADAM_LARC) {
        NET_TRY(check_adam(&opt->adam, opt->t, "cf_net_train_step"));
        if (!m || !v) return report(CF_ERR_INVALID, "cf_net_train_step: Adam needs moment arrays m and v");
    }
    const NetPlan P = plan_net(net, dtype, B);
    for (int i = 0; i < P.np; ++i) {
        if (!params[i] || ((uintptr_t)params[i] & 15u))
            return report(CF_ERR_INVALID, "cf_net_train_step: params[%d] null or misaligned", i);
        if (opt->kind == CF_OPT_ADAM_LARC && (!m[i] || !v[i] || (((uintptr_t)m[i] | (uintptr_t)v[i]) & 15u)))
            return report(CF_ERR_INVALID, "cf_net_train_step: moment %d null or misaligned", i);
    }
    if (((uintptr_t)X & 15u) || ((uintptr_t)targets & 15u) || ((uintptr_t)loss_out & 3u))
        return report(CF_ERR_INVALID, "cf_net_train_step: X / targets must be 16-byte aligned");
    if (ws_bytes < P.total) return report(CF_ERR_WORKSPACE, "cf_net_train_step: workspace %zu < %zu bytes", ws_bytes, P.total);
    if (!ws || ((uintptr_t)ws & 255u)) return report(CF_ERR_INVALID, "cf_net_train_step: workspace null or not 256-byte aligned");

    char* w = (char*)ws;
    auto F = [&](size_t o) { return (float*)(w + o); };
    const bool bf = dtype == CF_BF16;
    const float slope = net->slope;
    hipStream_t s = stream;

    // forward through the conv layers
    const void* ain = X;
    for (int i = 0; i < P.L; ++i) {
        const NetLayer& L = P.l[i];
        const void* Wc = params[L.pw];
        if (bf) {
            const int64_t n = P.n[L.pw];
            hipLaunchKernelGGL(cast_f32_bf16_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, params[L.pw],
                               (uint16_t*)(w + L.wb), n);
            NET_HIP(hipGetLastError(), "weight cast");
            Wc = w + L.wb;
        }
        NET_TRY(cf_conv3d_fwd(dtype, L.x, ain, Wc, L.f, L.geom, w + L.zb, w + P.cws, P.cws_bytes, s));
        const void* yp = w + L.zb;
        if (P.bn) {
            NET_TRY(cf_batchnorm_fwd(dtype, L.z, w + L.zb, params[L.pg], params[L.pb], net->bn_eps, w + L.yb,
                                     F(L.mean), F(L.invstd), w + P.bws, P.bws_bytes, s));
            yp = w + L.yb;
        }
        hipError_t e = hipSuccess;
        if (L.pool == CF_POOL_MAX)
            e = bf ? launch_pool_fwd<uint16_t>((const uint16_t*)yp, (uint16_t*)(w + L.ab), (uint8_t*)(w + L.idx), L.z,
                                               slope, s)
                   : launch_pool_fwd<float>((const float*)yp, (float*)(w + L.ab), (uint8_t*)(w + L.idx), L.z, slope, s);
        else if (L.pool == CF_POOL_AVG)
            e = bf ? launch_avgpool_fwd<uint16_t>((const uint16_t*)yp, (uint16_t*)(w + L.ab), L.z, slope, s)
                   : launch_avgpool_fwd<float>((const float*)yp, (float*)(w + L.ab), L.z, slope, s);
        else
            e = bf ? launch_lrelu<uint16_t>((const uint16_t*)yp, nullptr, (uint16_t*)(w + L.ab), vox(L.z) * L.f, slope, s)
                   : launch_lrelu<float>((const float*)yp, nullptr, (float*)(w + L.ab), vox(L.z) * L.f, slope, s);
        NET_HIP(e, "pool / activation forward");
        ain = w + L.ab;
    }

    // dense head, loss
    const NetLayer& last = P.l[P.L - 1];
    const float* h32 = bf ? nullptr : (const float*)(w + last.ab);
    const uint16_t* h16 = bf ? (const uint16_t*)(w + last.ab) : nullptr;
    for (int k = 0; k < P.K; ++k) {
        const float sk = k + 1 < P.K ? slope : -1.f;
        const float* xin = k == 0 ? h32 : F(P.y[k - 1]);
        const uint16_t* xin16 = k == 0 ? h16 : nullptr;
        NET_HIP(launch_dense_fwd(B, P.din[k], P.dout[k], xin, xin16, params[P.pwd[k]],
                                 P.bias ? params[P.pbd[k]] : nullptr, sk, F(P.pre[k]), F(P.y[k]), F(P.dws), s),
                "dense forward");
    }
    const int KO = P.dout[P.K - 1];
    NET_HIP(launch_mse(B, KO, F(P.y[P.K - 1]), targets, loss_out, F(P.dyhat), s), "mse");
    if (pred_out) NET_HIP(launch_copy_f32(F(P.y[P.K - 1]), pred_out, (int64_t)B * KO, s), "copy predictions");

    // dense backward; the first layer's input gradient is the last conv layer's dA
    const float* g = F(P.dyhat);
    for (int k = P.K - 1; k >= 0; --k) {
        const float sk = k + 1 < P.K ? slope : -1.f;
        const float* xin = k == 0 ? h32 : F(P.y[k - 1]);
        const uint16_t* xin16 = k == 0 ? h16 : nullptr;
        float* dx32 = k > 0 ? F(P.dx[k]) : (bf ? nullptr : F(last.da));
        uint16_t* dx16 = k == 0 && bf ? (uint16_t*)(w + last.da) : nullptr;
        NET_HIP(launch_dense_bwd(B, P.din[k], P.dout[k], xin, xin16, params[P.pwd[k]], F(P.pre[k]), g, sk, dx32, dx16,
                                 F(P.dwd[k]), F(P.dbd[k]), s),
                "dense backward");
        g = F(P.dx[k]);
    }

    // conv layers backward
    for (int i = P.L - 1; i >= 0; --i) {
        const NetLayer& L = P.l[i];
        const void* yp = P.bn ? (const void*)(w + L.yb) : (const void*)(w + L.zb);
        void* dy = w + P.g1;
        const int64_t nz = vox(L.z) * L.f;
        hipError_t e = hipSuccess;
        if (L.pool == CF_POOL_MAX)
            e = bf ? launch_pool_bwd<uint16_t>((const uint16_t*)(w + L.da), (const uint16_t*)(w + L.ab),
                                               (const uint8_t*)(w + L.idx), (uint16_t*)dy, L.z, slope, s)
                   : launch_pool_bwd<float>((const float*)(w + L.da), (const float*)(w + L.ab),
                                            (const uint8_t*)(w + L.idx), (float*)dy, L.z, slope, s);
        else if (L.pool == CF_POOL_AVG)
            e = bf ? launch_avgpool_bwd<uint16_t>((const uint16_t*)(w + L.da), (const uint16_t*)yp, (uint16_t*)dy, L.z,
                                                  slope, s)
                   : launch_avgpool_bwd<float>((const float*)(w + L.da), (const float*)yp, (float*)dy, L.z, slope, s);
        else
            e = bf ? launch_lrelu<uint16_t>((const uint16_t*)yp, (const uint16_t*)(w + L.da), (uint16_t*)dy, nz, slope, s)
                   : launch_lrelu<float>((const float*)yp, (const float*)(w + L.da), (float*)dy, nz, slope, s);
        NET_HIP(e, "pool / activation backward");
        void* dz = dy;
        if (P.bn) {
            dz = w + P.g2;
            NET_TRY(cf_batchnorm_bwd(dtype, L.z, w + L.zb, dy, params[L.pg], F(L.mean), F(L.invstd), dz, F(L.dgam),
                                     F(L.dbet), w + P.bws, P.bws_bytes, s));
        }
        const void* xin = i == 0 ? X : (const void*)(w + P.l[i - 1].ab);
        NET_TRY(cf_conv3d_bwd_weight(dtype, L.x, xin, dz, L.f, L.geom, F(L.dw), w + P.cws, P.cws_bytes, s));
        if (i > 0) {
            const void* Wc = bf ? (const void*)(w + L.wb) : (const void*)params[L.pw];
            NET_TRY(cf_conv3d_bwd_data(dtype, L.x, dz, Wc, L.f, L.geom, w + P.l[i - 1].da, w + P.cws, P.cws_bytes, s));
        }
    }

    // the update, parameters in cf_net_param_count's order
    const float* grads[CF_MAX_OPT_TENSORS];
    for (int i = 0; i < P.L; ++i) {
        grads[P.l[i].pw] = F(P.l[i].dw);
        if (P.bn) {
            grads[P.l[i].pg] = F(P.l[i].dgam);
            grads[P.l[i].pb] = F(P.l[i].dbet);
        }
    }
    for (int k = 0; k < P.K; ++k) {
        grads[P.pwd[k]] = F(P.dwd[k]);
        if (P.bias) grads[P.pbd[k]] = F(P.dbd[k]);
    }
    if (opt->kind == CF_OPT_SGD) {
        for (int i0 = 0; i0 < P.np; i0 += 16) {
            SgdList sl{};
            for (int i = i0; i < P.np && i < i0 + 16; ++i) {
                sl.w[sl.count] = params[i];
                sl.dw[sl.count] = grads[i];
                sl.n[sl.count] = P.n[i];
                ++sl.count;
            }
            NET_HIP(launch_sgd_multi(sl, opt->lr, s), "sgd");
        }
    } else {
        OptList ol{};
        ol.count = P.np;
        for (int i = 0; i < P.np; ++i) {
            ol.w[i] = params[i];
            ol.g[i] = grads[i];
            ol.m[i] = m[i];
            ol.v[i] = v[i];
            ol.n[i] = P.n[i];
        }
        NET_HIP(launch_adam_larc(ol, adam_args(&opt->adam, opt->t), F(P.ows), nullptr, s), "adam + larc");
    }
    return CF_OK;
}

}  // extern "C"
