/*
 * cf.h -- C ABI of libcf.so: the CosmoFlow-style 3D-CNN training step on one
 * AMD Instinct MI355X (gfx950).
 *
 * The network is a stack of blocks [3^3 convolution, zero "same" padding,
 * stride 1, no bias -> leaky ReLU -> 2^3 max pool, stride 2] followed by three
 * fully connected layers (leaky ReLU on all but the last), a mean-squared
 * error loss and an SGD update.  Sources for each operation are cited at its
 * declaration:
 *   [CF]  Mathuriya et al., "CosmoFlow: Using Deep Learning to Learn the
 *         Universe at Scale" (arXiv 1808.04728), Sec. III-A (network), III-B
 *         (optimizer), III-C (single-node conv / pooling primitives).
 *   [OY]  Oyama et al., "The Case for Strong Scaling in Deep Learning:
 *         Training Large 3D CNNs with Hybrid Parallelism" (arXiv 2007.12856),
 *         Sec. II-A (mini-batch SGD equation), Sec. IV and Table I (extended
 *         network: "same" padding, stride-1 convs, stride-2 pools, no conv
 *         bias, leaky ReLU except the last layer, MSE loss).
 *
 * Conventions common to every entry point
 * ---------------------------------------
 *  - Tensors are packed row-major.  Activations are NDHWC (channels
 *    innermost).  Conv weights are DHWIO: [3][3][3][Cin][Cout].  Dense
 *    weights are [in][out], biases [out].
 *  - Data types: CF_F32 = IEEE fp32; CF_BF16 = bfloat16 stored as 16-bit
 *    words.  Matrix work accumulates in fp32; bf16 outputs are rounded to
 *    nearest even.  Weight gradients, master weights and the dense head are
 *    always fp32.
 *  - Every pointer argument is a DEVICE pointer unless stated otherwise and
 *    must be 16-byte aligned.  The caller owns every buffer, stream and
 *    event; the library allocates no device memory and keeps no host state
 *    between calls other than the thread-local text of cf_last_error() and
 *    the per-device address of cf_conv3d_bwd_weight_noalloc's scratch.
 *  - Every call is asynchronous on `stream` (0 = the null stream) and never
 *    synchronises.  Outputs are overwritten, never accumulated into.
 *  - Arguments are validated before any GPU work is enqueued.  Failures
 *    return a negative cf_status and enqueue nothing; cf_last_error() then
 *    returns a thread-local message.  No call aborts or throws.
 *  - Workspaces are caller-provided device scratch of at least the size the
 *    matching *_workspace_size() call returns (CF_ERR_WORKSPACE otherwise).
 *    Their contents on entry do not matter; they must not alias any other
 *    argument, and concurrent calls must use distinct workspaces.
 */
#ifndef CF_H_
#define CF_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CF_ABI_VERSION 2
#define CF_MAX_BLOCKS 8
#define CF_MAX_OPT_TENSORS 32

typedef enum {
    CF_OK = 0,
    CF_ERR_INVALID = -1,      /* null pointer, non-positive size, misalignment, bad enum */
    CF_ERR_UNSUPPORTED = -2,  /* valid request this build does not implement (e.g. k != 3) */
    CF_ERR_WORKSPACE = -3,    /* ws_bytes smaller than the required workspace */
    CF_ERR_HIP = -4           /* a HIP launch failed; see cf_last_error() */
} cf_status;

typedef enum { CF_F32 = 0, CF_BF16 = 1 } cf_dtype;

/* Packed NDHWC tensor shape. */
typedef struct { int64_t n, d, h, w, c; } cf_dims;

/* Convolution geometry; `pad` is the zero padding below each dimension.
 * This build supports k = 3 with
 *  - stride 1, pad 1: the "same" stride-1 convolution of [OY] Sec. IV;
 *    the output has the input's d, h, w;
 *  - stride 2 with TensorFlow's "same" padding ([OY] Table I: c4 has stride
 *    2, every layer "same" padding): output ceil(d/2) x ceil(h/2) x ceil(w/2)
 *    and total padding (out - 1) * 2 + 3 - size per dimension, the smaller
 *    half below, so pad = 1 when d, h, w are odd and 0 when even (all three
 *    of one parity).  Output voxel o reads input voxels 2o + k - pad,
 *    k = 0, 1, 2.  Only cf_conv3d_fwd, cf_conv3d_bwd_data and
 *    cf_conv3d_bwd_weight take stride 2 (cout a multiple of 4); their
 *    output or upstream-gradient tensors then have the stride-2 output
 *    shape.
 * Anything else returns CF_ERR_UNSUPPORTED. */
typedef struct { int32_t k, stride, pad; } cf_conv;

/* Which pass a conv workspace is sized for. */
typedef enum {
    CF_CONV_FWD = 0,               /* cf_conv3d_fwd */
    CF_CONV_BWD_DATA = 1,          /* cf_conv3d_bwd_data */
    CF_CONV_BWD_WEIGHT = 2,        /* cf_conv3d_bwd_weight */
    CF_CONV_POOL_FWD = 3,          /* cf_conv3d_pool_fwd */
    CF_POOL_CONV_BWD_WEIGHT = 4    /* cf_pool_conv3d_bwd_weight */
} cf_conv_pass;

/* Network description for cf_train_step: `nblocks` blocks with output
 * channels filters[0..nblocks-1] applied to a cin x d x h x w input (each of
 * d, h, w divisible by 2^nblocks), then dense layers of widths dense[0],
 * dense[1], dense[2] (the last has no activation), leaky-ReLU slope
 * `slope` >= 0. */
typedef struct {
    int32_t nblocks;
    int32_t cin;
    int32_t d, h, w;
    int32_t filters[CF_MAX_BLOCKS];
    int32_t dense[3];
    float slope;
} cf_model_desc;

/* ---------------------------------------------------------------- conv3d */

/* Bytes of workspace the given conv pass needs (0 is possible).  `x` is the
 * shape of the forward input X (x.c = Cin); `cout` the forward output
 * channels.  Returns 0 also for invalid arguments (the call then fails). */
size_t cf_conv3d_workspace_size(cf_dtype dtype, cf_dims x, int32_t cout, cf_conv conv,
                                cf_conv_pass pass);

/* Forward 3D convolution ([CF] Sec. III-C; [OY] Sec. IV, Table I):
 *   Y[n,d,h,w,co] = sum_{kd,kh,kw in 0..2} sum_ci X[n,d+kd-1,h+kh-1,w+kw-1,ci]
 *                                                * W[kd,kh,kw,ci,co]
 * with X read as zero outside the volume (stride 1; for stride 2 see
 * cf_conv: Y[n,o,...] reads X[n, 2o + kd - pad, ...] and has the stride-2
 * output shape).
 *   X [x.n, x.d, x.h, x.w, x.c]  (dtype)      input
 *   W [3,3,3, x.c, cout]         (dtype)      weights, DHWIO
 *   Y [x.n, x.d, x.h, x.w, cout] (dtype)      output, overwritten */
cf_status cf_conv3d_fwd(cf_dtype dtype, cf_dims x, const void* X, const void* W, int32_t cout,
                        cf_conv conv, void* Y, void* ws, size_t ws_bytes, hipStream_t stream);

/* Backward-data of the forward convolution ([CF] Sec. III-C, the separate
 * backward-data operator): the adjoint with respect to X,
 *   dX[n,d,h,w,ci] = sum_taps sum_co dY[n,d-kd+1,h-kh+1,w-kw+1,co] * W[kd,kh,kw,ci,co]
 *   dY [x.n, x.d, x.h, x.w, cout] (dtype)     upstream gradient
 *   W  [3,3,3, x.c, cout]         (dtype)     forward weights, DHWIO
 *   dX [x.n, x.d, x.h, x.w, x.c]  (dtype)     output, overwritten */
cf_status cf_conv3d_bwd_data(cf_dtype dtype, cf_dims x, const void* dY, const void* W, int32_t cout,
                             cf_conv conv, void* dX, void* ws, size_t ws_bytes, hipStream_t stream);

/* Backward-weight of the forward convolution ([CF] Sec. III-C, the separate
 * backward-weight operator): the adjoint with respect to W,
 *   dW[kd,kh,kw,ci,co] = sum_{n,d,h,w} X[n,d+kd-1,h+kh-1,w+kw-1,ci] * dY[n,d,h,w,co]
 *   X  [x.n, x.d, x.h, x.w, x.c]  (dtype)     forward input
 *   dY [x.n, x.d, x.h, x.w, cout] (dtype)     upstream gradient
 *   dW [3,3,3, x.c, cout]         (fp32)      output, overwritten
 * The reduction over voxels is split into fixed partial sums that are added
 * in a fixed order: results are bitwise reproducible run to run. */
cf_status cf_conv3d_bwd_weight(cf_dtype dtype, cf_dims x, const void* X, const void* dY, int32_t cout,
                               cf_conv conv, float* dW, void* ws, size_t ws_bytes, hipStream_t stream);

/* Bytes of device scratch behind cf_conv3d_bwd_weight_noalloc (per device). */
#define CF_NOALLOC_SCRATCH_BYTES (64u << 20)

/* cf_conv3d_bwd_weight for callers that cannot allocate device memory or
 * pass a workspace: code under HIP graph capture, allocation-free serving
 * loops, harnesses that forbid hipMalloc.  Same operation, arguments (minus
 * the workspace) and result bit for bit as cf_conv3d_bwd_weight; the split
 * partial sums live in a static device array of CF_NOALLOC_SCRATCH_BYTES
 * that each device holds from the library's load until the process ends.
 * The call allocates nothing.  A shape whose partial sums need more than
 * that returns CF_ERR_WORKSPACE before anything is enqueued.  Every call on a
 * device shares that device's array: calls that may overlap in time on one
 * device (several streams or host threads) race and give wrong results;
 * serialise them.  The first call on a device looks up the array's device
 * address (hipGetSymbolAddress) with that device current. */
cf_status cf_conv3d_bwd_weight_noalloc(cf_dtype dtype, cf_dims x, const void* X, const void* dY, int32_t cout,
                                       cf_conv conv, float* dW, hipStream_t stream);

/* Fused block forward: exactly cf_conv3d_fwd followed by cf_pool3d_fwd on
 * its output (the conv output rounded to dtype first), i.e. one
 * [conv -> leaky ReLU -> 2^3 max pool] block of [CF] Sec. III-A / [OY]
 * Table I, without writing the full-resolution conv output to memory when
 * a fused kernel exists for the shape: bf16 with x.c == 4 and cout % 32 == 0,
 * or bf16 with x.c % 32 == 0 and cout % 32 == 0 where the kernel's plan uses
 * 64- or 128-channel blocks on 4x4x16 tiles and does not split the channel
 * reduction (cf_conv3d_workspace_size(..., CF_CONV_POOL_FWD) then counts no
 * conv output).  Other shapes run the two steps through the workspace.  The
 * result is the same bit for bit either way.
 *   X [x.n, x.d, x.h, x.w, x.c], W [3,3,3,x.c,cout]  (dtype)
 *   P [x.n, x.d/2, x.h/2, x.w/2, cout] (dtype) and idx (uint8, same shape): outputs
 * x.d, x.h, x.w must be even. */
cf_status cf_conv3d_pool_fwd(cf_dtype dtype, cf_dims x, const void* X, const void* W, int32_t cout,
                             cf_conv conv, float slope, void* P, uint8_t* idx, void* ws,
                             size_t ws_bytes, hipStream_t stream);

/* Fused block weight gradient: exactly cf_pool3d_bwd (dP, P, idx -> the conv
 * output gradient dZ, rounded to dtype) followed by cf_conv3d_bwd_weight(X,
 * dZ), without materialising dZ when a fused kernel exists for the shape
 * (bf16, x.c == 4, cout == 32); other shapes run the two steps through the
 * workspace.
 *   X [x.n, x.d, x.h, x.w, x.c] (dtype)
 *   dP, P [x.n, x.d/2, x.h/2, x.w/2, cout] (dtype), idx (uint8, same shape)
 *   dW [3,3,3,x.c,cout] fp32, overwritten */
cf_status cf_pool_conv3d_bwd_weight(cf_dtype dtype, cf_dims x, const void* X, const void* dP,
                                    const void* P, const uint8_t* idx, int32_t cout, cf_conv conv,
                                    float slope, float* dW, void* ws, size_t ws_bytes,
                                    hipStream_t stream);

/* ------------------------------------------------ leaky ReLU + max pooling */

/* Leaky ReLU followed by 2^3 max pooling with stride 2 ([CF] Sec. III-A
 * leaky ReLU on conv layers; 2^3 stride-2 pooling as in [OY] Table I; max
 * rather than average pooling):
 *   P[n,i,j,k,c] = max_{a,b,e in {0,1}} lrelu(Z[n,2i+a,2j+b,2k+e,c])
 *   idx[n,i,j,k,c] = a*4 + b*2 + e of the first strict maximum in (a,b,e)
 *                    lexicographic order
 * lrelu(z) = z if z > 0 else slope*z; slope = 1 gives plain max pooling.
 * slope must be >= 0 (leaky ReLU is then non-decreasing, so the maximum of
 * lrelu over a window is lrelu of the window maximum); a negative or NaN
 * slope returns CF_ERR_INVALID.  The same holds for every entry point below
 * that takes a pooling slope and for cf_model_desc.slope.
 *   Z   [z.n, z.d, z.h, z.w, z.c]         (dtype)  z.d, z.h, z.w even
 *   P   [z.n, z.d/2, z.h/2, z.w/2, z.c]   (dtype)  output
 *   idx same shape as P                   (uint8)  output */
cf_status cf_pool3d_fwd(cf_dtype dtype, cf_dims z, const void* Z, float slope, void* P,
                        uint8_t* idx, hipStream_t stream);

/* Backward of cf_pool3d_fwd: each pooled gradient goes to the window
 * position idx, scaled by the leaky-ReLU derivative there (1 if P > 0, slope
 * otherwise); the other seven positions of every window receive zero.
 *   dP, P [z.n, z.d/2, z.h/2, z.w/2, z.c] (dtype); idx (uint8) same shape
 *   dZ    [z.n, z.d, z.h, z.w, z.c]       (dtype)  output, fully overwritten */
cf_status cf_pool3d_bwd(cf_dtype dtype, cf_dims z, const void* dP, const void* P,
                        const uint8_t* idx, float slope, void* dZ, hipStream_t stream);

/* Leaky ReLU followed by 2^3 average pooling with stride 2 ([CF] Sec. III-A
 * stride-2 average pooling; Sec. III-C: each channel separately, constant
 * weights 1/(KS)^3 = 1/8):
 *   P[n,i,j,k,c] = (1/8) sum_{a,b,e in {0,1}} lrelu(Z[n,2i+a,2j+b,2k+e,c])
 * added in (a,b,e) order in fp32, then scaled; slope = 1 gives plain average
 * pooling (slope >= 0).  z.d, z.h, z.w even; z.c a multiple of 4.
 *   Z [z.n, z.d, z.h, z.w, z.c], P [z.n, z.d/2, z.h/2, z.w/2, z.c] (dtype) */
cf_status cf_avgpool3d_fwd(cf_dtype dtype, cf_dims z, const void* Z, float slope, void* P, hipStream_t stream);

/* Backward of cf_avgpool3d_fwd: every window position receives its window's
 * pooled gradient times 1/8 and the leaky-ReLU derivative at Z (1 if Z > 0,
 * slope otherwise).  dP as P, Z and dZ [z.n, z.d, z.h, z.w, z.c] (dtype). */
cf_status cf_avgpool3d_bwd(cf_dtype dtype, cf_dims z, const void* dP, const void* Z, float slope, void* dZ,
                           hipStream_t stream);

/* Elementwise leaky ReLU ([CF] Sec. III-A).  dy == NULL: out = lrelu(x).
 * Otherwise out = dy * (x > 0 ? 1 : slope) (the backward).  n elements of
 * dtype each. */
cf_status cf_lrelu(cf_dtype dtype, int64_t n, const void* x, const void* dy, float slope,
                   void* out, hipStream_t stream);

/* ------------------------------------------------------------ dense head */

/* Workspace bytes for cf_dense_fwd (partial sums of the split reduction). */
size_t cf_dense_workspace_size(int32_t B, int32_t in, int32_t out);

/* Fully connected layer with bias ([CF] Sec. III-A; [OY] Table I fc layers):
 *   pre[b,o] = sum_i X[b,i] * W[i,o] + bias[o];  Y = lrelu(pre) if slope >= 0
 *   else Y = pre (linear last layer).  All fp32.  bias may be NULL (zero).
 *   X [B,in], W [in,out], bias [out], pre [B,out], Y [B,out].
 * The reduction over `in` is split in fixed 256-row pieces summed in order. */
cf_status cf_dense_fwd(int32_t B, int32_t in, int32_t out, const float* X, const float* W,
                       const float* bias, float slope, float* pre, float* Y, void* ws,
                       size_t ws_bytes, hipStream_t stream);

/* Backward of cf_dense_fwd (chain rule):
 *   dpre = dY * lrelu'(pre)  (dY when slope < 0)
 *   dW[i,o] = sum_b X[b,i] dpre[b,o];  db[o] = sum_b dpre[b,o];
 *   dX[b,i] = sum_o dpre[b,o] W[i,o]   (skipped when dX is NULL). */
cf_status cf_dense_bwd(int32_t B, int32_t in, int32_t out, const float* X, const float* W,
                       const float* pre, const float* dY, float slope, float* dX, float* dW,
                       float* db, hipStream_t stream);

/* Mean squared error ([OY] Sec. IV) and its gradient, fp32:
 *   loss = (1/(B*K)) sum (yhat - t)^2 ;  dyhat = 2 (yhat - t) / (B*K).
 *   yhat, t, dyhat [B,K]; loss: one device float.  dyhat may be NULL. */
cf_status cf_mse(int32_t B, int32_t K, const float* yhat, const float* t, float* loss,
                 float* dyhat, hipStream_t stream);

/* SGD update W <- W - lr * dW on n fp32 values ([OY] Sec. II-A). */
cf_status cf_sgd(int64_t n, float lr, float* W, const float* dW, hipStream_t stream);

/* ------------------------------------------ Adam + LARC + polynomial decay */

/* Optimizer of [CF] Sec. III-B (Adam with LARC and polynomial decay of
 * power 1) and [OY] Sec. IV (Adam, beta1 0.9, beta2 0.999, eps 1e-8, linear
 * decay to 0.01x of the initial rate). */
typedef struct {
    float lr0;            /* initial nominal rate */
    float lr_end;         /* rate reached after decay_steps updates */
    int64_t decay_steps;  /* >= 1 */
    float power;          /* polynomial power, > 0 (1 = linear) */
    float beta1, beta2;   /* in [0, 1) */
    float eps;            /* > 0 */
    float trust;          /* LARC trust coefficient; <= 0 turns LARC off */
} cf_adam_larc_params;

/* Workspace bytes for cf_adam_larc over tensors of these sizes (HOST array). */
size_t cf_adam_larc_workspace_size(int32_t ntensors, const int64_t* n);

/* Update t (1-based) of ntensors fp32 parameter tensors, each one "layer":
 *   rate   lr_t = (lr0 - lr_end) (1 - min(t-1, T)/T)^power + lr_end
 *   Adam   m <- beta1 m + (1-beta1) g;  v <- beta2 v + (1-beta2) g^2
 *          u = (m / (1-beta1^t)) / (sqrt(v / (1-beta2^t)) + eps)
 *   LARC   lr_l = min(lr_t, trust ||w|| / ||g||), or lr_t when trust <= 0
 *          or either norm is 0 (norms over the tensor before the update)
 *          w <- w - lr_l u
 * n, w, g, m, v are HOST arrays of ntensors entries (1..CF_MAX_OPT_TENSORS);
 * w, g, m, v entries are DEVICE pointers to n[i] floats (w, m, v updated in
 * place; m and v start at zero before t = 1).  lr_out: NULL or a device
 * array receiving each tensor's lr_l.  The norms are reduced in a fixed
 * order: results are reproducible bit for bit. */
cf_status cf_adam_larc(const cf_adam_larc_params* hp, int64_t t, int32_t ntensors, const int64_t* n,
                       float* const* w, const float* const* g, float* const* m, float* const* v,
                       float* lr_out, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------ batch norm */

/* Workspace bytes for cf_batchnorm_fwd / cf_batchnorm_bwd on x. */
size_t cf_batchnorm_workspace_size(cf_dtype dtype, cf_dims x);

/* Training-mode batch normalisation ([OY] Sec. IV: after every convolution;
 * Sec. III: the per-channel sum and sum of squares are its statistics) over
 * (n, d, h, w) for each channel c of an NDHWC tensor:
 *   mean = sum x / M, var = sum x^2 / M - mean^2 (biased), M = n*d*h*w
 *   invstd = 1 / sqrt(var + eps);  Y = (X - mean) * gamma * invstd + beta
 *   X, Y [x.n, x.d, x.h, x.w, x.c] (dtype); gamma, beta, mean, invstd [x.c]
 *   fp32 (mean and invstd are outputs, for the backward).
 * x.c must be a multiple of 4 and at most 1024 (else CF_ERR_UNSUPPORTED);
 * eps must be positive and finite (else CF_ERR_INVALID: a constant channel
 * would divide by zero).  Statistics are reduced in a fixed order (fp64
 * across blocks). */
cf_status cf_batchnorm_fwd(cf_dtype dtype, cf_dims x, const void* X, const float* gamma, const float* beta,
                           float eps, void* Y, float* mean, float* invstd, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/* Backward of cf_batchnorm_fwd (chain rule through the batch statistics),
 * with xhat = (X - mean) * invstd from the forward's mean and invstd:
 *   dbeta = sum dY;  dgamma = sum dY xhat
 *   dX = gamma invstd (dY - dbeta / M - xhat dgamma / M) */
cf_status cf_batchnorm_bwd(cf_dtype dtype, cf_dims x, const void* X, const void* dY, const float* gamma,
                           const float* mean, const float* invstd, void* dX, float* dgamma, float* dbeta,
                           void* ws, size_t ws_bytes, hipStream_t stream);

/* --------------------------------------------------------- training step */

/* Caller-owned second stream for cf_train_step.  The blocks' weight
 * gradients read only tensors that the rest of the backward pass leaves
 * alone, so they can run beside it on a second stream; `fork` events order
 * that stream after the caller's stream and `join` orders the caller's
 * stream after it.  All handles belong to the device that was current when
 * they were created and must be used with streams of that device.  One
 * cf_step_aux serves one call at a time: calls that may overlap in time
 * (e.g. from several host threads) need one each, as they need distinct
 * workspaces. */
typedef struct {
    hipStream_t stream;                 /* non-blocking, default priority */
    hipEvent_t fork[CF_MAX_BLOCKS];     /* timing disabled */
    hipEvent_t join;                    /* timing disabled */
} cf_step_aux;

/* Create the stream and events of `aux` (HOST pointer) on the current device.
 * On failure nothing is left allocated and `aux` is zeroed. */
cf_status cf_step_aux_create(cf_step_aux* aux);
/* Destroy what cf_step_aux_create made and zero `aux`; NULL is a no-op.  No
 * call that uses `aux` may still be enqueued on a stream that has not
 * finished it (synchronise first). */
cf_status cf_step_aux_destroy(cf_step_aux* aux);

/* Workspace bytes for cf_train_step with this network, dtype and batch. */
size_t cf_train_step_workspace_size(const cf_model_desc* m, cf_dtype dtype, int32_t B);

/* One full training step ([CF] Sec. III; [OY] Sec. II-A, IV): forward through
 * every block and the dense head, MSE against `targets`, backward, and one
 * SGD update of every parameter with learning rate `lr`.
 *   m        host pointer to the network description
 *   dtype    CF_BF16: conv operands and activations in bf16 (weights are
 *            rounded from the fp32 masters at the start of the step); CF_F32:
 *            fp32 throughout
 *   X        [B, m->d, m->h, m->w, m->cin] (dtype)
 *   targets  [B, m->dense[2]] fp32
 *   params   HOST array of DEVICE pointers to the fp32 master parameters, in
 *            order: conv W_1..W_nblocks (DHWIO), then dense W1, b1, W2, b2,
 *            W3, b3.  Updated in place.
 *   loss_out one device float: the loss of this step (before the update)
 *   pred_out [B, m->dense[2]] fp32 predictions of this step, or NULL
 * Layer-1 backward-data is not computed (the input needs no gradient).
 * aux      HOST pointer to a cf_step_aux, or NULL.  With NULL every kernel
 *          runs on `stream`.  Otherwise the blocks' weight gradients and the
 *          updates of the parameters they feed run on aux->stream, forked from
 *          `stream` with aux->fork[] and joined back with aux->join within the
 *          call, so all of the step's work is still ordered on `stream` as the
 *          caller sees it.  Results are identical bit for bit either way.
 *          aux->stream must not be `stream`. */
cf_status cf_train_step(const cf_model_desc* m, cf_dtype dtype, int32_t B, const void* X,
                        const float* targets, float* const* params, float lr, float* loss_out,
                        float* pred_out, void* ws, size_t ws_bytes, hipStream_t stream,
                        const cf_step_aux* aux);

/* ------------------------------------------------- general network step */

/* What follows each convolution. */
typedef enum {
    CF_POOL_MAX = 0,   /* leaky ReLU, 2^3 max pool (cf_pool3d_fwd) */
    CF_POOL_AVG = 1,   /* leaky ReLU, 2^3 average pool (cf_avgpool3d_fwd) */
    CF_POOL_NONE = 2   /* leaky ReLU only */
} cf_pool_kind;

#define CF_MAX_DENSE 4

/* A network of `nlayers` conv layers (3^3, no bias, stride[l] 1 or 2 with
 * "same" padding) each followed by batch normalisation when batch_norm != 0,
 * leaky ReLU and pool[l]; then flatten (NDHWC order) and ndense fully
 * connected layers of widths dense[0..ndense-1] (with biases when
 * dense_bias != 0; leaky ReLU on all but the last), MSE against the targets.
 * This covers the benchmark network (stride 1, max pool, biases) and the
 * extended CosmoFlow network of [OY] Table I (c4 with stride 2, average
 * pooling as in [CF] Sec. III-A, no pool after c6/c7 at 128^3, fc
 * 2048-256-4 without bias, BN after every conv as in [OY] Sec. IV). */
typedef struct {
    int32_t nlayers;                  /* 1..CF_MAX_BLOCKS */
    int32_t cin, d, h, w;             /* input volume (channels, sizes) */
    int32_t filters[CF_MAX_BLOCKS];
    int32_t stride[CF_MAX_BLOCKS];    /* 1 or 2 */
    int32_t pool[CF_MAX_BLOCKS];      /* cf_pool_kind */
    int32_t batch_norm;               /* != 0: BN after every conv */
    float bn_eps;                     /* > 0 when batch_norm is set */
    int32_t ndense;                   /* 1..CF_MAX_DENSE */
    int32_t dense[CF_MAX_DENSE];
    int32_t dense_bias;               /* != 0: dense layers have biases */
    float slope;                      /* leaky-ReLU slope, >= 0 */
} cf_net_desc;

typedef enum { CF_OPT_SGD = 0, CF_OPT_ADAM_LARC = 1 } cf_opt_kind;

/* The update applied at the end of cf_net_train_step. */
typedef struct {
    int32_t kind;                     /* cf_opt_kind */
    float lr;                         /* SGD: W <- W - lr dW ([OY] Sec. II-A) */
    cf_adam_larc_params adam;         /* CF_OPT_ADAM_LARC, as cf_adam_larc */
    int64_t t;                        /* CF_OPT_ADAM_LARC: update count, >= 1 */
} cf_optimizer;

/* Number of parameter tensors of the network (at most CF_MAX_OPT_TENSORS),
 * or -1 for an invalid description.  If n is not NULL it receives each
 * tensor's element count (HOST array).  Order: for each conv layer its
 * weight [3,3,3,cin,filters] (DHWIO), then gamma [filters] and beta
 * [filters] when batch_norm; then for each dense layer W [in,out] and, when
 * dense_bias, b [out]. */
int32_t cf_net_param_count(const cf_net_desc* net, int64_t* n);

/* Workspace bytes for cf_net_train_step. */
size_t cf_net_train_step_workspace_size(const cf_net_desc* net, cf_dtype dtype, int32_t B);

/* One training step of `net`: forward, MSE against `targets`
 * [B, dense[ndense-1]], backward, and the optimizer's update of every
 * parameter (fp32 masters, `params`: HOST array of DEVICE pointers in
 * cf_net_param_count's order, updated in place).  For CF_OPT_ADAM_LARC, m
 * and v are HOST arrays of DEVICE pointers to the Adam moments in the same
 * order (zero before t = 1); for SGD they are ignored.  CF_BF16 stores every
 * activation and activation gradient in bf16 (conv weights rounded from the
 * masters each step); CF_F32 is fp32 throughout.  The first layer's
 * backward-data is not computed.  Composed of this library's other entry
 * points' kernels, on `stream`. */
cf_status cf_net_train_step(const cf_net_desc* net, cf_dtype dtype, int32_t B, const void* X, const float* targets,
                            float* const* params, const cf_optimizer* opt, float* const* m, float* const* v,
                            float* loss_out, float* pred_out, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- status */

/* Static description of a status code. */
const char* cf_status_string(cf_status s);
/* Detail of the last failure on the calling thread ("" if none). */
const char* cf_last_error(void);
/* CF_ABI_VERSION of the built library. */
int32_t cf_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CF_H_ */
