"""Benchmark: CosmoFlow-style 3D-CNN training step on one MI355X.

Workload (default): batch 8 of 128^3 x 4 synthetic lognormal-Poisson volumes
through 5 blocks [conv 3^3 pad 1 -> leaky ReLU 0.3 -> max-pool 2^3] with
filters 32, 64, 128, 256, 256, dense 16384 -> 128 -> 64 -> 3, MSE, SGD lr
1e-6, bf16 operands with fp32 accumulation and fp32 master weights.  One step
= one cf_train_step call (every kernel of the path: forward, backward,
update).  Inputs are resident in HBM before the timed region; the step time
is the median of the per-step HIP-event times of the timed steps.

Prints one JSON line.  Besides the step rate it times every conv / pool
entry point of the step on its own (HIP events on the launch stream) to give
conv TFLOP/s and a roofline entry per entry point, times the same step on the
fp32 path (matrix-core fp32 kernels) against the fp32 matrix peak, and times
the fp64 CPU oracle on one sample of the same workload as a reported
baseline.  --workload selects one of the other single-GPU workloads instead
(one JSON line each); --mfma-peak measures the matrix cores' sustained rate.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CosmoFlow 128^3x4 train samples/s; conv3d fwd+bwd TFLOP/s & % MFMA peak"
PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 4096 bf16 flop/clk x 2.4 GHz (dense MFMA)
PEAK_F32_TFLOPS = 157.3     # fp32 matrix (MFMA) peak
PEAK_HBM_GBS = 8000.0


WORKLOADS = ("train_bf16_128c4_b8", "train_f32_128c4_b8", "block_bf16_128c4_b4", "partial_bf16_512c4_b1",
             "train_bf16_512c4_b1", "table1_bf16_128_b8")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=WORKLOADS[0], choices=WORKLOADS)
    ap.add_argument("--op-reps", type=int, default=30, help="repetitions per entry point in the per-kernel timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-runs", type=int, default=3, help="oracle runs on one sample (median reported)")
    ap.add_argument("--no-ops", action="store_true", help="skip the per-entry-point timing")
    ap.add_argument("--no-fp32", action="store_true", help="skip the fp32-path step timing")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay timing of the step")
    ap.add_argument("--mfma-peak", action="store_true", help="only measure the matrix cores' sustained rate")
    ap.add_argument("--profile-op", default=None,
                    help="only run the named entry point of the per-entry-point timing --op-reps times "
                         "(for rocprofv3 passes), print nothing")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB --op-reps times (the reference "
                         "kernel that scales the HBM byte counters)")
    return ap.parse_args()


def build_inputs(dev, torch, cf, sd, c):
    st = sd.streams(c.seed_id)
    x = sd.lognormal_poisson_input(st["field"], st["poisson"], (c.batch, c.in_size, c.in_size, c.in_size),
                                   c.in_channels)
    params, cin = [], c.in_channels
    for f in c.filters:
        params.append(torch.from_numpy(sd.he_normal_conv(st["convw"], cin, f)).to(dev))
        cin = f
    fan = (c.in_size >> len(c.filters)) ** 3 * c.filters[-1]
    for o in c.dense:
        W, b = sd.he_normal_dense(st["densew"], fan, o)
        params += [torch.from_numpy(W).to(dev), torch.from_numpy(b).to(dev)]
        fan = o
    t = torch.from_numpy(sd.targets(st["targets"], c.batch)).to(dev)
    xd = torch.from_numpy(x).to(dev).to(torch.bfloat16)
    return xd, t, params


def time_region(torch, fn, reps, stream, warm=3):
    """Average ms of fn() over reps calls after `warm` untimed calls, HIP
    events recorded on `stream`."""
    for _ in range(warm):
        fn()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / reps


def build_ops(torch, cf, c, dev):
    """The step's conv and pool entry points at the workload's shapes (bf16),
    each as a callable with its algorithmic flops and HBM bytes.  Every block
    forward is timed as cf_conv3d_pool_fwd (fused where the step fuses it);
    the first block's pool backward + backward-weight runs fused as in the
    step.  Both fused forms count as conv work.
    Algorithmic bytes: every operand read once and every result written
    once (conv: input, weights, output; backward-weight: input, output
    gradient, fp32 weight gradient; pool: input, output, indices)."""
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    B, S, cin = c.batch, c.in_size, c.in_channels
    ops = []

    def ws_for(X, f, pas):
        return torch.empty(max(1, cf.cf_conv3d_workspace_size(cf.CF_BF16, X.shape, f, pas)), dtype=torch.uint8,
                           device=dev)

    for l, f in enumerate(c.filters):
        # every tensor of this layer is bound as a default argument, so each
        # callable keeps its own layer's tensors alive
        X = torch.randn((B, S, S, S, cin), generator=g, device=dev).to(torch.bfloat16)
        W = (torch.randn((3, 3, 3, cin, f), generator=g, device=dev) * 0.05).to(torch.bfloat16)
        P = torch.randn((B, S // 2, S // 2, S // 2, f), generator=g, device=dev).to(torch.bfloat16)
        idx = torch.randint(0, 8, P.shape, generator=g, device=dev, dtype=torch.uint8)
        dW = torch.empty((3, 3, 3, cin, f), dtype=torch.float32, device=dev)
        nvox = B * S ** 3
        flops = 2 * 27 * cin * f * nvox
        xb, zb, wb = X.numel() * 2, nvox * f * 2, 27 * cin * f * 2
        pb, ib = P.numel() * 2, P.numel()
        if l == 0:
            wsf = ws_for(X, f, cf.CF_CONV_POOL_FWD)
            wsw = ws_for(X, f, cf.CF_POOL_CONV_BWD_WEIGHT)
            Po, ido = torch.empty_like(P), torch.empty_like(idx)
            ops.append(dict(name="block1_conv_pool_fwd", kind="conv", flops=flops, bytes=xb + wb + pb + ib,
                            fn=lambda X=X, W=W, Po=Po, ido=ido, ws=wsf: cf.cf_conv3d_pool_fwd(X, W, 0.3, Po, ido, ws=ws)))
            ops.append(dict(name="block1_pool_bwd_weight", kind="conv", flops=flops,
                            bytes=xb + 2 * pb + ib + 27 * cin * f * 4,
                            fn=lambda X=X, P=P, idx=idx, dW=dW, ws=wsw:
                            cf.cf_pool_conv3d_bwd_weight(X, P, P, idx, 0.3, dW, ws=ws)))
        else:
            dZ = torch.randn((B, S, S, S, f), generator=g, device=dev).to(torch.bfloat16)
            Z, dX = torch.empty_like(dZ), torch.empty_like(X)
            wsf = ws_for(X, f, cf.CF_CONV_POOL_FWD)
            wsd = ws_for(X, f, cf.CF_CONV_BWD_DATA)
            wsw = ws_for(X, f, cf.CF_CONV_BWD_WEIGHT)
            Po, ido = torch.empty_like(P), torch.empty_like(idx)
            # the block forward as the step runs it: conv + leaky ReLU + pool in
            # one launch where the plan allows, else conv then pool
            ops.append(dict(name="block%d_conv_pool_fwd" % (l + 1), kind="conv", flops=flops,
                            bytes=xb + wb + pb + ib,
                            fn=lambda X=X, W=W, Po=Po, ido=ido, ws=wsf: cf.cf_conv3d_pool_fwd(X, W, 0.3, Po, ido, ws=ws)))
            ops.append(dict(name="pool%d_bwd" % (l + 1), kind="pool", flops=0, bytes=pb + pb + ib + zb,
                            fn=lambda P=P, idx=idx, Z=Z: cf.cf_pool3d_bwd(P, P, idx, 0.3, Z)))
            ops.append(dict(name="conv%d_bwd_data" % (l + 1), kind="conv", flops=flops, bytes=zb + wb + xb,
                            fn=lambda dZ=dZ, W=W, dX=dX, ws=wsd: cf.cf_conv3d_bwd_data(dZ, W, dX, ws=ws)))
            ops.append(dict(name="conv%d_bwd_weight" % (l + 1), kind="conv", flops=flops,
                            bytes=xb + zb + 27 * cin * f * 4,
                            fn=lambda X=X, dZ=dZ, dW=dW, ws=wsw: cf.cf_conv3d_bwd_weight(X, dZ, dW, ws=ws)))
        S //= 2
        cin = f
    return ops


def op_timings(torch, cf, c, dev, reps):
    """Average ms per call of every entry point (HIP events on the stream the
    calls are launched on)."""
    stream = torch.cuda.current_stream()
    ops = build_ops(torch, cf, c, dev)
    for o in ops:
        o["ms"] = time_region(torch, o["fn"], reps, stream)
        del o["fn"]
    torch.cuda.empty_cache()
    return ops


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


# a C/C++ comment, or a string or character literal (kept whole, so that a
# comment marker inside a literal is not taken for a comment)
_C_COMMENT_OR_STRING = re.compile(r'//[^\n]*|/\*.*?\*/|"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'', re.S)


def source_digest(paths):
    """sha256 of the code of `paths` (relative to the repository root) with
    comments and blank lines left out: C/C++ comments in the kernel sources,
    whole-line '#' comments in Python files.  String literals are kept.  A
    change of code changes it; a change of comments does not."""
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as fh:
            text = fh.read()
        if rel.endswith(".py"):
            lines = [l for l in text.split("\n") if not l.lstrip().startswith("#")]
        else:
            text = _C_COMMENT_OR_STRING.sub(lambda m: m.group(0) if m.group(0)[0] in "\"'" else " ", text)
            lines = text.split("\n")
        code = "\n".join(l.rstrip() for l in lines if l.strip())
        h.update(rel.encode() + b"\0" + code.encode() + b"\0")
    return h.hexdigest()


def measured_traffic(op_name):
    """HBM bytes per launch of `op_name` from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE passes (scaled by the same counters on a plain
    copy of known size), or None when there are none for this entry point or
    the code of its kernel sources has changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    # {"ops": {name: entry}} (one entry per profiled entry point) or one entry
    entries = t.get("ops") if isinstance(t.get("ops"), dict) else {t.get("op"): t}
    t = entries.get(op_name)
    if not isinstance(t, dict):
        return None
    try:
        digest = source_digest(t.get("sources", []))
    except OSError:
        return None
    if digest != t.get("code_sha256"):
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(c, runs, x1, conv, dense, t1):
    """The fp64 oracle's training step (bf16 storage model) on one 128^3 x 4
    sample of the workload's batch through the same blocks and head, median
    of `runs` runs: samples/s of the oracle on the host's cores."""
    import oracle
    times = []
    for _ in range(runs):
        t0 = time.time()
        oracle.train_step(x1, t1, conv, dense, c.lr, c.slope, storage="bf16")
        times.append(time.time() - t0)
    med = float(np.median(times))
    return {"value": 1.0 / med, "unit": "samples/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "fp64 oracle training step (bf16 storage model) on one 1 x %d^3 x %d sample of the seeded "
                      "batch, same 5 blocks and dense head; median of %d runs (%s s)"
                      % (c.in_size, c.in_channels, runs, ", ".join("%.2f" % v for v in times))}


def timed_steps(torch, step, steps, warmup, stream):
    """Run `warmup` untimed steps, then `steps` steps each bracketed by HIP
    events on `stream`; synchronise on both sides.  Returns (median ms,
    mean ms, per-step ms list, wall seconds)."""
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return float(np.median(per)), ev[0].elapsed_time(ev[steps]) / steps, per, wall


def roofline_of(o):
    """Roofline entry of one timed entry point: MFMA-bound if its algorithmic
    flop/byte ratio reaches the bf16 ridge (2516.6 TFLOP/s / 8 TB/s), else
    HBM-bound; achieved = algorithmic flops (or bytes) per launch / its
    HIP-event average."""
    ai = o["flops"] / o["bytes"] if o["bytes"] else 0.0
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if o["kind"] == "conv" and ai >= ridge:
        ach = o["flops"] / (o["ms"] / 1e3) / 1e12
        return {"kernel": o["name"], "bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(o["name"])}
    ach = o["bytes"] / (o["ms"] / 1e3) / 1e9
    return {"kernel": o["name"], "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": measured_traffic(o["name"])}


TRAFFIC_NOTE = ("traffic: TCC FETCH_SIZE + WRITE_SIZE per launch from rocprofv3 counter passes, scaled by the same "
                "counters on a plain device copy of known size; these count L2-miss bytes, of which reads may be "
                "served by the Infinity Cache rather than HBM")


def mfma_peak(torch, dev):
    """Sustained matrix-core rate: the probe library's independent MFMA
    chains on 4 x 256 blocks per CU, timed with HIP events."""
    import ctypes
    from cnn_cosmology_volumes_amd.build import PROBE_LIB
    if not os.path.exists(PROBE_LIB):
        raise ImportError("libcfprobe.so is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(PROBE_LIB)
    L.cf_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.cf_probe_mfma.restype = ctypes.c_int
    blocks = 256 * 8
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    res = {}
    for kind, name, flop, iters in ((0, "bf16_16x16x32", 16 * 16 * 32 * 2, 4000), (1, "f32_16x16x4", 16 * 16 * 4 * 2, 1000)):
        def run():
            rc = L.cf_probe_mfma(kind, blocks, iters, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError("cf_probe_mfma failed: %d" % rc)
        ms = time_region(torch, run, 5, stream)
        total = blocks * 4 * iters * 8 * flop          # 4 waves per block, 8 chains per round
        res[name] = round(total / (ms / 1e3) / 1e12, 1)
    return res


def step_inputs_f32(dev, torch, sd, c):
    st = sd.streams(c.seed_id)
    x = sd.lognormal_poisson_input(st["field"], st["poisson"], (c.batch, c.in_size, c.in_size, c.in_size),
                                   c.in_channels)
    conv, cin = [], c.in_channels
    for f in c.filters:
        conv.append(sd.he_normal_conv(st["convw"], cin, f))
        cin = f
    fan = (c.in_size >> len(c.filters)) ** 3 * c.filters[-1]
    dense = []
    for o in c.dense:
        dense.append(sd.he_normal_dense(st["densew"], fan, o))
        fan = o
    t = sd.targets(st["targets"], c.batch)
    return x, conv, dense, t


def device_params(torch, dev, conv, dense):
    ps = [torch.from_numpy(w).to(dev) for w in conv]
    for W, b in dense:
        ps += [torch.from_numpy(W).to(dev), torch.from_numpy(b).to(dev)]
    return ps


def train_step_line(a, torch, cf, sd, c, dev, dtype_name, graph=False):
    """Time cf_train_step on the 128^3 (or 512^3) network; returns the dict
    of step timings (samples/s from the median step)."""
    from cnn_cosmology_volumes_amd.configs import train_step_conv_flops
    x, conv, dense, t = step_inputs_f32(dev, torch, sd, c) if c.in_size <= 128 else (None, None, None, None)
    if c.in_size > 128:
        g = sd.torch_generator(5100, dev)
        xd = sd.lognormal_poisson_input_torch(g, (c.batch, c.in_size, c.in_size, c.in_size), c.in_channels, dev)
        st = sd.streams(c.seed_id)
        conv, cin = [], c.in_channels
        for f in c.filters:
            conv.append(sd.he_normal_conv(st["convw"], cin, f))
            cin = f
        fan = (c.in_size >> len(c.filters)) ** 3 * c.filters[-1]
        dense = []
        for o in c.dense:
            dense.append(sd.he_normal_dense(st["densew"], fan, o))
            fan = o
        td = torch.from_numpy(sd.targets(st["targets"], c.batch)).to(dev)
    else:
        xd = torch.from_numpy(x).to(dev).to(torch.bfloat16 if dtype_name == "bf16" else torch.float32)
        td = torch.from_numpy(t).to(dev)
    if dtype_name == "f32" and xd.dtype != torch.float32:
        xd = xd.float()
    params = device_params(torch, dev, conv, dense)
    m = cf.model_desc(c.in_channels, c.in_size, c.filters, c.dense, c.slope)
    dt = cf.CF_BF16 if dtype_name == "bf16" else cf.CF_F32
    ws = torch.empty(cf.cf_train_step_workspace_size(m, dt, c.batch), dtype=torch.uint8, device=dev)
    loss = torch.empty((1,), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    aux = cf.StepAux()
    first = []

    def step():
        cf.cf_train_step(m, xd, td, params, c.lr, ws=ws, loss=loss, aux=aux)
        if not first:
            first.append(float(loss.item()))

    med, mean, per, wall = timed_steps(torch, step, a.steps, a.warmup, stream)
    flops = train_step_conv_flops(c.network(), c.batch)
    res = {"ms_median": med, "ms_mean": mean, "wall_s": wall, "loss_first": first[0], "loss_last": float(loss.item()),
           "conv_flops": flops, "per_step_ms": [round(v, 4) for v in per]}
    if graph:
        # the same step captured once into a HIP graph (one warm-up step on
        # the capture stream first), then timed over as many replays
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cf.cf_train_step(m, xd, td, params, c.lr, ws=ws, loss=loss, aux=aux)
        gmed, gmean, _, _ = timed_steps(torch, g.replay, a.steps, 2, stream)
        res["graph_ms_median"], res["graph_ms_mean"] = gmed, gmean
        del g
    aux.close()
    del ws, params, xd
    torch.cuda.empty_cache()
    return res, (x, conv, dense, t)


def other_workload(a, torch, cf, sd, dev):
    """One of the other single-GPU workloads, one JSON line."""
    from cnn_cosmology_volumes_amd.configs import CONFIGS, oyama_table1_net, train_step_conv_flops
    stream = torch.cuda.current_stream()
    name = a.workload
    out = {"n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "data": "synthetic"}
    if name in ("train_f32_128c4_b8", "train_bf16_512c4_b1"):
        c = CONFIGS["train_bf16_128c4_b8" if name == "train_f32_128c4_b8" else name]
        dt = "f32" if name == "train_f32_128c4_b8" else "bf16"
        r, _ = train_step_line(a, torch, cf, sd, c, dev, dt)
        peak = PEAK_F32_TFLOPS if dt == "f32" else PEAK_BF16_TFLOPS
        tf = r["conv_flops"] / (r["ms_median"] / 1e3) / 1e12
        out.update({"metric": "CosmoFlow %d^3x4 train samples/s (%s)" % (c.in_size, dt),
                    "value": round(c.batch / (r["ms_median"] / 1e3), 3), "unit": "samples/s",
                    "ms_per_step": round(r["ms_median"], 4), "ms_per_step_mean": round(r["ms_mean"], 4), "dtype": dt,
                    "config": {"workload": name, "global_batch": c.batch, "input": "%d^3x4" % c.in_size,
                               "filters": c.filters, "dense": c.dense},
                    "step_conv_tflop": round(r["conv_flops"] / 1e12, 4), "step_conv_tflops": round(tf, 2),
                    "frac_matrix_peak": round(tf / peak, 4), "matrix_peak_tflops": peak,
                    "loss_first": r["loss_first"], "loss_last": r["loss_last"], "wall_s_timed": round(r["wall_s"], 3)})
        return out
    if name == "table1_bf16_128_b8":
        net = oyama_table1_net(128)
        B = 8
        pools = [cf.CF_POOL_AVG if L.pool else cf.CF_POOL_NONE for L in net.convs]
        m = cf.net_desc(4, 128, [L.cout for L in net.convs], [L.stride for L in net.convs], pools,
                        dense=net.dense, dense_bias=False, slope=0.3)
        rng = np.random.default_rng(7)
        x = sd.lognormal_poisson_input(rng, rng, (B, 128, 128, 128), 4)
        xd = torch.from_numpy(x).to(dev).to(torch.bfloat16)
        td = torch.from_numpy(sd.targets(rng, B, 4)).to(dev)
        params = []
        for n_ in cf.cf_net_param_count(m):
            params.append((torch.randn(n_, generator=torch.Generator().manual_seed(n_)) * 0.02).to(dev))
        ws = torch.empty(cf.lib().cf_net_train_step_workspace_size(ctypes_ref(cf, m), cf.CF_BF16, B), dtype=torch.uint8,
                         device=dev)
        loss = torch.empty((1,), dtype=torch.float32, device=dev)
        opt = cf.sgd_optimizer(1e-6)
        med, mean, per, wall = timed_steps(torch, lambda: cf.cf_net_train_step(m, xd, td, params, opt, ws=ws, loss=loss),
                                           a.steps, a.warmup, stream)
        fl = net.conv_fwd_flops()
        flops = (2 * sum(fl) + sum(fl[1:])) * B
        tf = flops / (med / 1e3) / 1e12
        out.update({"metric": "Oyama et al. Table I network, 128^3x4, train samples/s (bf16)",
                    "value": round(B / (med / 1e3), 2), "unit": "samples/s", "ms_per_step": round(med, 4),
                    "ms_per_step_mean": round(mean, 4), "dtype": "bf16",
                    "config": {"workload": name, "global_batch": B, "input": "128^3x4",
                               "layers": "c1..c7 16,32,64,128(stride 2),256,256,256, average pool after c1..c5",
                               "dense": net.dense, "dense_bias": False},
                    "step_conv_tflop": round(flops / 1e12, 4), "step_conv_tflops": round(tf, 2),
                    "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4), "wall_s_timed": round(wall, 3)})
        return out
    # the one-block (4 x 128^3 x 4 -> 32) and two-block (1 x 512^3 x 4) forward + backward workloads
    c = CONFIGS[name]
    B, S = c.batch, c.in_size
    g = sd.torch_generator(4001 if S == 512 else 2001, dev)
    x = sd.lognormal_poisson_input_torch(g, (B, S, S, S), 4, dev)
    ws_list, calls, flops = [], [], 0
    cin, s_, a_in = 4, S, x
    layers = []
    for l, f in enumerate(c.filters):
        W = (torch.randn((3, 3, 3, cin, f), generator=g, device=dev) * np.sqrt(2.0 / (27 * cin))).to(torch.bfloat16)
        pshape = (B, s_ // 2, s_ // 2, s_ // 2, f)
        P = torch.empty(pshape, dtype=torch.bfloat16, device=dev)
        idx = torch.empty(pshape, dtype=torch.uint8, device=dev)
        layers.append(dict(x=a_in, W=W, P=P, idx=idx, cin=cin, f=f, s=s_))
        flops += 2 * 27 * cin * f * B * s_ ** 3 * (3 if (l > 0 or name == "block_bf16_128c4_b4") else 2)
        a_in, cin, s_ = P, f, s_ // 2
    dP = sd.normal_torch(g, layers[-1]["P"].shape, dev)
    bufs = {}

    def ws_for(key, shape, f, pas):
        if key not in bufs:
            bufs[key] = torch.empty(max(1, cf.cf_conv3d_workspace_size(cf.CF_BF16, shape, f, pas)), dtype=torch.uint8,
                                    device=dev)
        return bufs[key]

    for L_ in layers:
        L_["dW"] = torch.empty((3, 3, 3, L_["cin"], L_["f"]), dtype=torch.float32, device=dev)
        if L_["cin"] != 4 or name == "block_bf16_128c4_b4":
            L_["dZ"] = torch.empty(tuple(L_["x"].shape[:4]) + (L_["f"],), dtype=torch.bfloat16, device=dev)
            L_["dX"] = torch.empty_like(L_["x"])

    def step():
        for i, L_ in enumerate(layers):
            cf.cf_conv3d_pool_fwd(L_["x"], L_["W"], 0.3, L_["P"], L_["idx"],
                                  ws=ws_for(("f", i), L_["x"].shape, L_["f"], cf.CF_CONV_POOL_FWD))
        dp = dP
        for i in reversed(range(len(layers))):
            L_ = layers[i]
            if L_["cin"] == 4:
                cf.cf_pool_conv3d_bwd_weight(L_["x"], dp, L_["P"], L_["idx"], 0.3, L_["dW"],
                                             ws=ws_for(("pw", i), L_["x"].shape, L_["f"], cf.CF_POOL_CONV_BWD_WEIGHT))
                if name == "block_bf16_128c4_b4":
                    cf.cf_pool3d_bwd(dp, L_["P"], L_["idx"], 0.3, L_["dZ"])
                    cf.cf_conv3d_bwd_data(L_["dZ"], L_["W"], L_["dX"],
                                          ws=ws_for(("d", i), L_["x"].shape, L_["f"], cf.CF_CONV_BWD_DATA))
            else:
                cf.cf_pool3d_bwd(dp, L_["P"], L_["idx"], 0.3, L_["dZ"])
                cf.cf_conv3d_bwd_weight(L_["x"], L_["dZ"], L_["dW"],
                                        ws=ws_for(("w", i), L_["x"].shape, L_["f"], cf.CF_CONV_BWD_WEIGHT))
                cf.cf_conv3d_bwd_data(L_["dZ"], L_["W"], L_["dX"],
                                      ws=ws_for(("d", i), L_["x"].shape, L_["f"], cf.CF_CONV_BWD_DATA))
                dp = L_["dX"]

    med, mean, per, wall = timed_steps(torch, step, a.steps, a.warmup, stream)
    tf = flops / (med / 1e3) / 1e12
    out.update({"metric": "%s: blocks fwd+bwd samples/s" % name, "value": round(B / (med / 1e3), 3), "unit": "samples/s",
                "ms_per_step": round(med, 4), "ms_per_step_mean": round(mean, 4), "dtype": "bf16",
                "config": {"workload": name, "global_batch": B, "input": "%d^3x4" % S, "filters": c.filters},
                "conv_tflop": round(flops / 1e12, 4), "conv_tflops": round(tf, 2),
                "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4), "wall_s_timed": round(wall, 3)})
    return out


def ctypes_ref(cf, m):
    import ctypes
    return ctypes.byref(m)


def main():
    a = parse()
    if a.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (got --gpus %d)" % a.gpus,
              file=sys.stderr)
        sys.exit(2)
    import torch
    from cnn_cosmology_volumes_amd import cf
    from cnn_cosmology_volumes_amd.configs import CONFIGS
    import synthdata as sd

    c = CONFIGS["train_bf16_128c4_b8"]
    dev = torch.device("cuda:0")
    if a.mfma_peak:
        print(json.dumps({"metric": "sustained MFMA rate (probe)", "unit": "TFLOP/s", **mfma_peak(torch, dev),
                          "spec_bf16": PEAK_BF16_TFLOPS, "spec_f32": PEAK_F32_TFLOPS}), flush=True)
        return
    if a.copy_mib:
        src = torch.ones(a.copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(a.op_reps):
            dst.copy_(src)
        torch.cuda.synchronize()
        return
    if a.profile_op:
        sel = [o for o in build_ops(torch, cf, c, dev) if o["name"] == a.profile_op]
        if not sel:
            print("unknown entry point %r" % a.profile_op, file=sys.stderr)
            sys.exit(2)
        for _ in range(a.op_reps):
            sel[0]["fn"]()
        torch.cuda.synchronize()
        return
    if a.workload != WORKLOADS[0]:
        print(json.dumps(other_workload(a, torch, cf, sd, dev)), flush=True)
        return

    r, host = train_step_line(a, torch, cf, sd, c, dev, "bf16", graph=not a.no_graph)
    ms = r["ms_median"]
    value = c.batch / (ms / 1000.0)
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "samples/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms, 4), "ms_per_step_mean": round(r["ms_mean"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "cosmoflow_train_step_128c4_b8: 5 blocks (32,64,128,256,256) + dense 128-64-3, "
                               "MSE, SGD lr %g" % c.lr, "global_batch": c.batch, "input": "128^3x4",
                   "parallelism": "single GPU"},
        "wall_s_timed": round(r["wall_s"], 3),
        "step_conv_tflop": round(r["conv_flops"] / 1e12, 4),
        "step_tflops_whole_step": round(r["conv_flops"] / (ms / 1e3) / 1e12, 2),
        "loss_first": r["loss_first"],
        "loss_last": r["loss_last"],
    }
    if "graph_ms_median" in r:
        gms = r["graph_ms_median"]
        out["graph_step"] = {"ms": round(gms, 4), "ms_mean": round(r["graph_ms_mean"], 4),
                             "samples_per_s": round(c.batch / (gms / 1e3), 2), "steps": a.steps,
                             "note": "the same step captured once into a HIP graph and replayed; median of the "
                                     "replays (value is the eager call)"}
    if not a.no_ops:
        ops = op_timings(torch, cf, c, dev, a.op_reps)
        conv_ms = sum(o["ms"] for o in ops if o["kind"] == "conv")
        pool_ms = sum(o["ms"] for o in ops if o["kind"] == "pool")
        out["conv_ms_per_step"] = round(conv_ms, 4)
        out["pool_ms_per_step"] = round(pool_ms, 4)
        out["conv_tflops"] = round(r["conv_flops"] / (conv_ms / 1e3) / 1e12, 2)
        out["conv_frac_mfma_peak"] = round(out["conv_tflops"] / PEAK_BF16_TFLOPS, 4)
        out["ops"] = {o["name"]: round(o["ms"], 4) for o in ops}
        dom = max(ops, key=lambda o: o["ms"])
        out["roofline"] = roofline_of(dom)
        out["rooflines"] = {o["name"]: {k: v for k, v in roofline_of(o).items() if k != "kernel"} for o in ops}
        out["traffic_note"] = TRAFFIC_NOTE
    if not a.no_fp32:
        fa = argparse.Namespace(**vars(a))
        fa.steps, fa.warmup = 5, 2
        rf, _ = train_step_line(fa, torch, cf, sd, c, dev, "f32")
        tf = rf["conv_flops"] / (rf["ms_median"] / 1e3) / 1e12
        out["fp32_step"] = {"ms": round(rf["ms_median"], 3), "samples_per_s": round(c.batch / (rf["ms_median"] / 1e3), 2),
                            "conv_tflops": round(tf, 2), "peak": PEAK_F32_TFLOPS, "unit": "TFLOP/s",
                            "frac": round(tf / PEAK_F32_TFLOPS, 4), "steps": fa.steps,
                            "note": "same step, fp32 throughout (fp32 matrix-core conv kernels), median of 5 steps"}
    if not a.no_cpu_baseline:
        x, conv, dense, t = host
        out["cpu_baseline"] = cpu_baseline(c, a.cpu_runs, x[:1], conv, dense, t[:1])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
