"""Benchmark: CosmoFlow-style 3D-CNN training step on one MI355X.

Workload: batch 8 of 128^3 x 4 synthetic lognormal-Poisson volumes through
5 blocks [conv 3^3 pad 1 -> leaky ReLU 0.3 -> max-pool 2^3] with filters
32, 64, 128, 256, 256, dense 16384 -> 128 -> 64 -> 3, MSE, SGD lr 1e-6, bf16
operands with fp32 accumulation and fp32 master weights.  One step = one
cf_train_step call (every kernel of the path: forward, backward, update).
Inputs are resident in HBM before the timed region.

Prints one JSON line.  Besides the step rate it times every conv / pool
entry point of the step on its own (HIP events on the launch stream) to give
conv TFLOP/s and the roofline of the dominant kernel, and times the fp64 CPU
oracle on a bounded sample of the same workload as a reported baseline.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CosmoFlow 128^3x4 train samples/s; conv3d fwd+bwd TFLOP/s & % MFMA peak"
PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 4096 bf16 flop/clk x 2.4 GHz (dense MFMA)
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--op-reps", type=int, default=30, help="repetitions per entry point in the per-kernel timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-ops", action="store_true", help="skip the per-entry-point timing")
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


def measured_traffic(op_name):
    """HBM bytes per launch of `op_name` from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE passes (scaled by the same counters on a plain
    copy of known size), or None when there are none for this entry point or
    its kernel source has changed since they were taken."""
    import hashlib
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
    h = hashlib.sha256()
    for rel in t.get("sources", []):
        try:
            with open(os.path.join(ROOT, rel), "rb") as fh:
                h.update(fh.read())
        except OSError:
            return None
    if h.hexdigest() != t.get("sources_sha256"):
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(c, seconds):
    """The fp64 oracle's training step on one 64^3 x 4 sample through the
    same blocks (1/8 of a 128^3 sample's voxels, hence of its conv work),
    repeated for about `seconds`; scaled to 128^3-sample equivalents/s."""
    import oracle
    import synthdata as sd
    st = sd.streams(c.seed_id)
    s = c.in_size // 2
    x = sd.lognormal_poisson_input(st["field"], st["poisson"], (1, s, s, s), c.in_channels)
    conv, cin = [], c.in_channels
    for f in c.filters:
        conv.append(sd.he_normal_conv(st["convw"], cin, f))
        cin = f
    dense, fan = [], (s >> len(c.filters)) ** 3 * c.filters[-1]
    for o in c.dense:
        dense.append(sd.he_normal_dense(st["densew"], fan, o))
        fan = o
    t = sd.targets(st["targets"], 1)
    runs, t0 = 0, time.time()
    while True:
        oracle.train_step(x, t, conv, dense, c.lr, c.slope, storage="bf16")
        runs += 1
        if time.time() - t0 >= seconds:
            break
    dt = (time.time() - t0) / runs
    frac = (s / c.in_size) ** 3
    return {"value": frac / dt, "unit": "samples/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "fp64 oracle training step (bf16 storage model) on 1 x %d^3 x %d, same 5 blocks and dense "
                      "head; %d run(s), %.2f s each; scaled by the voxel ratio %.4f to 128^3-sample equivalents"
                      % (s, c.in_channels, runs, dt, frac)}


def main():
    a = parse()
    if a.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (got --gpus %d)" % a.gpus,
              file=sys.stderr)
        sys.exit(2)
    import torch
    from cnn_cosmology_volumes_amd import cf
    from cnn_cosmology_volumes_amd.configs import CONFIGS, train_step_conv_flops
    import synthdata as sd

    c = CONFIGS["train_bf16_128c4_b8"]
    dev = torch.device("cuda:0")
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
    net = c.network()
    conv_flops = train_step_conv_flops(net, c.batch)
    xd, t, params = build_inputs(dev, torch, cf, sd, c)
    m = cf.model_desc(c.in_channels, c.in_size, c.filters, c.dense, c.slope)
    ws = torch.empty(cf.cf_train_step_workspace_size(m, cf.CF_BF16, c.batch), dtype=torch.uint8, device=dev)
    loss = torch.empty((1,), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    aux = cf.StepAux()

    def step():
        cf.cf_train_step(m, xd, t, params, c.lr, ws=ws, loss=loss, aux=aux)

    loss_first = None
    for _ in range(a.warmup):
        step()
        if loss_first is None:
            loss_first = float(loss.item())
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(a.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / a.steps
    value = c.batch / (ms / 1000.0)
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "samples/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "cosmoflow_train_step_128c4_b8: 5 blocks (32,64,128,256,256) + dense 128-64-3, "
                               "MSE, SGD lr %g" % c.lr, "global_batch": c.batch, "input": "128^3x4",
                   "parallelism": "single GPU"},
        "wall_s_timed": round(wall, 3),
        "step_conv_tflop": round(conv_flops / 1e12, 4),
        "step_tflops_whole_step": round(conv_flops / (ms / 1e3) / 1e12, 2),
        "loss_first": loss_first,
        "loss_last": float(loss.item()),
    }
    if not a.no_ops:
        ops = op_timings(torch, cf, c, dev, a.op_reps)
        conv_ms = sum(o["ms"] for o in ops if o["kind"] == "conv")
        pool_ms = sum(o["ms"] for o in ops if o["kind"] == "pool")
        out["conv_ms_per_step"] = round(conv_ms, 4)
        out["pool_ms_per_step"] = round(pool_ms, 4)
        out["conv_tflops"] = round(conv_flops / (conv_ms / 1e3) / 1e12, 2)
        out["conv_frac_mfma_peak"] = round(out["conv_tflops"] / PEAK_BF16_TFLOPS, 4)
        out["ops"] = {o["name"]: round(o["ms"], 4) for o in ops}
        dom = max(ops, key=lambda o: o["ms"])
        ai = dom["flops"] / dom["bytes"] if dom["bytes"] else 0.0
        ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
        if dom["kind"] == "conv" and ai >= ridge:
            ach = dom["flops"] / (dom["ms"] / 1e3) / 1e12
            out["roofline"] = {"kernel": dom["name"], "bound": "mfma", "achieved": round(ach, 2),
                               "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                               "traffic": measured_traffic(dom["name"])}
        else:
            ach = dom["bytes"] / (dom["ms"] / 1e3) / 1e9
            out["roofline"] = {"kernel": dom["name"], "bound": "hbm", "achieved": round(ach, 1),
                               "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                               "traffic": measured_traffic(dom["name"])}
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(c, a.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
