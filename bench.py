"""Benchmark of the routed bit-sliced linear on one MI355X.

Prints one JSON line.  A step is one pass of the per-batch hot path on the decode
workload (Qwen2.5-7B-like up-projection, W 18944 x 3584 bf16 with 0.5% outlier columns,
G = 128, 3 slices, a batch of 16 bf16 tokens): router logits + argmax + stable regroup
and the routed decode linear, in one call (mbq_route_linear with the plan's choices: at 16
tokens two launches, the first preparing the fp8 operands and the partial router logits
once, the second routing and streaming the weights on the fp8 x fp4 matrix instruction).
Packing is an offline, once-per-weight step and is timed separately (under "extra").

value = tokens / s over the timed steps (inputs resident in HBM), replayed from HIP graphs
(one graph holding a step per weight copy, so neither the host's per-call overhead nor a
per-replay submission gaps the kernels; the same steps launched one by one are reported as
eager_ms_per_step, and the step's other forms beside it: one launch on either multiply, and
the two calls mbq_route then mbq_linear).  The roofline object is for the dominant kernel
(the streaming linear): algorithmic bytes per launch (the slices the batch needs, the
prepared operands or the activations, y, and the routing inputs and outputs) over its
average duration, from HIP events on the launch stream around graph replays of that kernel
alone (mbq_route_linear_prepared on prepared operands, one launch per step); the committed
rocprofv3 trace of the same command gives the kernel's own duration.  The packed weight is
rotated over enough copies (> 512 MiB) that neither L2 nor the 256 MiB Infinity Cache can
serve a repeat.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed bit-sliced linear: tokens/s + effective weight GB/s (decode), TFLOP/s (prefill)"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
ROTATE_BYTES = 512 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--tokens", type=int, default=16, help="decode batch (1, 4 or 16)")
    ap.add_argument("--no-extra", action="store_true", help="skip the secondary measurements")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", choices=["decode", "prefill", "sweep", "layer", "traffic", "route_mlp", "lowrank", "bitplane"], default=None,
                    help="run one workload only (for profiling); prints its own JSON line.  "
                         "'traffic' runs a copy kernel of known size and then the decode linear, "
                         "for the FETCH_SIZE / WRITE_SIZE counter passes")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


WARM_PREFILL = 200   # untimed prefill launches before a prefill timing (~50 ms at 2048 tokens)


def copies_for(nbytes: int) -> int:
    return max(2, math.ceil(ROTATE_BYTES / nbytes))


def make_blobs(api, torch, W, group, slices, dev):
    p = api.pack(W, group=group, slices=slices)
    n = copies_for(p.blob.numel())
    blobs = [p] + [api.PackedLinear(p.desc, p.blob.clone()) for _ in range(n - 1)]
    torch.cuda.synchronize()
    return blobs


def decode_bytes(p, T, jmax, router=False, prep_bytes=0):
    """Algorithmic bytes of one routed decode launch: the slices the batch needs, the
    activations (or, on the prepared path, the prepared operands), y, and the routing
    inputs and outputs (perm and offsets read; with the router in the launch, Wr or the
    partial logits read and logits, budget, perm and offsets written)."""
    d = p.desc
    xin = prep_bytes if prep_bytes else T * d.k * 2
    base = jmax * int(d.slice_stride) + xin + T * d.n * 2
    if router:
        wr = 0 if prep_bytes else d.k * d.slices * 4
        return base + wr + T * d.slices * 4 + 2 * T * 4 + (d.slices + 1) * 4
    return base + T * 4 + (d.slices + 1) * 4


def weight_bytes(p, jmax):
    return jmax * int(p.desc.slice_stride)


def time_events(torch, fn, iters):
    """Average duration (s) of fn() on the current stream, bracketed by HIP events."""
    s = [torch.cuda.Event(enable_timing=True) for _ in range(iters)]
    e = [torch.cuda.Event(enable_timing=True) for _ in range(iters)]
    for i in range(iters):
        s[i].record()
        fn(i)
        e[i].record()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in zip(s, e)) / iters / 1e3


def graph_time(torch, fn, calls=10, replays=5):
    """Average device time (s) of fn() from replays of a HIP graph holding `calls` calls
    (no host launch overhead between kernels)."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                      # first use on the capture stream, outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / 1e3 / (calls * replays)


def traffic_from_profile(kernel_src: str, name: str):
    """HBM bytes per launch from committed rocprofv3 counters, if the kernel is unchanged."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    src = open(os.path.join(ROOT, "token_adaptive_bit_amd", "csrc", kernel_src), "rb").read()
    if vals.get("source_sha256") != hashlib.sha256(src).hexdigest():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def graph_steps(torch, fn, nb, steps, warmup):
    """Exactly `steps` calls fn(i) (i cycling over the nb weight copies) from HIP graphs: one
    graph holding a call per copy, replayed steps // nb times, then one-call graphs for the
    rest, so neither the host's launch overhead nor a per-replay submission gaps the
    kernels.  Returns (s per call by the host clock, s per call from HIP events on the
    replay stream)."""
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        fn(0)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    big = torch.cuda.CUDAGraph()
    with torch.cuda.graph(big):
        for c in range(nb):
            fn(c)
    single = []
    for c in range(steps % nb):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn(c)
        single.append(g)
    for _ in range(max(1, warmup // nb)):
        big.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for _ in range(steps // nb):
        big.replay()
    for g in single:
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps, a.elapsed_time(b) / 1e3 / steps


def bench_decode(api, torch, inputs, T, steps, warmup, dev, variants=True):
    """The decode step on the 18944 x 3584 workload: route (logits, argmax, regroup) and the
    routed linear through mbq_route_linear with the plan's choices; its dominant kernel (the
    streaming linear) timed alone on prepared operands; and the step's other forms."""
    d = inputs.make_workload("decode_18944x3584")
    W = torch.from_numpy(d["W"]).to(dev, torch.bfloat16)
    X = torch.from_numpy(d["X"][:T]).to(dev, torch.bfloat16)
    Wr = torch.from_numpy(d["Wr"]).to(dev, torch.float32)
    blobs = make_blobs(api, torch, W, 128, 3, dev)
    del W
    nb = len(blobs)
    logits = torch.empty((T, 3), dtype=torch.float32, device=dev)
    budget = torch.empty(T, dtype=torch.int32, device=dev)
    perm = torch.empty(T, dtype=torch.int32, device=dev)
    off = torch.empty(4, dtype=torch.int32, device=dev)
    y = torch.empty((T, d["N"]), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(api.route_linear_workspace(blobs[0], T), 1), dtype=torch.uint8, device=dev)
    prep_bytes = api.route_prepare_workspace(blobs[0], T)
    out = {"T": T, "copies": nb, "blob_bytes": int(blobs[0].blob.numel()), "N": d["N"], "K": d["K"]}

    def step(i, o=None):
        api.route_linear(blobs[i % nb], X, Wr, y=y, logits=logits, budget=budget, perm=perm, offsets=off,
                         workspace=ws, options=o)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    out["eager_step_s"] = (time.perf_counter() - t0) / steps
    if variants:
        out["one_launch_fp8fp4_step_s"] = graph_steps(torch, lambda i: step(i, api.opts(decode_mul="fp8fp4", decode_launches=1)),
                                                      nb, steps, warmup)[1]
        out["one_launch_bf16_step_s"] = graph_steps(torch, lambda i: step(i, api.opts(decode_mul="bf16")),
                                                    nb, steps, warmup)[1]
        out["two_call_step_s"] = graph_steps(torch, lambda i: (api.route(X, Wr, logits, budget, perm, off),
                                                               api.linear(blobs[i % nb], X, perm, off, y=y)),
                                             nb, steps, warmup)[1]
    out["step_s"], out["step_event_s"] = graph_steps(torch, step, nb, steps, warmup)
    # the plan's path: two launches when the operands are prepared (prep_bytes > 0 and the
    # fp8 x fp4 multiply), else one; the dominant kernel alone on prepared operands
    two = prep_bytes > 0 and T > 8
    out["launches"] = 2 if two else 1
    if two:
        prep = api.route_prepare(blobs[0], X, Wr)
        out["prepare_s"] = graph_steps(torch, lambda i: api.route_prepare(blobs[0], X, Wr, prep=prep), nb, steps, warmup)[1]
        out["kernel_s"] = graph_steps(torch, lambda i: api.route_linear_prepared(
            blobs[i % nb], T, prep, y=y, logits=logits, budget=budget, perm=perm, offsets=off), nb, steps, warmup)[1]
    else:
        out["kernel_s"] = out["step_event_s"]
    step(0)                              # last, so logits .. offsets hold the plan's routes
    torch.cuda.synchronize()
    jmax = int((off[:3] < T).sum().item())      # slices with at least one token
    out.update({"jmax": jmax, "budget_counts": torch.diff(off).cpu().tolist(),
                "bytes": decode_bytes(blobs[0], T, jmax, router=True, prep_bytes=prep_bytes if two else 0),
                "weight_bytes": weight_bytes(blobs[0], jmax), "prep_bytes": prep_bytes if two else 0})
    return out


def bench_pack(api, torch, inputs, dev):
    d = inputs.make_workload("decode_18944x3584")
    W = torch.from_numpy(d["W"]).to(dev, torch.bfloat16)
    out = torch.empty(int(api.describe(d["N"], d["K"], 128, 3).total_bytes), dtype=torch.uint8, device=dev)
    api.pack(W, 128, 3, out=out)
    torch.cuda.synchronize()
    return time_events(torch, lambda i: api.pack(W, 128, 3, out=out), 5)


def bench_prefill(api, torch, inputs, dev, iters=20):
    d = inputs.make_workload("prefill_11008x4096")
    W = torch.from_numpy(d["W"]).to(dev, torch.bfloat16)
    X = torch.from_numpy(d["X"]).to(dev, torch.bfloat16)
    budget = torch.from_numpy(d["budget"]).to(dev)
    blobs = make_blobs(api, torch, W, 128, 3, dev)   # > 512 MiB of copies: no cache serves a repeat
    nb = len(blobs)
    perm, off = api.regroup(budget, 3)
    y = torch.empty((d["T"], d["N"]), dtype=torch.bfloat16, device=dev)
    # ~50 ms of launches first: the clocks settle under sustained MFMA load (the first
    # milliseconds run up to ~15% slower)
    for i in range(WARM_PREFILL):
        api.linear(blobs[i % nb], X, perm, off, y=y)
    torch.cuda.synchronize()
    s = time_events(torch, lambda i: api.linear(blobs[i % nb], X, perm, off, y=y), iters)
    flops = 2.0 * d["T"] * d["N"] * d["K"]
    return {"T": d["T"], "linear_s": s, "tflops": flops / s / 1e12, "copies": nb,
            "mfma_frac": flops / s / 1e12 / BF16_PEAK_TFLOPS, "budget_counts": torch.diff(off).cpu().tolist()}


def bench_copy(torch, dev, nbytes=1 << 30):
    a = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    s = time_events(torch, lambda i: b.copy_(a), 10)
    return 2 * nbytes / s / 1e9


def bench_sweep(api, torch, inputs, dev, iters=20):
    """Elasticity sweep, W 14336 x 4096: T in {32, 1024}, budgets forced to 1, 2, 3 and
    router-mixed; bytes of weight read and throughput for each."""
    d = inputs.make_workload("sweep_14336x4096")
    W = torch.from_numpy(d["W"]).to(dev, torch.bfloat16)
    blobs = make_blobs(api, torch, W, 128, 3, dev)
    del W
    nb = len(blobs)
    Wr = torch.from_numpy(d["Wr"]).to(dev, torch.float32)
    out = {}
    for T in (32, 1024):
        X = torch.from_numpy(d["X"][:T]).to(dev, torch.bfloat16)
        y = torch.empty((T, d["N"]), dtype=torch.bfloat16, device=dev)
        for mode in ("b1", "b2", "b3", "router"):
            if mode == "router":
                _, _, perm, off = api.route(X, Wr)
            else:
                perm, off = api.regroup(torch.full((T,), int(mode[1]), dtype=torch.int32, device=dev), 3)
            for i in range(3 if T <= 64 else WARM_PREFILL):
                api.linear(blobs[i % nb], X, perm, off, y=y)
            torch.cuda.synchronize()
            fn = lambda i: api.linear(blobs[i % nb], X, perm, off, y=y)
            # decode launches from replays of graphs that hold one launch per weight copy (no
            # host submission between launches), the prefill's long launches eagerly
            s = graph_steps(torch, fn, nb, nb * max(2, -(-iters // nb)), nb)[1] if T <= 64 else time_events(torch, fn, iters)
            counts = torch.diff(off).cpu().tolist()
            jmax = max(j + 1 for j in range(3) if counts[j] > 0)
            r = {"us": s * 1e6, "tokens_per_s": T / s, "budget_counts": counts,
                 "weight_bytes_read": weight_bytes(blobs[0], jmax)}
            if T <= 64:
                r["hbm_frac"] = decode_bytes(blobs[0], T, jmax) / s / 1e9 / HBM_PEAK_GBS
            else:
                r["tflops"] = 2.0 * T * d["N"] * d["K"] / s / 1e12
            out[f"t{T}_{mode}"] = r
    return out


def bench_route_mlp(api, torch, inputs, dev, iters=50):
    """The pages' MLP router (hidden 256, 3 slices, delta 0.5) on the decode (T=16, K=3584)
    and prefill (T=2048, K=4096) layer inputs: time per call (hidden-layer MFMA kernel,
    gate, regroup) next to the linear-argmax router, the hidden kernel's TFLOP/s, and a
    delta sweep of the average weight bit width with the delta that lands on 3, 4, 5 bits."""
    out = {}
    for T, K in ((16, 3584), (2048, 4096)):
        r = inputs.make_mlp_router(21, K, slices=3, hidden=256)
        R = api.MlpRouter(*(torch.from_numpy(r[n]).to(dev, torch.bfloat16 if n == "W1" else torch.float32)
                            for n in ("W1", "b1", "W2", "b2")))
        d = inputs.make_linear(22, 16, K, T)
        X = torch.from_numpy(d["X"]).to(dev, torch.bfloat16)
        Wr = torch.from_numpy(d["Wr"]).to(dev, torch.float32)
        sc, b, perm, off = api.route_mlp(X, R, 0.5)
        ws = torch.empty(max(1, api.route_mlp_workspace(T, K, 256)), dtype=torch.uint8, device=dev)
        for _ in range(3):
            api.route_mlp(X, R, 0.5, sc, b, perm, off, workspace=ws)
        torch.cuda.synchronize()
        b_eager = b.clone()
        lg, lb, lp, lo = api.route(X, Wr)
        torch.cuda.synchronize()
        t_mlp = time_events(torch, lambda i: api.route_mlp(X, R, 0.5, sc, b, perm, off, workspace=ws), iters)
        t_lin = time_events(torch, lambda i: api.route(X, Wr, lg, lb, lp, lo), iters)
        # device time without host launch overhead: 10 calls captured in a HIP graph
        g_mlp = graph_time(torch, lambda: api.route_mlp(X, R, 0.5, sc, b, perm, off, workspace=ws))
        ok = bool(torch.equal(b, b_eager))
        g_lin = graph_time(torch, lambda: api.route(X, Wr, lg, lb, lp, lo))
        res = {"us_per_call_eager": t_mlp * 1e6, "us_per_call_graph": g_mlp * 1e6,
               "linear_router_us_eager": t_lin * 1e6, "linear_router_us_graph": g_lin * 1e6,
               "graph_replay_matches_eager": ok,
               "hidden_tflops_graph": 2.0 * T * K * 256 / g_mlp / 1e12,
               "budget_counts_delta_0.5": torch.diff(off).cpu().tolist()}
        sweep = {}
        for delta in (0.1, 0.2, 0.3, 0.4, 0.5, 0.6, 0.7, 0.8, 0.9):
            bb, _, _ = api.route_mlp_from_scores(sc, delta)
            sweep[f"{delta:.1f}"] = 2.0 * bb.double().mean().item()
        res["avg_bits_by_delta"] = sweep
        hits = {}
        for target in (3.0, 4.0, 5.0):
            lo_d, hi_d = 0.0, 1.0          # average bits fall as delta rises
            for _ in range(30):
                mid = 0.5 * (lo_d + hi_d)
                bb, _, _ = api.route_mlp_from_scores(sc, mid)
                if 2.0 * bb.double().mean().item() > target:
                    lo_d = mid
                else:
                    hi_d = mid
            bb, _, _ = api.route_mlp_from_scores(sc, hi_d)
            hits[f"{target:.0f}"] = {"delta": hi_d, "avg_bits": 2.0 * bb.double().mean().item()}
        res["delta_for_bits"] = hits
        out[f"t{T}_k{K}"] = res
    return out


def bench_bitplane(api, torch, inputs, dev):
    """Residual slices against bit-plane slices on the decode weight (18944 x 3584, G128,
    S3): relative error of x . W^(b)^T against the float32 product x . W^T for each b
    (every token forced to b), the routed linear's time on each blob, and pack times."""
    d = inputs.make_workload("decode_18944x3584")
    T = 16
    W = torch.from_numpy(d["W"]).to(dev, torch.bfloat16)
    X = torch.from_numpy(d["X"][:T]).to(dev, torch.bfloat16)
    ref = X.float() @ W.float().t()
    out = {}
    for name, fn in (("residual", api.pack), ("bitplane", api.pack_bitplane)):
        p = fn(W, 128, 3)
        torch.cuda.synchronize()
        tp = time_events(torch, lambda i: fn(W, 128, 3, out=p.blob), 5)
        res = {"pack_us": tp * 1e6}
        y = torch.empty((T, d["N"]), dtype=torch.float32, device=dev)
        ws = torch.empty(max(1, api.linear_workspace(p, T)), dtype=torch.uint8, device=dev)
        for b in (1, 2, 3):
            perm, off = api.regroup(torch.full((T,), b, dtype=torch.int32, device=dev), 3)
            api.linear(p, X, perm, off, y=y, workspace=ws)
            torch.cuda.synchronize()
            res[f"rel_err_b{b}"] = float(((y - ref).norm() / ref.norm()).item())
            res[f"linear_us_b{b}"] = time_events(torch, lambda i: api.linear(p, X, perm, off, y=y, workspace=ws), 20) * 1e6
        out[name] = res
        del p
    return out


def bench_lowrank(api, torch, inputs, dev, iters=30):
    """The low-rank side path (rank 16) on the decode workload (T = 16) and the prefill
    workload (T = 2048): routed linear with and without it over rotated weight copies
    (decode from graph replays, prefill eagerly)."""
    out = {}
    for name, T, seed in (("decode_18944x3584", 16, 102), ("prefill_11008x4096", 2048, 103)):
        d = inputs.make_workload(name)
        N, K = d["N"], d["K"]
        W = torch.from_numpy(d["W"]).to(dev, torch.bfloat16)
        blobs = make_blobs(api, torch, W, 128, 3, dev)
        del W
        nb = len(blobs)
        X = torch.from_numpy(d["X"][:T]).to(dev, torch.bfloat16)
        if d["budget"] is not None:
            perm, off = api.regroup(torch.from_numpy(d["budget"]).to(dev), 3)
        else:
            _, _, perm, off = api.route(X, torch.from_numpy(d["Wr"]).to(dev, torch.float32))
        lr = inputs.make_lowrank(seed, N, K, rank=16)
        A = torch.from_numpy(lr["A"]).to(dev, torch.bfloat16)
        B = torch.from_numpy(lr["B"]).to(dev, torch.bfloat16)
        y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
        ws0 = torch.empty(max(1, api.linear_workspace(blobs[0], T)), dtype=torch.uint8, device=dev)
        ws1 = torch.zeros(max(1, api.linear_lowrank_workspace(blobs[0], T, 16)), dtype=torch.uint8, device=dev)  # call state starts at zero
        plain = lambda i: api.linear(blobs[i % nb], X, perm, off, y=y, workspace=ws0)
        side = lambda i: api.linear_lowrank(blobs[i % nb], X, perm, off, A, B, y=y, workspace=ws1)
        for f in (plain, side):
            for i in range(3 if T <= 64 else WARM_PREFILL):
                f(i)
        torch.cuda.synchronize()
        if T <= 64:
            steps = nb * max(2, -(-iters // nb))
            t0 = graph_steps(torch, plain, nb, steps, nb)[1]
            t1 = graph_steps(torch, side, nb, steps, nb)[1]
            how = "graph"
        else:
            t0 = time_events(torch, plain, iters)
            t1 = time_events(torch, side, iters)
            how = "eager"
        torch.cuda.synchronize()
        # the side path's call state words: launches that computed u inside the streaming
        # decode, an unused word (0), error flags (0)
        state = ws1[:12].view(torch.int32).cpu().tolist()
        out[f"t{T}_{N}x{K}"] = {"N": N, "K": K, "T": T, "rank": 16, "copies": nb, "timing": how,
                                "linear_us": t0 * 1e6, "linear_lowrank_us": t1 * 1e6,
                                "overhead_frac": t1 / t0 - 1.0, "u_in_launch_state": state}
        del blobs
    return out


def bench_layer(api, torch, inputs, dev, iters=20):
    """Seven linears of a 14B-like decoder layer at T = 64 with one router on the layer
    input: total time of route + 7 routed linears, and HBM fraction of the linears; then
    the same layer with q/k/v and gate/up fused (one blob and one launch per shared input):
    route + 4 routed linears."""
    lay = inputs.make_workload("layer14b_t64")
    T = lay["T"]
    x0 = torch.from_numpy(lay["X_layer"]).to(dev, torch.bfloat16)
    Wr = torch.from_numpy(lay["Wr"]).to(dev, torch.float32)
    lin = {l["name"]: l for l in lay["linears"]}
    Wd = {n: torch.from_numpy(l["W"]).to(dev, torch.bfloat16) for n, l in lin.items()}
    Xd = {n: torch.from_numpy(l["X"]).to(dev, torch.bfloat16) for n, l in lin.items()}
    _, _, perm, off = api.route(x0, Wr)

    def run(groups):
        # groups: (weight names, activation name) sharing one blob and one launch; two
        # copies of the layer's blobs (2 x 267.6 MB, over 512 MiB) alternate between steps,
        # so neither L2 nor the 256 MiB Infinity Cache serves a repeat
        packs, xs, ys = [[], []], [], []
        for names, xn in groups:
            p, _ = api.pack_concat([Wd[n] for n in names], 128, 3)
            packs[0].append(p)
            packs[1].append(api.PackedLinear(p.desc, p.blob.clone()))
            xs.append(x0 if xn == "layer" else Xd[xn])
            ys.append(torch.empty((T, p.n), dtype=torch.bfloat16, device=dev))
        torch.cuda.synchronize()

        def step(i):
            api.route(x0, Wr, perm=perm, offsets=off)
            for p, x, y in zip(packs[i % 2], xs, ys):
                api.linear(p, x, perm, off, y=y)

        s = graph_steps(torch, step, 2, iters, 100)[1]
        counts = torch.diff(off).cpu().tolist()
        jmax = max(j + 1 for j in range(3) if counts[j] > 0)
        nbytes = sum(decode_bytes(p, T, jmax) for p in packs[0])
        return {"us": s * 1e6, "tokens_per_s": T / s, "launches": 2 + len(groups), "layer_copies": 2,
                "budget_counts": counts, "hbm_frac_incl_route": nbytes / s / 1e9 / HBM_PEAK_GBS}

    out = {"T": T}
    out["separate"] = run([([n], "layer" if n == "q" else n) for n in lin])
    out["fused_qkv_gateup"] = run([(["q", "k", "v"], "layer"), (["o"], "o"), (["gate", "up"], "gate"),
                                   (["down"], "down")])
    out["note"] = ("steps replayed from HIP graphs over two copies of the layer's blobs (535 MB); the router "
                   "(two launches) runs on the layer input once per step; its logits are not fused into "
                   "the previous op (norm and residual lie outside this path)")
    return out


def run_traffic(api, torch, inputs, dev, T, launches=20):
    """For the counter passes: a copy of 1 GiB (known bytes), then `launches` decode steps
    (mbq_route_linear, the plan's path) over rotated weight copies."""
    bench_copy(torch, dev)
    d = inputs.make_workload("decode_18944x3584")
    W = torch.from_numpy(d["W"]).to(dev, torch.bfloat16)
    X = torch.from_numpy(d["X"][:T]).to(dev, torch.bfloat16)
    Wr = torch.from_numpy(d["Wr"]).to(dev, torch.float32)
    blobs = make_blobs(api, torch, W, 128, 3, dev)
    del W
    y = torch.empty((T, d["N"]), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(api.route_linear_workspace(blobs[0], T), 1), dtype=torch.uint8, device=dev)
    for i in range(launches):          # the decode step as timed
        _, _, _, _, off = api.route_linear(blobs[i % len(blobs)], X, Wr, y=y, workspace=ws)
    torch.cuda.synchronize()
    counts = torch.diff(off).cpu().tolist()
    jmax = max(j + 1 for j in range(3) if counts[j] > 0)
    prep = api.route_prepare_workspace(blobs[0], T) if T > 8 else 0
    return {"workload": "traffic", "copy_bytes": 2 * (1 << 30),
            "decode_bytes": decode_bytes(blobs[0], T, jmax, router=True, prep_bytes=prep), "launches": launches}


def cpu_baseline(inputs, T):
    """The oracle as it stands, timed on the host on a bounded sample of the same step:
    route + regroup + routed linear for the same T tokens against a row slice of W."""
    import numpy as np
    from oracle import mbq_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = 1
    d = inputs.make_workload("decode_18944x3584")
    rows = 4736                                  # a quarter of the 18944 output rows
    p = O.pack(d["W"][:rows], 128, 3)
    X = d["X"][:T]
    reps = 0
    t0 = time.perf_counter()
    while True:
        deq = O.dequant_slices(p["codes"], p["scale"], p["zero"], 128)
        b = O.route_from_logits(O.router_logits(X, d["Wr"]))
        O.regroup(b, 3)
        O.linear(X, deq, b)
        reps += 1
        if time.perf_counter() - t0 > 10.0:
            break
    s = (time.perf_counter() - t0) / reps
    # scale to the full step: the sample is a quarter of the rows
    full_step_s = s * d["N"] / rows
    return {"value": T / full_step_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} oracle steps (route + regroup + float64 dequant and linear) for "
                      f"{T} tokens on {rows} of {d['N']} rows, scaled by {d['N'] / rows:.0f}x; "
                      f"{s:.2f} s per sample step"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the library has no "
              f"multi-GPU path.  Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    from token_adaptive_bit_amd import api, inputs
    dev = "cuda:0"
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.only == "prefill":
        bench_copy(torch, dev)          # a copy of known size first: the counter passes' calibration
        r = bench_prefill(api, torch, inputs, dev, iters=max(args.steps, 1))
        print(json.dumps({"workload": "prefill", **r}))
        return
    if args.only == "sweep":
        print(json.dumps({"workload": "sweep", **bench_sweep(api, torch, inputs, dev)}))
        return
    if args.only == "layer":
        print(json.dumps({"workload": "layer", **bench_layer(api, torch, inputs, dev)}))
        return
    if args.only == "bitplane":
        print(json.dumps({"workload": "bitplane", **bench_bitplane(api, torch, inputs, dev)}))
        return
    if args.only == "lowrank":
        print(json.dumps({"workload": "lowrank", **bench_lowrank(api, torch, inputs, dev)}))
        return
    if args.only == "route_mlp":
        print(json.dumps({"workload": "route_mlp", **bench_route_mlp(api, torch, inputs, dev)}))
        return
    if args.only == "traffic":
        print(json.dumps(run_traffic(api, torch, inputs, dev, args.tokens, launches=max(args.steps, 1))))
        return

    log(f"decode T={args.tokens}: {args.warmup} warmup + {args.steps} timed steps")
    r = bench_decode(api, torch, inputs, args.tokens, args.steps, args.warmup, dev)
    kernel = "decode_stream_kernel (prepared operands)" if r["launches"] == 2 else "decode_stream_kernel"
    achieved = r["bytes"] / r["kernel_s"] / 1e9
    traffic = traffic_from_profile("decode_stream.hip", f"decode_stream_18944x3584_t{args.tokens}_traffic.txt")
    out = {
        "metric": METRIC,
        "value": args.tokens / r["step_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["step_s"] * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 io; fp8 (e4m3 hi+lo) x fp4 (e2m1 codes) mfma, fp32 acc",
        "data": "synthetic",
        "config": {"workload": "decode GEMV 18944x3584 (Qwen2.5-7B-like up-proj), G128, S3, "
                               f"bf16, T{args.tokens}, router argmax",
                   "N": r["N"], "K": r["K"], "group": 128, "slices": 3, "tokens": args.tokens,
                   "budget_counts": r["budget_counts"], "slices_read": r["jmax"],
                   "weight_copies_rotated": r["copies"], "launches_per_step": r["launches"],
                   "multiply": "fp8 x fp4 (activations as exact e4m3 hi + lo pairs, one e8m0 scale per "
                               "token and 128 inputs; codes as e2m1)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": kernel, "kernel_us": r["kernel_s"] * 1e6,
                     "algorithmic_bytes_per_launch": r["bytes"]},
        "effective_weight_gbs": r["weight_bytes"] / r["kernel_s"] / 1e9,
        "step_launch": f"hip_graph, {r['launches']} kernel(s) per step (mbq_route_linear)",
        "step_us_events": r["step_event_s"] * 1e6,
        "prepare_us": r.get("prepare_s", 0.0) * 1e6,
        "eager_ms_per_step": r["eager_step_s"] * 1e3,
        "one_launch_fp8fp4_ms_per_step": r["one_launch_fp8fp4_step_s"] * 1e3,
        "one_launch_bf16_ms_per_step": r["one_launch_bf16_step_s"] * 1e3,
        "two_call_ms_per_step": r["two_call_step_s"] * 1e3,
    }
    if not args.no_extra and args.only is None:  # (--only decode prints the headline line alone)
        extra = {}
        for T in (1, 4):
            if T != args.tokens:
                log(f"decode T={T}")
                q = bench_decode(api, torch, inputs, T, 100, 10, dev, variants=False)
                extra[f"decode_t{T}"] = {"tokens_per_s": T / q["step_s"], "step_us": q["step_event_s"] * 1e6,
                                         "kernel_us": q["kernel_s"] * 1e6, "launches": q["launches"],
                                         "slices_read": q["jmax"],
                                         "hbm_frac": q["bytes"] / q["kernel_s"] / 1e9 / HBM_PEAK_GBS,
                                         "effective_weight_gbs": q["weight_bytes"] / q["kernel_s"] / 1e9}
        log("prefill 11008x4096 T=2048")
        pf = bench_prefill(api, torch, inputs, dev)
        extra["prefill_11008x4096_t2048"] = {"tflops": pf["tflops"], "mfma_frac": pf["mfma_frac"],
                                             "linear_us": pf["linear_s"] * 1e6,
                                             "budget_counts": pf["budget_counts"],
                                             "hbm_traffic_bytes": traffic_from_profile(
                                                 "prefill_mfma.hip", "prefill_mfma_11008x4096_t2048_traffic.txt")}
        log("elasticity sweep 14336x4096")
        extra["sweep_14336x4096"] = bench_sweep(api, torch, inputs, dev)
        log("MLP router with threshold delta")
        extra["route_mlp_h256_s3"] = bench_route_mlp(api, torch, inputs, dev)
        log("bit-plane slices")
        extra["bitplane_vs_residual_18944x3584"] = bench_bitplane(api, torch, inputs, dev)
        log("low-rank side path")
        extra["lowrank_r16"] = bench_lowrank(api, torch, inputs, dev)
        log("14B-like layer, T=64")
        extra["layer14b_t64"] = bench_layer(api, torch, inputs, dev)
        log("pack")
        extra["pack_18944x3584_s3_us"] = bench_pack(api, torch, inputs, dev) * 1e6
        extra["copy_kernel_gbs"] = bench_copy(torch, dev)
        out["extra"] = extra
    if not args.no_cpu:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(inputs, args.tokens)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
