"""Benchmark of one tensor-parallel rank's MLP shard on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path for one rank: the fused
column-parallel up-projection + activation, the row-parallel down-projection,
the local reduction of the t partial sums (the other ranks' partials are
stand-in buffers resident in HBM, the bias added once), the backward (dgrad
through W2 with the activation derivative, both weight gradients, dgrad
through W1) and the reduction of the t partial input gradients.  Inputs are
seeded synthetic bf16 tensors already resident in HBM.  Prints one JSON line.

Also reported in the same line: per-kernel average durations (HIP events on
the launch stream after every kernel, from a timed pass of its own),
the roofline of the dominant kernel, the one-token decode GEMV path
(``llama3_70b_decode_t4``, weights rotated over several copies so the
256 MiB Infinity Cache cannot hold them), and the fp64 oracle timed on the
host cores on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "per-rank TP MLP fwd+bwd TFLOP/s (bf16) and % MFMA peak; decode GB/s % HBM"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    # about 85 ms of the step before timing: the chip's clock takes tens of
    # milliseconds of sustained load to settle (with 5 warm-up steps the
    # timed steps ran about 2.5% slower)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--workload", default="gpt3_train_t8")
    p.add_argument("--decode-workload", default="llama3_70b_decode_t4")
    p.add_argument("--decode-steps", type=int, default=200)
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-attn", action="store_true")
    p.add_argument("--no-ln", action="store_true")
    p.add_argument("--no-other", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    return p.parse_args()


class GpuMetrics:
    """The GPU's gfx clock (per XCD) and socket power from amdsmi's GPU
    metrics table.  The table is refreshed about once a second, so a clock
    figure needs a pass of about that length: see clock_pass.  None where
    amdsmi or the metrics are not available."""

    def __init__(self):
        self.err, self._h = None, None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._amdsmi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
        except Exception as e:  # no amdsmi, no permission, no device
            self.err = f"{type(e).__name__}: {e}"

    def read(self):
        """(table counter, per-XCD clocks in MHz, socket power in W) or None."""
        if self._h is None:
            return None
        try:
            m = self._amdsmi.amdsmi_get_gpu_metrics_info(self._h)
        except Exception as e:
            self.err = f"{type(e).__name__}: {e}"
            return None
        clks = m.get("current_gfxclks")
        vals = [float(v) for v in clks if isinstance(v, (int, float)) and 0 < v < 65535] if isinstance(clks, list) else []
        if not vals and isinstance(m.get("current_gfxclk"), (int, float)):
            vals = [float(m["current_gfxclk"])]
        pw = m.get("current_socket_power")
        return (m.get("system_clock_counter"), vals, float(pw) if isinstance(pw, (int, float)) else None)


def clock_pass(step, torch, seconds=3.0, settle=1.2, batch=100):
    """The gfx clock and socket power while `step` runs back to back for
    `seconds`: distinct snapshots of the metrics table taken after `settle`
    seconds (the table lags by up to about a second)."""
    import statistics
    gm = GpuMetrics()
    if gm.read() is None:
        return {"mhz_mean": None, "error": gm.err}
    snaps, seen = [], set()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(batch):
            step()
        r = gm.read()
        torch.cuda.synchronize()
        if r and time.perf_counter() - t0 > settle and r[0] not in seen and r[1]:
            seen.add(r[0])
            snaps.append(r)
    if not snaps:
        return {"mhz_mean": None, "error": "no metrics snapshot during the pass"}
    nx = max(len(v) for _, v, _ in snaps)
    per_xcd = [round(statistics.mean(v[i] for _, v, _ in snaps if len(v) == nx), 1) for i in range(nx)]
    pw = [p for _, _, p in snaps if p is not None]
    return {"mhz_mean": round(statistics.mean(statistics.mean(v) for _, v, _ in snaps), 1),
            "per_xcd_mhz_mean": per_xcd, "socket_power_w_mean": round(statistics.mean(pw), 1) if pw else None,
            "snapshots": len(snaps), "pass_s": round(time.perf_counter() - t0, 2),
            "source": "amdsmi GPU metrics (current_gfxclks, current_socket_power), distinct snapshots while the "
                      "headline step runs back to back in a pass of its own right after the timed steps (the "
                      "table refreshes about once a second, longer than the timed steps)"}


def train_step(w, steps, warmup, B, I, torch, np, to_dev, clock_s=True):
    """Time `steps` passes of rank 0's whole hot path for workload w: forward,
    reduce of the t partial sums (+ bias), backward (+ bias gradient), reduce
    of the t dX partials, launched through the step entry points (the
    composite entry points launch exactly these kernels in this order).

    Two timed passes of `steps` steps each, after `warmup` untimed ones:
    the first records a HIP event on the launch stream after every kernel
    (the per-kernel durations, from which the longest GEMM is the dominant
    kernel); the second, the headline, records events only around the
    dominant kernel, whose average duration it also gives.  An event after
    every kernel costs about 1% of the GPT-3 shard's step, which the headline
    does not carry.  The buffers are freed on return."""
    dev = "cuda"
    bf, f32 = torch.bfloat16, torch.float32
    sw = w.act == "swiglu"
    N, h, Fi, t = w.N, w.h, w.Fi, w.t
    log(f"[bench] generating inputs for {w.name}: N={N} h={h} F_i={Fi} t={t} act={w.act}")
    host = {"X": I.gen_x(w.wid, N, h), "dY": I.gen_dy(w.wid, N, h), "W1_i": I.gen_w_up_shard(w.wid, h, Fi, 0),
            "W2_i": I.gen_w_down_shard(w.wid, h, Fi, 0)}
    if sw:
        host["Wg_i"] = I.gen_w_gate_shard(w.wid, h, Fi, 0)
    if w.bias:
        host["b2"] = I.gen_b2(w.wid, h)
    # the bf16 bit patterns' digests: the inputs can be regenerated and checked
    digests = {k: hashlib.sha256(np.ascontiguousarray(v).tobytes()).hexdigest()[:16] for k, v in host.items()}
    X, dY, W1, W2 = (to_dev(host[k]) for k in ("X", "dY", "W1_i", "W2_i"))
    Wg = to_dev(host["Wg_i"]) if sw else None
    b2 = to_dev(host["b2"]) if w.bias else None
    del host
    shape = B.make_shape(N, h, w.F, t, 0, w.act)
    Y = torch.empty(N, h, dtype=bf, device=dev)
    A = torch.empty(N, Fi, dtype=bf, device=dev)
    U = torch.empty(N, Fi, dtype=bf, device=dev)
    G = torch.empty(N, Fi, dtype=bf, device=dev) if sw else None
    dU = torch.empty(N, w.g * Fi, dtype=bf, device=dev)
    dW1 = torch.empty(h, Fi, dtype=f32, device=dev)
    dWg = torch.empty(h, Fi, dtype=f32, device=dev) if sw else None
    dW2 = torch.empty(Fi, h, dtype=f32, device=dev)
    dX = torch.empty(N, h, dtype=bf, device=dev)
    db2 = torch.empty(h, dtype=f32, device=dev) if w.bias else None
    Yred = torch.empty(N, h, dtype=bf, device=dev)
    dXred = torch.empty(N, h, dtype=bf, device=dev)
    ws_f = B.alloc_workspace(B.workspace_bytes(shape, False))
    ws_b = B.alloc_workspace(B.workspace_bytes(shape, True))
    # the other ranks' partial sums (stand-ins: resident bf16 buffers)
    B.tp_mlp_fwd_shard(shape, X, W1, Wg, W2, Y, A, U, G, ws_f)
    others_y = [Y.clone() for _ in range(t - 1)]
    B.tp_mlp_bwd_shard(shape, X, W1, Wg, W2, dY, A, U, G, dU, dW1, dWg, dW2, dX, db2, ws_b)
    others_dx = [dX.clone() for _ in range(t - 1)]
    torch.cuda.synchronize()

    ws_db = B.alloc_workspace(B.bias_grad_workspace_bytes(N, h)) if w.bias else None
    if ws_f is not None:
        # a forward that needs a workspace takes the small-batch split-K path
        # (N <= 128), which only the composite call runs
        kernels = [("fwd", 2 * N * h * Fi * (w.g + 1),
                    lambda: B.tp_mlp_fwd_shard(shape, X, W1, Wg, W2, Y, A, U, G, ws_f))]
    else:
        kernels = [("up_act", 2 * N * h * Fi * w.g, lambda: B.tp_mlp_up_act_shard(shape, X, W1, Wg, A, U, G)),
                   ("down", 2 * N * h * Fi, lambda: B.tp_mlp_down_shard(shape, A, W2, Y))]
    kernels += [("reduce_y", 0, lambda: B.tp_mlp_reduce_partials_local([Y] + others_y, Yred, bias=b2))]
    if ws_f is not None:
        # few tokens: the composite backward (split-K input gradients, then both
        # weight gradients in one launch)
        kernels += [("bwd", 4 * N * h * Fi * (w.g + 1),
                     lambda: B.tp_mlp_bwd_shard(shape, X, W1, Wg, W2, dY, A, U, G, dU, dW1, dWg, dW2, dX))]
    else:
        # dU and dW2, then dX_partial and dW1 (dWg): one mixed launch each when their
        # tiles fill the GPU
        kernels += [
            ("down_bwd", 4 * N * h * Fi, lambda: B.tp_mlp_down_bwd_shard(shape, dY, W2, U, G, A, dU, dW2)),
            ("up_bwd", 4 * N * h * Fi * w.g, lambda: B.tp_mlp_up_bwd_shard(shape, X, dU, W1, Wg, dX, dW1, dWg)),
        ]
    if w.bias:
        kernels.append(("bias_grad", 0, lambda: B.tp_mlp_bias_grad(dY, db2, ws_db)))
    kernels.append(("reduce_dx", 0, lambda: B.tp_mlp_reduce_partials_local([dX] + others_dx, dXred)))

    for _ in range(warmup):
        for _, _, fn in kernels:
            fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    # pass 1: an event after every kernel
    nk = len(kernels)
    evs = [ev() for _ in range(steps * nk + 1)]
    evs[0].record(stream)
    for s in range(steps):
        for j, (_, _, fn) in enumerate(kernels):
            fn()
            evs[s * nk + j + 1].record(stream)
    torch.cuda.synchronize()
    kern_ms = {name: float(np.mean([evs[s * nk + j].elapsed_time(evs[s * nk + j + 1]) for s in range(steps)]))
               for j, (name, _, _) in enumerate(kernels)}
    ms_all_events = evs[0].elapsed_time(evs[-1]) / steps
    gemms = [(n, fl) for n, fl, _ in kernels if fl > 0]
    dom = max(gemms, key=lambda x: kern_ms[x[0]])[0]
    # pass 2 (the headline): events only around the dominant kernel
    e0, e1 = ev(), ev()
    dev_evs = [(ev(), ev()) for _ in range(steps)]
    t_wall = time.perf_counter()
    e0.record(stream)
    for s in range(steps):
        for name, _, fn in kernels:
            if name == dom:
                dev_evs[s][0].record(stream)
                fn()
                dev_evs[s][1].record(stream)
            else:
                fn()
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    clk = clock_pass(lambda: [fn() for _, _, fn in kernels], torch) if clock_s else None
    ms = e0.elapsed_time(e1) / steps
    dom_ms = float(np.mean([a.elapsed_time(b) for a, b in dev_evs]))
    # one step each: from the event before the dominant kernel to the same event of the next step
    per_step = [dev_evs[s][0].elapsed_time(dev_evs[s + 1][0]) for s in range(steps - 1)]
    flops = w.flops_train()
    tflops = flops / (ms * 1e-3) / 1e12
    # a short step is partly the host's launch time: its steps also run from a captured graph
    ms_graph = graph_time(torch, [lambda: [fn() for _, _, fn in kernels]] * steps) * 1e-3 if ms < 0.5 else None
    log(f"[bench] {w.name}: {ms:.3f} ms/step, {tflops:.1f} TFLOP/s (wall {t_wall * 1e3 / steps:.3f} ms/step; "
        f"{ms_all_events:.3f} ms/step with an event after every kernel"
        + (f"; {ms_graph:.3f} ms/step replayed from a captured graph" if ms_graph else "") + f"); {dom} {dom_ms:.3f} ms")
    return {"ms": ms, "tflops": tflops, "kern_ms": kern_ms, "ms_all_events": ms_all_events, "dom": dom,
            "ms_graph": ms_graph,
            "step_ms_median": float(np.median(per_step)) if per_step else ms,
            "step_ms_min": float(np.min(per_step)) if per_step else ms,
            "dom_ms": dom_ms, "flops": flops, "inputs_sha256": digests, "gemms": gemms, "clock": clk}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the benchmark runs one tensor-parallel rank's shard on a single "
              f"MI355X (the t shards of a group are run one after another on it); --gpus {args.gpus} "
              f"is not supported.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from megatron_tensor_transformer_rank_amd import binding as B
    from megatron_tensor_transformer_rank_amd import inputs as I
    from megatron_tensor_transformer_rank_amd.configs import WORKLOADS

    B.lib()  # raises if libtpmlp.so is missing: there is no other path
    w = WORKLOADS[args.workload]
    N, h, Fi, t = w.N, w.h, w.Fi, w.t

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")

    st = train_step(w, args.steps, args.warmup, B, I, torch, np, to_dev)
    ms, tflops, kern_ms, gemms, flops = st["ms"], st["tflops"], st["kern_ms"], st["gemms"], st["flops"]
    dom = st["dom"]
    dom_fl = dict(gemms)[dom]
    achieved = dom_fl / (st["dom_ms"] * 1e-3) / 1e12
    traffic = counter_traffic(f"gemm_hbm_traffic_{w.name}.md", GEMM_SOURCES, dom)
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic["bytes"] if traffic else None,
                "flops_per_launch": dom_fl, "avg_launch_ms": round(st["dom_ms"], 4)}
    if traffic:
        roofline["traffic_unit"] = ("bytes per launch the L2s fetch from and write to the fabric (FETCH_SIZE + "
                                    "WRITE_SIZE: Infinity Cache hits included, so not HBM bytes alone), each "
                                    "scaled by its reading for a device copy of known size")
        roofline["algorithmic_bytes"] = traffic["algorithmic_bytes"]
    log("[bench] per-kernel ms: " + ", ".join(f"{k}={v:.3f}" for k, v in kern_ms.items()))
    copy = copy_probe(torch)
    log(f"[bench] copy probe: {copy['GB/s']:.0f} GB/s")

    result = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "N": N, "h": h, "F": w.F, "t": t, "F_i": Fi, "act": w.act,
                   "bias": w.bias, "step": "one rank fwd+bwd + local reduce of t partials (Y and dX)",
                   "flops_per_step": flops, "tokens_per_s": round(N / (ms * 1e-3), 1),
                   "frac_of_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
                   "inputs_sha256": st["inputs_sha256"]},
        "roofline": roofline,
        "kernels_ms": {k: round(v, 4) for k, v in kern_ms.items()},
        "ms_per_step_event_per_kernel": round(st["ms_all_events"], 4),
        "step_ms_median": round(st["step_ms_median"], 4), "step_ms_min": round(st["step_ms_min"], 4),
        "copy_probe": copy,
        "gpu_clock": st["clock"],
    }

    torch.cuda.empty_cache()
    # ---- decode (one token, and small batches), HBM bound; weights rotated over copies
    if not args.no_decode:
        result["decode"] = bench_decode(args, WORKLOADS[args.decode_workload], B, I, torch, np, to_dev)
        torch.cuda.empty_cache()
    # ---- the other training configurations, same step, reported beside the headline
    if not args.no_other:
        other = {}
        for name in ("mlp128_h1024_gelu_t2", "llama_7b_train_t2", "llama3_70b_prefill_t4"):
            if name == w.name:
                continue
            o = train_step(WORKLOADS[name], 10, 3, B, I, torch, np, to_dev, clock_s=False)
            ow = WORKLOADS[name]
            other[name] = {"ms_per_step": round(o["ms"], 4), "TFLOP/s": round(o["tflops"], 1),
                           "frac_of_bf16_peak": round(o["tflops"] / PEAK_BF16_TFLOPS, 4),
                           "tokens_per_s": round(ow.N / (o["ms"] * 1e-3), 1), "flops_per_step": o["flops"],
                           "kernels_ms": {k: round(v, 4) for k, v in o["kern_ms"].items()}}
            if o["ms_graph"]:
                other[name]["ms_per_step_graph"] = round(o["ms_graph"], 4)
            torch.cuda.empty_cache()
        result["other_configs"] = other
    # ---- attention block projections of the same model scale
    if not args.no_attn:
        result["attention_projections"] = bench_attn(args, B, I, torch, np, to_dev)
    if not args.no_ln:
        result["sp_layernorm"] = {name: bench_ln(B, I, torch, to_dev, name, N, h, t)
                                  for name, N, h, t in (("gpt3_sp_t8", 2048, 12288, 8),
                                                        ("llama3_70b_prefill_sp_t4", 16384, 8192, 4))}
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        gpu = {w.name: {"TFLOP/s": round(tflops, 2), "ms_per_step": round(ms, 4)}}
        for name, o in result.get("other_configs", {}).items():
            gpu[name] = {"TFLOP/s": o["TFLOP/s"], "ms_per_step": o["ms_per_step"]}
        if "decode" in result:
            gpu[result["decode"]["workload"]] = {"GB/s_of_weights": result["decode"]["value"],
                                                 "us_per_token": result["decode"]["us_per_token"]}
        result["cpu_baseline"] = cpu_baseline(w, I, list(CPU_ORACLE_ROWS), gpu)
    print(json.dumps(result), flush=True)



DECODE_WINDOWS = 5
GEMM_SOURCES = ("gemm.hip", "gemm.h", "tiles.h", "common.h")
GEMV_SOURCES = ("gemv.hip", "gemv.h", "common.h")


def code_only(text: str) -> str:
    """C/C++ source without its comments, trailing blanks and empty lines (a
    change of comments alone does not change a kernel)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":                       # string or character literal, copied whole
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            while i < n and text[i] != "\n":
                i += 1
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = (ln.rstrip() for ln in "".join(out).split("\n"))
    return "\n".join(ln for ln in lines if ln)


def source_hash(files):
    """sha256 over the code of the named kernel sources (csrc/), comments
    excluded."""
    hsh = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "megatron_tensor_transformer_rank_amd", "csrc", f), encoding="utf-8") as fh:
            hsh.update(code_only(fh.read()).encode())
    return hsh.hexdigest()


def counter_traffic(summary, files, kernel):
    """L2<->fabric bytes per launch of `kernel` (what the L2s fetch and write
    back, Infinity Cache hits included), from a committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, each scaled by what the same counter
    reads for a plain copy of known size).  None when there is no summary or
    the kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    info = None
    with open(path) as fh:
        for line in fh:
            if line.startswith("traffic_json: "):
                info = json.loads(line[len("traffic_json: "):])
    if not info or info.get("source_sha256") != source_hash(files):
        return None
    return info.get("kernels", {}).get(kernel)


def copy_probe(torch, nbytes=1 << 30, reps=5):
    """Device-to-device copy of a 1 GiB buffer: the plain streaming rate."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / reps
    del src, dst
    return {"bytes_moved": 2 * nbytes, "GB/s": round(2 * nbytes / sec / 1e9, 1)}

def bench_decode(args, w, B, I, torch, np, to_dev):
    bf = torch.bfloat16
    h, Fi = w.h, w.Fi
    sw = w.act == "swiglu"
    log(f"[bench] decode {w.name}: h={h} F_i={Fi} act={w.act}")
    x = to_dev(I.gen_x(w.wid, 1, h))
    W1 = to_dev(I.gen_w_up_shard(w.wid, h, Fi, 0))
    W2 = to_dev(I.gen_w_down_shard(w.wid, h, Fi, 0))
    Wg = to_dev(I.gen_w_gate_shard(w.wid, h, Fi, 0)) if sw else None
    wbytes = w.weight_bytes()
    nsets = max(4, int(np.ceil(1.5e9 / wbytes)))      # > 1.5 GB of weights: no cache holds them
    sets = [(W1, Wg, W2)] + [(W1.clone(), Wg.clone() if sw else None, W2.clone()) for _ in range(nsets - 1)]
    shape = B.make_shape(1, h, w.F, w.t, 0, w.act)
    ws = B.alloc_workspace(B.workspace_bytes(shape, False))
    Y = torch.empty(1, h, dtype=bf, device="cuda")
    A = torch.empty(1, Fi, dtype=bf, device="cuda")
    for i in range(10):
        a, g, b = sets[i % nsets]
        B.tp_mlp_fwd_shard(shape, x, a, g, b, Y, A, None, None, ws)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = args.decode_steps
    windows = []
    for _ in range(DECODE_WINDOWS):       # the median window is reported, every window listed
        e0.record(stream)
        for i in range(n):
            a, g, b = sets[i % nsets]
            B.tp_mlp_fwd_shard(shape, x, a, g, b, Y, A, None, None, ws)
        e1.record(stream)
        torch.cuda.synchronize()
        windows.append(e0.elapsed_time(e1) * 1e3 / n)
    us = float(np.median(windows))
    # warm (same weights every call) for context
    e0.record(stream)
    for i in range(n):
        B.tp_mlp_fwd_shard(shape, x, W1, Wg, W2, Y, A, None, None, ws)
    e1.record(stream)
    torch.cuda.synchronize()
    us_warm = e0.elapsed_time(e1) * 1e3 / n
    gbs = wbytes / (us * 1e-6) / 1e9
    traffic = counter_traffic(f"gemv_hbm_traffic_{w.name}.md", GEMV_SOURCES, "decode")
    log(f"[bench] decode: {us:.2f} us/token cold ({gbs:.0f} GB/s), {us_warm:.2f} us warm")
    # small-batch decode (2 <= N <= 128 takes the split-K MFMA path), same rotated weights
    small = {}
    for nb in (8, 32, 128):
        xb = to_dev(I.normal_bf16([w.wid, 40, nb], (nb, h)))
        sb = B.make_shape(nb, h, w.F, w.t, 0, w.act)
        wsb = B.alloc_workspace(B.workspace_bytes(sb, False))
        Yb = torch.empty(nb, h, dtype=bf, device="cuda")
        Ab = torch.empty(nb, Fi, dtype=bf, device="cuda")
        for i in range(10):
            a, g, b = sets[i % nsets]
            B.tp_mlp_fwd_shard(sb, xb, a, g, b, Yb, Ab, None, None, wsb)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(n):
            a, g, b = sets[i % nsets]
            B.tp_mlp_fwd_shard(sb, xb, a, g, b, Yb, Ab, None, None, wsb)
        e1.record(stream)
        torch.cuda.synchronize()
        usb = e0.elapsed_time(e1) * 1e3 / n
        small[str(nb)] = {"us_per_step": round(usb, 3), "GB/s_of_weights": round(wbytes / (usb * 1e-6) / 1e9, 1),
                          "tokens_per_s": round(nb / (usb * 1e-6), 1)}
        log(f"[bench] small-batch decode N={nb}: {usb:.2f} us ({wbytes / (usb * 1e-6) / 1e9:.0f} GB/s of weights)")
    # few-token backward (the split-K input gradients, then the weight gradients), same rotated
    # weights: bytes = the weights read once + the float32 weight gradients written once
    small_bwd = {}
    f32 = torch.float32
    dW1, dW2 = torch.empty(h, Fi, dtype=f32, device="cuda"), torch.empty(Fi, h, dtype=f32, device="cuda")
    dWg = torch.empty(h, Fi, dtype=f32, device="cuda") if sw else None
    bwd_bytes = wbytes * 3
    for nb in (8, 128):
        sb = B.make_shape(nb, h, w.F, w.t, 0, w.act)
        xb = to_dev(I.normal_bf16([w.wid, 40, nb], (nb, h)))
        dyb = to_dev(I.normal_bf16([w.wid, 43, nb], (nb, h)))
        Ab, Ub = (to_dev(I.normal_bf16([w.wid, 44 + k, nb], (nb, Fi))) for k in range(2))
        Gb = to_dev(I.normal_bf16([w.wid, 46, nb], (nb, Fi))) if sw else None
        dUb = torch.empty(nb, w.g * Fi, dtype=bf, device="cuda")
        dXb = torch.empty(nb, h, dtype=bf, device="cuda")

        def bwd(i):
            a, g, b = sets[i % nsets]
            B.tp_mlp_bwd_shard(sb, xb, a, g, b, dyb, Ab, Ub, Gb, dUb, dW1, dWg, dW2, dXb)
        for i in range(6):
            bwd(i)
        torch.cuda.synchronize()
        nbw = max(10, n // 4)
        e0.record(stream)
        for i in range(nbw):
            bwd(i)
        e1.record(stream)
        torch.cuda.synchronize()
        usb = e0.elapsed_time(e1) * 1e3 / nbw
        small_bwd[str(nb)] = {"us_per_step": round(usb, 3), "GB/s": round(bwd_bytes / (usb * 1e-6) / 1e9, 1)}
        log(f"[bench] small-batch backward N={nb}: {usb:.2f} us ({bwd_bytes / (usb * 1e-6) / 1e9:.0f} GB/s of "
            f"weights read and float32 gradients written)")
    del dW1, dW2, dWg
    return {"workload": w.name, "value": round(gbs, 1), "unit": "GB/s", "us_per_token": round(us, 3),
            "small_batch": small,
            "small_batch_backward": small_bwd,
            "small_batch_backward_bytes": bwd_bytes,
            "us_per_token_windows": [round(v, 3) for v in windows], "calls_per_window": n,
            "bytes_per_token": wbytes, "weight_sets_rotated": nsets,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": traffic["bytes"] if traffic else None,
                         "scope": "whole decode call (gate/up GEMV + down GEMV)"},
            "us_per_token_warm_cache": round(us_warm, 3)}


def bench_attn(args, B, I, torch, np, to_dev, N=2048, h=12288, heads=96, kv=96, d=128, t=8):
    """One rank's attention projections at the GPT-3-scale shape of the MLP
    workload (t = 8: 12 query heads of 128 per rank): QKV projection, output
    projection, and both backwards (dO and dW_o; dX and dW_qkv), 6 GEMMs per
    step.  The attention core between them is not part of this path."""
    bf, f32 = torch.bfloat16, torch.float32
    s = B.make_attn_shape(N, h, heads, kv, d, t, 0)
    qc, wc = s.q_cols, s.qkv_cols
    sig = I.WEIGHT_SIGMA
    X, dY = to_dev(I.normal_bf16([900, 0], (N, h))), to_dev(I.normal_bf16([900, 1], (N, h)))
    Wqkv, Wo = to_dev(I.normal_bf16([900, 2], (h, wc), sig)), to_dev(I.normal_bf16([900, 3], (qc, h), sig))
    O, dQKV = to_dev(I.normal_bf16([900, 4], (N, qc))), to_dev(I.normal_bf16([900, 5], (N, wc)))
    QKV, Y, dO = (torch.empty(N, c, dtype=bf, device="cuda") for c in (wc, h, qc))
    dWo, dWqkv = torch.empty(qc, h, dtype=f32, device="cuda"), torch.empty(h, wc, dtype=f32, device="cuda")
    dX = torch.empty(N, h, dtype=bf, device="cuda")

    ws_do = B.alloc_workspace(B.attn_out_dgrad_workspace_bytes(s))

    def step():
        B.tp_attn_qkv_shard(s, X, Wqkv, QKV)       # N > 128: no workspace
        B.tp_attn_out_shard(s, O, Wo, Y)
        # dO alone (the attention core's backward needs only it); then dX, dW_qkv
        # and the deferred dW_o in one launch
        B.tp_attn_out_dgrad_shard(s, dY, Wo, dO, workspace=ws_do)
        B.tp_attn_qkv_bwd_out_wgrad_shard(s, X, Wqkv, dQKV, dY, O, dWqkv, dX, dWo)
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 10
    e0.record(stream)
    for _ in range(n):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    flops = 3 * 2 * N * h * (wc + qc)
    tf = flops / (ms * 1e-3) / 1e12
    log(f"[bench] attention projections gpt3 t=8: {ms:.3f} ms/step, {tf:.1f} TFLOP/s")
    small = bench_attn_small(B, I, torch, to_dev)
    return {"small_batch_llama3_70b_t4": small,"workload": f"gpt3_attn_t{t}: N={N} h={h} heads={heads} head_dim={d} t={t} (qkv {wc}, o {qc} cols/rank)",
            "ms_per_step": round(ms, 4), "TFLOP/s": round(tf, 1), "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "flops_per_step": flops,
            "step": "QKV fwd, O fwd, dO (k-split), then dX + dW_qkv + dW_o (the output projection's weight "
                    "gradient deferred into the QKV backward's launch)"}


def graph_time(torch, calls, windows=5):
    """Microseconds per call of `calls` (closures enqueuing library calls on
    the current stream), captured into one HIP graph on a side stream and
    replayed: the GPU time of launch-bound sequences without the host's
    per-call launch overhead (what a caller that captures its loop sees).
    The median over `windows` replays, after one untimed replay."""
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        for c in calls[:3]:
            c()
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for c in calls:
            c()
    torch.cuda.synchronize()
    ts = []
    for _ in range(windows + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(s):
            e0.record(s)
            g.replay()
            e1.record(s)
        s.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e3 / len(calls))
    del g
    return float(sorted(ts[1:])[len(ts[1:]) // 2])


def bench_attn_small(B, I, torch, to_dev, h=8192, heads=64, kv=8, d=128, t=4):
    """The forward attention projections (QKV and output) of one rank of the
    70B block at decode batches of 8 and 32 tokens: the small-batch path,
    HBM bound on the weights (Wqkv_i + Wo_i), rotated over 5 copies so no
    cache holds them.  GB/s of weights."""
    bf = torch.bfloat16
    s0 = B.make_attn_shape(8, h, heads, kv, d, t, 0)
    qc, wc = s0.q_cols, s0.qkv_cols
    sig = I.WEIGHT_SIGMA
    Wqkv = to_dev(I.normal_bf16([901, 2], (h, wc), sig))
    Wo = to_dev(I.normal_bf16([901, 3], (qc, h), sig))
    sets = [(Wqkv, Wo)] + [(Wqkv.clone(), Wo.clone()) for _ in range(4)]
    wbytes = (h * wc + qc * h) * 2
    out = {}
    for N in (8, 32):
        s = B.make_attn_shape(N, h, heads, kv, d, t, 0)
        X, O = to_dev(I.normal_bf16([901, 0, N], (N, h))), to_dev(I.normal_bf16([901, 4, N], (N, qc)))
        QKV, Y = torch.empty(N, wc, dtype=bf, device="cuda"), torch.empty(N, h, dtype=bf, device="cuda")
        ws = B.alloc_workspace(B.attn_workspace_bytes(s))

        def step(i):
            a, b = sets[i % len(sets)]
            B.tp_attn_qkv_shard(s, X, a, QKV, workspace=ws)
            B.tp_attn_out_shard(s, O, b, Y, workspace=ws)
        for i in range(10):
            step(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        n = 100
        e0.record(torch.cuda.current_stream())
        for i in range(n):
            step(i)
        e1.record(torch.cuda.current_stream())
        torch.cuda.synchronize()
        us_eager = e0.elapsed_time(e1) * 1e3 / n
        us = graph_time(torch, [lambda i=i: step(i) for i in range(n)])
        out[str(N)] = {"us_per_step": round(us, 2), "GB/s_of_weights": round(wbytes / (us * 1e-6) / 1e9, 1),
                       "frac_of_hbm_peak": round(wbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                       "us_per_step_eager": round(us_eager, 2)}
        log(f"[bench] attention projections 70b t=4, N={N}: {us:.1f} us ({wbytes / (us * 1e-6) / 1e9:.0f} GB/s of "
            f"weights; {us_eager:.1f} us launched one call at a time)")
    out["weight_bytes"] = wbytes
    out["step"] = ("QKV projection + output projection forward (small-batch path), weights rotated over 5 copies; "
                   "us_per_step from 100 steps captured into a HIP graph and replayed, us_per_step_eager with "
                   "each call launched from the host")
    return out


def bench_ln(B, I, torch, to_dev, name, N, h, t):
    """One rank's sequence-parallel LayerNorm: the fused reduce-scatter +
    bias + residual + LayerNorm forward over its N/t rows (reading its block
    of all t partial sums), and the LayerNorm backward with the residual
    branch's gradient, dgamma and dbeta.  GB/s on algorithmic bytes (every
    operand read once, every output written once); the calls are timed as 20
    captured into a HIP graph and replayed (`us`), and launched one at a time
    from the host (`us_eager`)."""
    bf, f32 = torch.bfloat16, torch.float32
    n = N // t
    parts = [to_dev(I.normal_bf16([990, 1, k], (N, h))) for k in range(t)]
    res, dy, dres = (to_dev(I.normal_bf16([990, j], (n, h))) for j in (2, 3, 4))
    bias, g, beta = to_dev(I.gen_b2(990, h)), to_dev(I.gen_ln_weight(990, h)), to_dev(I.gen_ln_bias(990, h))
    z, y, dx = (torch.empty(n, h, dtype=bf, device="cuda") for _ in range(3))
    mean, rstd = torch.empty(n, dtype=f32, device="cuda"), torch.empty(n, dtype=f32, device="cuda")
    dg, db = torch.empty(h, dtype=f32, device="cuda"), torch.empty(h, dtype=f32, device="cuda")
    ws = B.alloc_workspace(B.layernorm_bwd_workspace_bytes(n, h))

    def fwd():
        B.tp_sp_reduce_scatter_layernorm_local(parts, t - 1, z, g, y, bias=bias, residual=res, beta=beta, mean=mean,
                                               rstd=rstd)

    def bwd():
        B.tp_sp_layernorm_bwd(z, g, mean, rstd, dy, dx, dg, dbeta=db, dres=dres, workspace=ws)

    stream = torch.cuda.current_stream()
    out = {}
    nbytes = {"fwd": (t + 4) * n * h * 2 + 3 * h * 2 + 8 * n,     # t partial blocks, residual in; z, y out
              "bwd": 4 * n * h * 2 + h * 2 + 8 * n + 2 * h * 4}   # z, dy, dres in; dx out
    for key, fn in (("fwd", fwd), ("bwd", bwd)):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 20
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        us_eager = e0.elapsed_time(e1) * 1e3 / reps
        us = graph_time(torch, [fn] * reps)
        gbs = nbytes[key] / (us * 1e-6) / 1e9
        out[key] = {"us": round(us, 2), "GB/s": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                    "algorithmic_bytes": nbytes[key], "us_eager": round(us_eager, 2)}
    log(f"[bench] sp layernorm {name}: fused rs+ln fwd {out['fwd']['us']:.1f} us ({out['fwd']['GB/s']:.0f} GB/s), "
        f"bwd {out['bwd']['us']:.1f} us ({out['bwd']['GB/s']:.0f} GB/s); launched one call at a time "
        f"{out['fwd']['us_eager']:.1f} / {out['bwd']['us_eager']:.1f} us")
    out["workload"] = f"{name}: {N} tokens, h={h}, t={t}: {n} rows per rank"
    out["fwd"]["step"] = "reduce-scatter of t partials + bias + residual -> z, LayerNorm(z) -> y (one kernel)"
    out["bwd"]["step"] = "LayerNorm backward + residual gradient -> dx; dgamma, dbeta (row kernel + slab sums)"
    return out


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo (None where absent)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max(int(p.get("num_threads", 1)) for p in threadpool_info() if p.get("user_api") == "blas")
    except Exception:
        return os.cpu_count()


# Token rows of rank 0's shard the oracle is timed on: every row (None) for
# the four smaller workloads; a stated quarter of the 70B prefill shard (its
# full run is about 17 TFLOP of float64, some 20 s on 16 host threads).
CPU_ORACLE_ROWS = {"mlp128_h1024_gelu_t2": None, "llama3_70b_decode_t4": None, "llama_7b_train_t2": None,
                   "gpt3_train_t8": None, "llama3_70b_prefill_t4": 4096}


def cpu_oracle_workload(w, rows, I, min_s=1.0):
    """The fp64 oracle (as it stands) on rank 0's shard of workload w: the
    forward (+ backward for the training workloads) over the first `rows`
    token rows (all of them when None), on the host's BLAS threads, repeated
    until at least min_s seconds have run; the time per pass is reported."""
    import numpy as np

    import oracle
    f = oracle.bf16_bits_to_f64
    sw = w.act == "swiglu"
    n = w.N if rows is None else min(rows, w.N)
    X = f(I.gen_x(w.wid, w.N, w.h)[:n])
    dY = f(I.gen_dy(w.wid, w.N, w.h)[:n]) if w.backward else None
    W1 = f(I.gen_w_up_shard(w.wid, w.h, w.Fi, 0))
    W2 = f(I.gen_w_down_shard(w.wid, w.h, w.Fi, 0))
    Wg = f(I.gen_w_gate_shard(w.wid, w.h, w.Fi, 0)) if sw else None
    dt, reps = 0.0, 0
    while dt < min_s:
        t0 = time.perf_counter()
        oracle.shard_forward(w.act, X, W1, W2, Wg)
        if w.backward:
            oracle.shard_backward(w.act, X, W1, W2, dY, Wg)
        dt += time.perf_counter() - t0
        reps += 1
    sec = dt / reps
    fl = (6 if w.backward else 2) * n * w.h * w.Fi * (w.g + 1)
    out = {"seconds_per_pass": round(sec, 4), "passes": reps, "token_rows": n, "full_run": n == w.N,
           "flops_per_pass": fl, "TFLOP/s": round(fl / sec / 1e12, 5)}
    if not w.backward:
        out["us_per_token"] = round(sec / n * 1e6, 1)
        out["GB/s_of_weights"] = round(w.weight_bytes() / (sec / n) / 1e9, 3)
    return out


def cpu_baseline(w, I, names, gpu):
    """The fp64 oracle timed on the host cores, per workload (rank 0's shard;
    a full run where CPU_ORACLE_ROWS says so, else the stated sample), beside
    the GPU's figure for the same workload.  The top-level value is the
    headline workload's."""
    from megatron_tensor_transformer_rank_amd.configs import WORKLOADS
    cores = blas_threads()
    per = {}
    for name in names:
        ww = WORKLOADS[name]
        log(f"[bench] cpu baseline: oracle on {name} ({'all' if CPU_ORACLE_ROWS[name] is None else CPU_ORACLE_ROWS[name]} "
            f"token rows), {cores} BLAS threads")
        r = cpu_oracle_workload(ww, CPU_ORACLE_ROWS[name], I)
        g = gpu.get(name)
        if g is not None:
            r["gpu"] = g
            key = "GB/s_of_weights" if not ww.backward else "TFLOP/s"
            if key in g and r.get(key):
                r["gpu_over_cpu"] = round(g[key] / r[key], 1)
        per[name] = r
    head = per[w.name]
    return {"value": head["TFLOP/s"], "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(), "full_run": head["full_run"], "seconds": head["seconds_per_pass"],
            "sample": f"{'all ' if head['full_run'] else ''}{head['token_rows']} token rows of rank 0's shard of {w.name}, "
                      f"forward + backward, {head['flops_per_pass']:.3e} algorithmic FLOPs per pass; numpy float64 "
                      f"on the host BLAS; per_workload gives every workload (full runs except where stated)",
            "per_workload": per}


if __name__ == "__main__":
    main()
