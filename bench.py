"""MoE-layer throughput on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 10] [--workload deepseek_v3_large]
                    [--dist ...] [--no-backward] [--no-extra] [--no-flush] [--no-cpu-baseline]

One step = one pass of the whole single-GPU layer over one batch of seeded
synthetic input already resident in HBM:

    moe_route -> moe_layout -> moe_grouped_gate_up_gather -> moe_grouped_down -> moe_combine

(the permute fused into the gate/up GEMM's row loads; moe_permute on its own is
timed with the calls outside the step). The default workload is the large DeepSeek-V3-shaped layer (65536 tokens,
hidden 7168, 256 experts all local, top-8, intermediate 2048, bf16, severe
skew), the largest that fits one GPU. Prints ONE JSON line (everything else
goes to stderr):
  value        tokens/s of the layer, steps run back to back (for an EP share:
               the share's own tokens per rank, T/ep, per step)
  roofline     the dominant kernel's algorithmic FLOP/s (or bytes/s) per launch over
               its average launch time, measured with HIP events on the stream the
               library launches on, against the MI355X datasheet peak
  stages       the same per stage (back to back, as inside a model)
  stages_cold  the same per stage from a cold cache: a 512 MB buffer is read and
               written before every stage, outside its events
               (both also carry permute_alone: moe_permute timed on its own on the
               same routing, since the step fuses the permute into gate/up)
  backward     the training and variant calls, each timed on its own
  extra        the one-GPU share of the DeepSeek-V3 EP=8 layer (balanced
               routing) as its own step, and the combine alone at the large
               DeepSeek-V3 shape ([T*8, H] expert rows, no padding), warm and cold
  cpu_baseline the CPU oracle timed on a bounded sample of the same workload
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
PEAK_BF16_TFLOPS = 2516.6  # dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz (the 2.5 PF figure)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="deepseek_v3_large")
    ap.add_argument("--dist", default=None)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip timing the backward calls")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the extra workloads (the DeepSeek-V3 EP=8 share and the "
                         "combine-only case)")
    ap.add_argument("--no-flush", action="store_true",
                    help="skip the per-stage timing from a cold cache (a 512 MB buffer "
                         "read and written before every stage, outside its events)")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the CPU baseline sample")
    ap.add_argument("--layout-sweep", action="store_true",
                    help="only time the layout stage alone from 64 K to 64 M assignments "
                         "(256 experts, top-8, all local) and exit")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (the reference "
                         "kernel for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE readings) and exit")
    return ap.parse_args()


def calibrate_copy(mib: int):
    """A plain device-to-device copy of known size: its FETCH_SIZE and WRITE_SIZE
    readings (KiB per dispatch) against the true mib*1024 KiB give the factor that
    turns the counters into HBM bytes."""
    import torch
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "launches": 5}), flush=True)


def roof_entry(ms: float, bound: str, amount) -> dict:
    """Achieved rate of one stage against its roofline. HBM stages carry their
    algorithmic bytes. GEMM stages carry (flops, bytes), bytes being the least
    traffic the product needs (each weight of an expert with rows read once,
    activations read once, outputs written once): the binding ceiling is the
    lower of the MFMA peak and intensity x HBM peak, so a product below the
    ridge point (2516.6 TFLOP/s / 8 TB/s = 315 flop/byte) is HBM-bound."""
    sec = ms * 1e-3
    if bound == "hbm":
        ach = amount / sec / 1e9
        return {"ms": round(ms, 4), "bound": "hbm", "GB/s": round(ach, 1),
                "frac": round(ach / PEAK_HBM_GBS, 4), "bytes": int(amount)}
    flops, nbytes = amount
    tf, gbs = flops / sec / 1e12, nbytes / sec / 1e9
    intensity = flops / nbytes
    out = {"ms": round(ms, 4), "TFLOP/s": round(tf, 1), "GB/s": round(gbs, 1),
           "flops": flops, "bytes": int(nbytes), "flop_per_byte": round(intensity, 1),
           "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
    if intensity * PEAK_HBM_GBS * 1e9 >= PEAK_BF16_TFLOPS * 1e12:
        out.update(bound="mfma", frac=round(tf / PEAK_BF16_TFLOPS, 4))
    else:
        out.update(bound="hbm", frac=round(gbs / PEAK_HBM_GBS, 4))
    return out


# the sources a grouped-GEMM kernel is built from (its counters are tied to them)
GEMM_SOURCES = ("grouped_gemm.hip", "moe_internal.h")


def source_hash(*paths: str) -> str:
    """First 16 hex digits of the sha256 of the source files' code, in order:
    comment-only and blank lines are dropped and trailing comments stripped,
    so a comment edit keeps counters taken on the same code valid."""
    import hashlib
    import re
    lines = []
    for path in paths:
        for line in open(path, encoding="utf-8"):
            code = re.sub(r"//.*$", "", line).rstrip()
            if code.strip():
                lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]


def gemm_source_hash() -> str:
    return source_hash(*(os.path.join(ROOT, "combine_top_router_amd", "csrc", f)
                         for f in GEMM_SOURCES))


def traffic_record(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if line.startswith("- ") and ":" in line:
            k, v = line[2:].split(":", 1)
            rec[k.strip()] = v.strip().strip("`")
    if rec.get("source_sha256_16") != gemm_source_hash() or "hbm_bytes_per_launch" not in rec:
        return None
    return float(rec["hbm_bytes_per_launch"])


def cpu_baseline(cfg, dist, layer_args, budget_s):
    """The oracle, as it stands, on the first S tokens of the same workload."""
    import numpy as np
    import torch
    import threadpoolctl

    from oracle import bf16 as obf16, layer as olayer, route as oroute

    x, logits, w1, w3, w2, share = layer_args
    ep = cfg.ep_size
    dec = lambda t: obf16.decode(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))  # noqa: E731
    logits_np = logits.cpu().numpy()
    first = cfg.local_experts(share)[0]
    cache = {}

    def weights_for(tokens):
        idx, _ = oroute.route(logits_np[:tokens], cfg.top_k)
        need = sorted({int(e) - first for e in np.unique(idx)
                       if 0 <= int(e) - first < len(cfg.local_experts(share))})
        for e in need:
            if e not in cache:
                cache[e] = (dec(w1[e]), dec(w3[e]), dec(w2[e]))
        return need

    def run(tokens):
        weights_for(tokens)  # decoding the bf16 weights is not oracle work: untimed
        xs = dec(x[:tokens])
        t0 = time.perf_counter()
        olayer.layer(xs, logits_np[:tokens], cfg.top_k, lambda e: cache[e], cfg.num_experts,
                     ep, share, cfg.align)
        return time.perf_counter() - t0

    per_expert_bytes = 3 * cfg.hidden * cfg.inter * 8
    max_experts = max(1, int(48e9 // per_expert_bytes))
    s = ep * max(1, 32 // ep)
    t = run(s)
    while t < budget_s / 8 and s < cfg.num_tokens:
        s = min(cfg.num_tokens, s * 4)
        if len(weights_for(s)) > max_experts:
            s //= 4
            break
        t = run(s)
    target = int(s * budget_s / max(t, 1e-3)) // ep * ep
    target = max(ep, min(cfg.num_tokens, target))
    while target > s and len(weights_for(target)) > max_experts:
        target = max(s, target // 2 // ep * ep)
    if target != s:
        s, t = target, run(target)
    # a sample capped by host memory (the fp64 weights of the experts it
    # touches) finishes early: repeat it until the budget is spent, report the mean
    reps = 1
    total = t
    while total < budget_s * 0.75:
        total += run(s)
        reps += 1
    t = total / reps
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    per_rank = s // ep
    return {"value": per_rank / t, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": (f"first {s} of {cfg.num_tokens} tokens ({per_rank} per rank), whole oracle "
                       f"layer (route, layout, permute, fp64 SwiGLU experts, fp64 combine), "
                       f"{t:.2f} s per run, mean of {reps} run(s), numpy BLAS threads {threads}, "
                       f"{len(os.sched_getaffinity(0))} host cores visible")}


def time_backward(args, cfg, layer, moe, stream, t_loc, n_loc, weights, x):
    """Per-call times of the calls outside the step, on this step's routing
    and rows, after the forward timing (not part of ``value``): the permute on
    its own, the forward gate/up that also keeps the pre-activations, then the
    backward chain
    combine -> routing -> down -> gate/up (data and weight gradients) ->
    permute, each call fed by the one before it, and the per-rank
    deduplicated dispatch layout."""
    import numpy as np
    import torch

    import workloads

    T, H, E, k, I = cfg.num_tokens, cfg.hidden, cfg.num_experts, cfg.top_k, cfg.inter
    dev = layer.y.device
    w1, w3, w2 = weights
    L = layer.L
    e_loc = w1.shape[0]
    G = workloads.gen.output_gradient(cfg, args.seed, device=dev)
    gy = torch.zeros_like(layer.y)
    gw = torch.empty((T, k), dtype=torch.float32, device=dev)
    gl = torch.empty((T, E), dtype=torch.float32, device=dev)
    gu = torch.empty((layer.m_cap, 2 * I), dtype=torch.bfloat16, device=dev)
    dgu = torch.empty_like(gu)
    dxp = torch.empty_like(layer.x_perm)
    gx = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    dw1 = torch.empty((e_loc, H, I), dtype=torch.bfloat16, device=dev)
    dw3 = torch.empty_like(dw1)
    dw2 = torch.empty((e_loc, I, H), dtype=torch.bfloat16, device=dev)
    dst, off, cnt = L.dst_row, L.offsets, L.local_counts
    dl_ep = max(cfg.ep_size, 8) if E % max(cfg.ep_size, 8) == 0 else cfg.ep_size
    sh = workloads.gen.random_rows(cfg, T, torch.bfloat16, args.seed, device=dev)
    n_grp = int(off[-1].item())  # rows of the expert groups, padding included
    nhi = float(n_loc) * H * I
    e_act = int((L.local_counts > 0).sum().item())
    wbytes = float(e_act) * H * I * 2  # one expert matrix of each active expert
    calls = [
        # the permute on its own (in the layer it is fused into gate/up's loads);
        # it also fills x_perm, which the training calls below read
        ("permute", lambda: moe.ops.permute(x, dst, L.src_row, off, layer.m_cap,
                                            out=layer.x_perm),
         "hbm", (t_loc + n_grp) * H * 2 + n_grp * 4),
        ("gate_up_save", lambda: moe.ops.grouped_gate_up_save(
            layer.x_perm, off, cnt, layer.w1t, layer.w3t, layer.h, gu), "gemm",
         (4 * nhi, 2 * wbytes + n_loc * (H + I + 2 * I) * 2)),
        ("combine_backward", lambda: moe.ops.combine_backward(G, layer.y, dst, layer.topk_w, gy, gw),
         "hbm", t_loc * H * 2 + 2 * n_loc * H * 2 + T * k * 12),
        ("route_backward", lambda: moe.ops.route_backward(layer.topk_idx, layer.topk_w, gw, E, gl),
         "hbm", T * E * 4 + T * k * 12),
        ("down_backward", lambda: moe.ops.grouped_down_backward(gy, gu, off, cnt, w2, dgu),
         "gemm", (2 * nhi, wbytes + n_loc * (H + 4 * I) * 2)),
        ("down_wgrad", lambda: moe.ops.grouped_down_wgrad(layer.h, gy, off, cnt, dw2),
         "gemm", (2 * nhi, float(e_loc) * H * I * 2 + n_loc * (I + H) * 2)),
        ("gate_up_backward", lambda: moe.ops.grouped_gate_up_backward(dgu, off, cnt, w1, w3, dxp),
         "gemm", (4 * nhi, 2 * wbytes + n_loc * (2 * I + H) * 2)),
        ("gate_up_wgrad", lambda: moe.ops.grouped_gate_up_wgrad(layer.x_perm, dgu, off, cnt, dw1, dw3),
         "gemm", (4 * nhi, 2 * float(e_loc) * H * I * 2 + n_loc * (H + 2 * I) * 2)),
        ("permute_backward", lambda: moe.ops.permute_backward(dxp, dst, gx),
         "hbm", n_loc * H * 2 + T * H * 2 + T * k * 4),
        # restore variants: the shared expert's rows merged, and the permute
        # that applies the score before the experts
        ("combine_shared", lambda: moe.ops.combine_rows(layer.y, dst, layer.topk_w, sh, gx),
         "hbm", n_loc * H * 2 + T * k * 8 + 2 * T * H * 2),
        ("permute_weighted", lambda: moe.ops.permute_weighted(x, dst, layer.topk_w,
                                                              layer.m_cap, dxp),
         "hbm", (t_loc + n_loc) * H * 2 + T * k * 8),
        # the per-rank deduplicated layout (over the workload's ep virtual
        # ranks, at least 8): T*k ids read, the [T, ep] table and positions written
        ("dispatch_layout", lambda: moe.ops.dispatch_layout(layer.topk_idx, E, dl_ep),
         "hbm", T * k * 4 + T * dl_ep * 5),
    ]
    reps = max(3, args.steps)
    out = {}
    for name, run, bound, amount in calls:
        for _ in range(3):
            run()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        # a short device-side wait first, so the calls queue up behind it and
        # the events time the GPU, not the host's launch rate
        torch.cuda._sleep(4_000_000)
        ev[0].record(stream)
        for r in range(reps):
            run()
            ev[r + 1].record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([ev[r].elapsed_time(ev[r + 1]) for r in range(reps)]))
        out[name] = roof_entry(ms, bound, amount)
    return out


FLUSH_BYTES = 512 << 20  # twice the 256 MB last-level cache


class Flusher:
    """Reads and writes a 512 MB buffer: after it, nothing a stage touched
    before is left in the L2s or the last-level cache."""

    def __init__(self, dev):
        import torch
        self.buf = torch.zeros(FLUSH_BYTES // 4, dtype=torch.int32, device=dev)

    def __call__(self):
        self.buf.add_(1)


def layer_work(cfg, layer):
    """Algorithmic bytes (HBM stages) and (flops, bytes) (GEMM stages) of one
    step on this batch's routing, read once outside any timed region."""
    import numpy as np
    counts = layer.L.local_counts.cpu().numpy().astype(np.int64)
    dst = layer.L.dst_row.cpu().numpy()
    n_loc = int(counts.sum())
    t_loc = int((dst >= 0).any(axis=1).sum())
    n_grp = int(layer.L.offsets[-1].item())  # rows of the expert groups, padding included
    e_act = int((counts > 0).sum())
    T, H, I, E, k = cfg.num_tokens, cfg.hidden, cfg.inter, cfg.num_experts, cfg.top_k
    N = T * k
    wbytes = float(e_act) * H * I * 2  # one expert matrix of each active expert
    work = {
        "route": ("hbm", T * E * 4 + N * 8),
        "layout": ("hbm", N * 4 * 2 + n_loc * 4),
        # token rows read once, local rows written, padding rows zeroed, src_row read
        "permute": ("hbm", (t_loc + n_grp) * H * 2 + n_grp * 4),
        "gate_up": ("gemm", (4.0 * n_loc * H * I, 2 * wbytes + n_loc * (H + I) * 2)),
        "down": ("gemm", (2.0 * n_loc * H * I, wbytes + n_loc * (I + H) * 2)),
        "combine": ("hbm", n_loc * H * 2 + N * 8 + T * H * 2),
    }
    return work, n_loc, t_loc


def stage_times(stages, stream, n, flush=None):
    """Mean time of each stage over n steps, an event between every two
    stages. With ``flush``, the caches are flushed before every stage, outside
    its events: the stage then starts from a cold cache."""
    import numpy as np
    import torch
    n_st = len(stages)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * n_st)] for _ in range(n)]
    for s in range(n):
        for i, (_, run) in enumerate(stages):
            if flush is not None:
                flush()
            evs[s][2 * i].record(stream)
            run()
            evs[s][2 * i + 1].record(stream)
    torch.cuda.synchronize()
    return {name: float(np.mean([evs[s][2 * i].elapsed_time(evs[s][2 * i + 1])
                                 for s in range(n)]))
            for i, (name, _) in enumerate(stages)}


def run_layer(cfg, dist, args, dev, flush):
    """Builds the layer on seeded inputs and times it. Returns the record
    parts and what the CPU baseline and the backward timing need."""
    import numpy as np
    import torch

    import combine_top_router_amd as moe
    import workloads

    share = cfg.local_rank
    log(f"workload {cfg.name} dist {dist} share {share}: generating inputs")
    x, logits = workloads.gen.routing_inputs(cfg, dist, args.seed, device=dev)
    w1, w3, w2 = workloads.gen.expert_weights(cfg, cfg.local_experts(share), args.seed, device=dev)
    layer = moe.MoELayer(cfg.num_tokens, cfg.hidden, cfg.num_experts, cfg.top_k, cfg.inter,
                         w1, w3, w2, cfg.ep_size, share, cfg.align)
    stages = layer.stages(x, logits)
    stream = torch.cuda.current_stream(dev)

    wev = [torch.cuda.Event(enable_timing=True) for _ in range(args.warmup + 1)]
    wev[0].record(stream)
    for w in range(args.warmup):
        for _, run in stages:
            run()
        wev[w + 1].record(stream)
    torch.cuda.synchronize()
    if args.warmup:
        ws = [wev[i].elapsed_time(wev[i + 1]) for i in range(args.warmup)]
        log("warmup step ms: first %.3f, last %.3f, min %.3f" % (ws[0], ws[-1], min(ws)))

    work, n_loc, t_loc = layer_work(cfg, layer)
    n_st = len(stages)

    # the dominant stage, from untimed steps; the timed steps record events only
    # around it (an event between every two stages adds GPU time to each step)
    probe = stage_times(stages, stream, 3)
    dom_i = max(range(n_st), key=lambda i: probe[stages[i][0]])
    dom = stages[dom_i][0]
    dev_ = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        for i, (_, run) in enumerate(stages):
            if i == dom_i:
                dev_[s][0].record(stream)
                run()
                dev_[s][1].record(stream)
            else:
                run()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    dom_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in dev_]))

    # the other stages' times from as many steps again, after the timed region
    stage_ms = stage_times(stages, stream, args.steps)
    stage_ms[dom] = dom_ms
    out = {
        "value": cfg.num_tokens // cfg.ep_size * args.steps / elapsed,
        "ms_per_step": elapsed / args.steps * 1e3,
        "dom": dom,
        "local_rows": n_loc,
        "stages": {name: roof_entry(ms, *work[name]) for name, ms in stage_ms.items()},
    }
    if flush is not None:
        cold = stage_times(stages, stream, args.steps, flush)
        out["stages_cold"] = {name: roof_entry(ms, *work[name]) for name, ms in cold.items()}
    if not any(name == "permute" for name, _ in stages):
        # the permute is fused into gate/up in the step; time moe_permute on its
        # own as well, on the same routing (not part of the step)
        alone = [("permute", lambda: moe.ops.permute(x, layer.L.dst_row, layer.L.src_row,
                                                      layer.L.offsets, layer.m_cap,
                                                      out=layer.x_perm))]
        ms = stage_times(alone, stream, args.steps)["permute"]
        out["stages"]["permute_alone"] = roof_entry(ms, *work["permute"])
        if flush is not None:
            ms = stage_times(alone, stream, args.steps, flush)["permute"]
            out["stages_cold"]["permute_alone"] = roof_entry(ms, *work["permute"])
    return out, (layer, x, logits, (w1, w3, w2), stream, t_loc, n_loc)


def roofline_of(cfg, stage_out, dom):
    d = stage_out[dom]
    traffic = traffic_record(dom, cfg.name) if dom in ("gate_up", "down") else None
    if d["bound"] == "mfma":
        return {"bound": "mfma", "kernel": dom, "achieved": d["TFLOP/s"],
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": d["frac"],
                "traffic": traffic}
    return {"bound": "hbm", "kernel": dom, "achieved": d["GB/s"], "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": d["frac"], "traffic": traffic}


def combine_only(cfg, args, dev, flush):
    """The fused restore on its own at this workload's routing: expert outputs
    [T*k, H] bf16 in expert order with no padding (alignment 1), N(0, 1), into
    [T, H]; timed back to back and from a cold cache."""
    import numpy as np
    import torch

    import combine_top_router_amd as moe
    import workloads

    T, H, k = cfg.num_tokens, cfg.hidden, cfg.top_k
    _, logits = workloads.gen.routing_inputs(cfg, cfg.dists[0], args.seed, device=dev)
    idx, w = moe.route(logits, k)
    L = moe.layout(idx, cfg.num_experts, 1, -1, 1)
    del logits
    y = workloads.gen.expert_outputs(cfg, T * k, seed=7, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    run = lambda: moe.ops.combine(y, L.dst_row, w, out=out)  # noqa: E731
    for _ in range(3):
        run()
    nbytes = T * k * H * 2 + T * k * 8 + T * H * 2
    rec = {"shape": f"y [{T * k}, {H}] bf16, alignment 1 -> out [{T}, {H}]",
           "bytes": nbytes}
    for name, fl in (("warm", None), ("cold", flush)):
        if name == "cold" and fl is None:
            continue
        ms = stage_times([("combine", run)], stream, max(args.steps, 5), fl)["combine"]
        rec[name] = roof_entry(ms, "hbm", nbytes)
    del y, out, L
    return rec


def layout_sweep(args):
    """The layout stage on its own at growing sizes: T*8 assignments over 256
    experts (top-8, softmax routing of N(0, 1) logits, every expert local,
    alignment 128), 64 K to 64 M assignments. Each point: the mean of 20 calls
    back to back, priced on the layout's algorithmic bytes (the expert ids
    read once, dst_row and src_row written once)."""
    import numpy as np
    import torch

    import combine_top_router_amd as moe

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    E, k, reps = 256, 8, 20
    points = []
    for n in [1 << p for p in range(16, 27, 2)]:
        T = n // k
        g = torch.Generator(device=dev)
        g.manual_seed(n)
        logits = torch.randn((T, E), generator=g, device=dev)
        idx, _ = moe.route(logits, k)
        del logits
        L = moe.layout(idx, E, 1, -1, 128)
        for _ in range(3):
            moe.layout(idx, E, 1, -1, 128, out=L)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(stream)
        for r in range(reps):
            moe.layout(idx, E, 1, -1, 128, out=L)
            ev[r + 1].record(stream)
        torch.cuda.synchronize()
        ms = float(np.mean([ev[r].elapsed_time(ev[r + 1]) for r in range(reps)]))
        nbytes = n * 4 * 2 + n * 4
        points.append({"assignments": n, "tokens": T, "us": round(ms * 1e3, 2),
                       "bytes": nbytes, "GB/s": round(nbytes / ms / 1e6, 1),
                       "frac": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4)})
        log(f"layout {n} assignments: {ms * 1e3:.1f} us")
        del idx, L
        torch.cuda.empty_cache()
    print(json.dumps({"layout_sweep": points, "experts": E, "top_k": k, "align": 128}),
          flush=True)


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.layout_sweep:
        layout_sweep(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): it measures one "
              "GPU's share of the layer; sharding across GPUs is not implemented.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import combine_top_router_amd as moe
    import workloads

    cfg = workloads.get(args.workload)
    dist = args.dist or cfg.dists[0]
    share = cfg.local_rank
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    flush = None if args.no_flush else Flusher(dev)

    head, (layer, x, logits, weights, stream, t_loc, n_loc) = run_layer(cfg, dist, args, dev,
                                                                        flush)
    roof = roofline_of(cfg, head["stages"], head["dom"])
    backward = None if args.no_backward else time_backward(args, cfg, layer, moe, stream,
                                                            t_loc, n_loc, weights, x)
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(cfg, dist, (x, logits) + tuple(weights) + (share,), args.cpu_budget)
    del layer, x, logits, weights
    torch.cuda.empty_cache()

    extra = {}
    if not args.no_extra:
        # the one-GPU share of the DeepSeek-V3 EP=8 layer, balanced routing
        if cfg.name != "deepseek_v3_ep8_share":
            c4 = workloads.get("deepseek_v3_ep8_share")
            rec, parts = run_layer(c4, "balanced", args, dev, flush)
            del parts
            torch.cuda.empty_cache()
            extra["deepseek_v3_ep8_share"] = {
                "value": round(rec["value"], 1), "unit": "tokens/s per GPU (1024 tokens per rank)",
                "ms_per_step": round(rec["ms_per_step"], 4), "routing": "balanced",
                "local_rows": rec["local_rows"], "roofline": roofline_of(c4, rec["stages"], rec["dom"]),
                "stages": rec["stages"], "stages_cold": rec.get("stages_cold")}
        # the restore alone at the large DeepSeek-V3 shape
        big = workloads.get("deepseek_v3_large")
        extra["combine_only_deepseek_v3_large"] = combine_only(big, args, dev, flush)
        torch.cuda.empty_cache()

    rec = {
        "metric": "MoE layer tokens/s on 1 MI355X; % HBM roofline (perm/combine), % MFMA (GEMM)",
        "value": round(head["value"], 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(head["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": cfg.num_tokens, "hidden": cfg.hidden,
                   "experts": cfg.num_experts, "local_experts": len(cfg.local_experts(share)),
                   "top_k": cfg.top_k, "inter": cfg.inter, "ep_size": cfg.ep_size,
                   "local_rank": share, "align": cfg.align, "routing": dist,
                   "local_rows": head["local_rows"], "seed": args.seed,
                   "permute": "fused into the gate/up GEMM's row loads"},
        "roofline": roof, "stages": head["stages"], "stages_cold": head.get("stages_cold"),
        "backward": backward, "extra": extra or None, "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
