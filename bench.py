#!/usr/bin/env python3
"""Benchmark: latent tokens/s inverted by video-aware block-wise Jacobi on one
MI355X, with the roofline of the dominant kernel and the CPU oracle beside it.

    python bench.py [--steps K] [--warmup W] [--workload frame480p]

A step is one af_inverse_jacobi call over one batch of synthetic latents
(every kernel of the hot path: shift+embed, LayerNorm, QKV/O/MLP GEMMs,
attention over the KV cache, head, fused affine/residual kernel, host stop
test).  Inputs are resident in HBM before timing.  Prints ONE JSON line.

Workloads (autoregressive_normalizing_flow_amd.synth.WORKLOADS):
  frame480p      one 1560-token frame, 8 layers d=1024, B=1560   (default)
  video21        21 frames, block = frame, previous-frame warm start
  shallow_stack  T=4 alternating blocks, 2 layers d=512, 21 frames batched
  wide_prefix    4 layers d=4096, 2-frame prefix, batch 2
  tiny_f32       one 8x8 frame, fp32
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6    # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3      # MI355X fp32 (vector / matrix)
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
METRIC = "latent tokens/s inverted via block Jacobi (1 GPU); % MFMA/HBM peak; iters/blk"
GEMM_CLASSES = ("gemm_qkv", "gemm_o", "gemm_mlp1", "gemm_mlp2", "gemm_head")
ALL_CLASSES = GEMM_CLASSES + ("attention", "layernorm", "embed", "affine")


def gemm_flops_per_launch(cls, M, cfg):
    d, C = cfg.d, cfg.C
    return {"gemm_qkv": 2 * M * 3 * d * d, "gemm_o": 2 * M * d * d,
            "gemm_mlp1": 2 * M * 4 * d * d, "gemm_mlp2": 2 * M * d * 4 * d,
            "gemm_head": 2 * M * 2 * C * d}[cls]


class Runner:
    """Sets up one workload on cuda:0 and exposes step()."""

    def __init__(self, name, torch, binding, synth):
        self.torch = torch
        w = synth.WORKLOADS[name]
        self.w = w
        cfg = w.block
        self.cfg = cfg
        self.params = synth.make_params(cfg, 0, n_blocks=w.n_blocks)
        self.plan = binding.AFPlan(cfg, self.params)
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
        N, L, C = w.batch, w.length, cfg.C
        self.rows = min(w.jacobi_block, L)
        self.M = N * self.rows
        self.kw = {}
        if w.x_noise is not None:
            # forward first: the inverse inverts the forward's z
            x = synth.noisy_latents((N, L, C), 2, w.x_noise)
            self.x_fwd = dev(x)
            self.z, _ = self.plan.forward(self.x_fwd)
        else:
            self.x_fwd = dev(synth.normal((N, L, C), 2))
            self.z = dev(synth.normal((N, L, C), 1))
        if w.prefix:
            xp = synth.normal((N, w.prefix, C), 2)
            self.plan.prefill(dev(xp), rows=self.rows)
            self.kw = dict(init="given", x_init=dev(xp[:, -L:]), prefix_len=w.prefix,
                           x_last=dev(xp[:, -1]))
        elif w.init == "prev_frame":
            self.kw = dict(init="prev_frame", frame_len=w.frame_len)
        # output, iteration counts and workspace allocated once: every step
        # makes the same call on the same buffers
        self.binding = binding
        self.x = torch.empty_like(self.z)
        self.iters = np.zeros((w.n_blocks, -(-L // w.jacobi_block)), np.int32)
        nb = -(-L // w.jacobi_block)
        # (rows for two blocks: --fused-refresh may merge a block's cache
        # refresh into the next block's first pass)
        self.ws = self.plan.workspace(N, min(2 * w.jacobi_block, L) if nb > 1 else self.rows)
        torch.cuda.synchronize()
        self.tokens_per_step = N * L

    def step(self):
        kw = self.kw
        self.binding.af_inverse_jacobi(
            self.plan, self.z, self.w.jacobi_block, self.w.tau, 0, kw.get("init", "zero"),
            kw.get("x_init"), kw.get("frame_len", 0), kw.get("prefix_len", 0),
            kw.get("x_last"), self.x, self.iters, self.ws)
        return self.x


def cpu_baseline(runner, synth, budget_tokens):
    """Time the fp64 oracle (as it stands) on a bounded sample of the same
    workload: block-wise Jacobi on the first `budget_tokens` tokens of sample 0
    with the same tau (for the stack, the last block of the stack only)."""
    from threadpoolctl import threadpool_info
    from oracle import af_oracle as O
    w, cfg = runner.w, runner.cfg
    S = min(budget_tokens, w.length)
    z = runner.z[:1, :S].detach().cpu().numpy().astype(np.float64)
    t_idx = w.n_blocks - 1
    p64 = O.to64(runner.params[t_idx])
    kw = {}
    if w.prefix:  # keep the sample small: encode a prefix of equal length
        xp = synth.normal((1, w.prefix, cfg.C), 2)[:, -S:].astype(np.float64)
        cache, x_last = O.prefill(p64, xp, cfg.n_heads)
        kw = dict(pos0=S, cache=cache, x_last=x_last)
    t0 = time.perf_counter()
    _, it = O.inverse_jacobi_block(p64, z, cfg.n_heads, S, w.tau,
                                   direction=O.direction_of(t_idx), **kw)
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": S / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "seconds": round(dt, 2), "iters": it.tolist(),
            "sample": f"oracle fp64 block-Jacobi of the first {S} tokens of sample 0 "
                      f"(one Jacobi block of {S}, tau={w.tau}"
                      + (", after a prefix of equal length" if w.prefix else "")
                      + (f", stack block {t_idx} only" if w.n_blocks > 1 else "") + ")"}


def affine_sweep(torch, binding, tokens, reps=5):
    """The fused affine kernel alone (inverse mode), HBM-cold: `tokens` rows of
    C=48, buffers far larger than the 256 MB Infinity Cache.  Algorithmic
    bytes: read mu, raw, z, x_old and write x = 20*C bytes per token."""
    C = 48
    head = torch.randn(tokens, 2 * C, device="cuda")
    z = torch.randn(tokens, C, device="cuda")
    x = torch.randn(tokens, C, device="cuda")
    part = torch.empty(binding.afk_affine_partials_bytes(1, tokens, C), dtype=torch.uint8,
                       device="cuda")
    res = torch.empty(1, 2, device="cuda")
    binding.afk_affine(0, head, z, x, 1, tokens, C, res, part)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record()
        binding.afk_affine(0, head, z, x, 1, tokens, C, res, part)
        b.record()
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
    nbytes = 20 * C * tokens
    del head, z, x, part
    return {"tokens": tokens, "ms": round(ms, 4), "GB/s": round(nbytes / ms / 1e6, 1),
            "frac": round(nbytes / ms / 1e6 / PEAK_HBM_GBS, 4)}


def kernel_sources_hash():
    """Short hash of the HIP kernel sources (names and contents)."""
    import glob
    import hashlib
    csrc = os.path.join(ROOT, "autoregressive_normalizing_flow_amd", "csrc")
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.h"))):
        h.update(os.path.basename(p).encode())
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counter_traffic(workload, cls):
    """HBM bytes per launch of a kernel class from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary (scaled by the copy calibration), or None
    when there is none for this workload or the kernels changed since."""
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    sha = kernel_sources_hash()
    with open(path) as f:
        for line in f:
            t = line.split()
            if len(t) >= 3 and t[0] == "traffic-per-launch" and t[1] == cls:
                src = [x for x in t if x.startswith("sources=")]
                if src and src[0] == "sources=" + sha:
                    return int(t[2])
    return None


def timed_call(torch, fn, reps):
    """Median wall time (ms) of fn() over reps calls after one warm-up call."""
    fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        t0 = time.perf_counter()
        out = fn()
        torch.cuda.synchronize()
        ts.append((time.perf_counter() - t0) * 1e3)
    return float(np.median(ts)), out


def schedule_sweep(torch, binding, synth, reps):
    """Jacobi block size, warm start and schedule on the deep block (the
    frame480p and video21 shapes): tokens/s and iterations per block.  B = 1
    is sequential decoding on the GPU (one update per token), the baseline
    the Jacobi speed-up is quoted against."""
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    w = synth.WORKLOADS["frame480p"]
    params = synth.make_params(w.block, 0)
    plan = binding.AFPlan(w.block, params)
    F = w.length
    z = dev(synth.normal((1, F, w.block.C), 1))
    rows = []
    for B in (1, 64, 128, 256, 512, F):
        ms, (x, it) = timed_call(torch, lambda: plan.inverse_jacobi(z, B, w.tau),
                                 1 if B == 1 else reps)
        rows.append({"B": B, "ms": round(ms, 2), "tokens_per_s": round(F / ms * 1e3, 1),
                     "iters_total": int(it.sum()), "iters_max": int(it.max()),
                     "blocks": int(it.size)})
    seq = next(r for r in rows if r["B"] == 1)
    for r in rows:
        r["speedup_vs_sequential"] = round(seq["ms"] / r["ms"], 2)

    v = synth.WORKLOADS["video21"]
    T = v.length // F
    vplan = binding.AFPlan(v.block, synth.make_params(v.block, 0))
    zv = dev(synth.normal((1, v.length, v.block.C), 1))
    warm = {}
    for init in ("zero", "prev_frame"):
        kw = dict(init=init, frame_len=F) if init == "prev_frame" else {}
        ms, (xv, it) = timed_call(torch, lambda: vplan.inverse_jacobi(zv, F, v.tau, **kw), 1)
        warm[init] = {"ms": round(ms, 2), "tokens_per_s": round(v.length / ms * 1e3, 1),
                      "iters": it[0].tolist()}
    # asymmetric schedule: frame 0 with B = 64, then its K/V as the prefix of
    # frames 1.. solved with B = 512 and the previous-frame warm start
    def asym():
        x0, it0 = vplan.inverse_jacobi(zv[:, :F].contiguous(), 64, v.tau)
        vplan.prefill(x0, rows=512)
        x1, it1 = vplan.inverse_jacobi(zv[:, F:].contiguous(), 512, v.tau, init="prev_frame",
                                       frame_len=F, prefix_len=F, x_last=x0[:, -1].contiguous())
        return it0, it1
    ms, (it0, it1) = timed_call(torch, asym, 1)
    asym_row = {"ms": round(ms, 2), "tokens_per_s": round(v.length / ms * 1e3, 1),
                "frame0_B64_iters_total": int(it0.sum()),
                "frames1_B512_iters_total": int(it1.sum()), "frames": T}
    return {"block_sweep_frame480p": rows, "warm_start_video21": warm,
            "asymmetric_video21": asym_row}


def pipeline_bench(torch, binding, synth, reps, graphs=False, fused_refresh=False,
                   row_split=True):
    """End-to-end inverse of the deep o shallow flow over 21 frames (deep:
    the video21 block, shallow: the shallow_stack stack), three schedules:
    stages (the deep block over all frames in one call, then the shallow
    stack on all frames batched), frames one after another on one stream,
    and the pipeline (shallow stack of frame n on a second stream and host
    thread while the deep block solves frame n+1)."""
    from autoregressive_normalizing_flow_amd.pipeline import DeepShallowFlow
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    v, sh = synth.WORKLOADS["video21"], synth.WORKLOADS["shallow_stack"]
    F = v.frame_len
    deep = binding.AFPlan(v.block, synth.make_params(v.block, 0))
    shallow = binding.AFPlan(sh.block, synth.make_params(sh.block, 0, n_blocks=sh.n_blocks))
    for plan in (deep, shallow):
        plan.set_graphs(graphs)
        plan.set_fused_refresh(fused_refresh)
        plan.set_row_split(row_split)
    flow = DeepShallowFlow(deep, shallow, F)
    z = dev(synth.normal((1, v.length, v.block.C), 1))
    nf = v.length // F
    out = {"frames": nf, "tokens": v.length}

    def stages():
        u, itd = deep.inverse_jacobi(z, F, v.tau, init="prev_frame", frame_len=F)
        x, its = shallow.inverse_jacobi(u.reshape(nf, F, -1).contiguous(), F, v.tau)
        return itd, its
    for name, fn in (("stages", stages),
                     ("frames_serial", lambda: flow.inverse(z, v.tau, pipelined=False)),
                     ("pipelined", lambda: flow.inverse(z, v.tau, pipelined=True))):
        ms, _ = timed_call(torch, fn, reps)
        out[name] = {"ms": round(ms, 2), "tokens_per_s": round(v.length / ms * 1e3, 1)}
    ms, _ = timed_call(torch, lambda: deep.inverse_jacobi(z, F, v.tau, init="prev_frame",
                                                          frame_len=F), reps)
    out["deep_only"] = {"ms": round(ms, 2), "tokens_per_s": round(v.length / ms * 1e3, 1)}
    # the deep block alone by a sliding window of 7 frames with 1 frame of
    # overlap re-encoded per chunk (chunks of 7, 6, 6 and 2 frames)
    from autoregressive_normalizing_flow_amd.pipeline import stream_inverse
    ms, (_, its) = timed_call(torch, lambda: stream_inverse(deep, z, 7 * F, F, F, v.tau,
                                                            frame_len=F), reps)
    out["deep_streaming_w7_o1"] = {"ms": round(ms, 2),
                                   "tokens_per_s": round(v.length / ms * 1e3, 1),
                                   "chunk_iters": [i.tolist() for i in its]}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="frame480p")
    ap.add_argument("--cpu-tokens", type=int, default=1024,
                    help="oracle sample size for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-row-split", action="store_true",
                    help="run every Jacobi update as one pass (no two-stream row split)")
    ap.add_argument("--fused-refresh", action="store_true",
                    help="recompute an early-stopped block's K/V in the next block's "
                         "first update instead of in a pass of its own")
    ap.add_argument("--graphs", action="store_true",
                    help="replay the captured Jacobi update as a HIP graph instead "
                         "of launching every kernel directly")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (to scale HBM counters)")
    ap.add_argument("--pipeline", action="store_true",
                    help="only run the deep o shallow end-to-end inverse (stages, "
                         "frames serial, pipelined)")
    ap.add_argument("--schedule-sweep", action="store_true",
                    help="only run the block-size / warm-start / schedule sweep "
                         "(B = 1 is the GPU sequential baseline)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: there is no multi-GPU path; the "
              "per-GPU kernels are measured at their real shape.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        # a plain copy of known size: 256 MiB read + 256 MiB written per launch
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": src.numel() * 4, "launches": 5}))
        return
    from autoregressive_normalizing_flow_amd import binding, synth
    binding.load_library()
    assert torch.cuda.is_available(), "no GPU"
    if args.pipeline:
        print(json.dumps(pipeline_bench(torch, binding, synth, max(args.steps, 1),
                                        args.graphs, args.fused_refresh,
                                        not args.no_row_split)), flush=True)
        return
    if args.schedule_sweep:
        print(json.dumps(schedule_sweep(torch, binding, synth, max(args.steps, 1))), flush=True)
        return

    r = Runner(args.workload, torch, binding, synth)
    cfg, w = r.cfg, r.w
    r.plan.set_graphs(args.graphs)
    r.plan.set_fused_refresh(args.fused_refresh)
    r.plan.set_row_split(not args.no_row_split)
    for _ in range(args.warmup):
        r.step()
    torch.cuda.synchronize()

    # per-class breakdown: one untimed profiled step per class
    breakdown = {}
    for cls in ALL_CLASSES:
        r.plan.profile_enable(cls)
        r.step()
        n, ms = r.plan.profile_read()
        r.plan.profile_disable()
        breakdown[cls] = {"launches": n, "ms": round(ms, 4)}
    dominant = max(GEMM_CLASSES, key=lambda c: breakdown[c]["ms"])

    # timed region: K steps as a user runs them (Jacobi updates launched
    # directly, or replayed as graphs with --graphs)
    r.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        r.step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = r.tokens_per_step / ((t1 - t0) / args.steps)

    # the dominant kernel timed live by HIP events on the stream it is launched
    # on, over K more steps of the same workload; these launch directly, as
    # events recorded inside a graph carry no timing on this runtime
    r.plan.profile_enable(dominant)
    torch.cuda.synchronize()
    p0 = time.perf_counter()
    for _ in range(args.steps):
        r.step()
    torch.cuda.synchronize()
    p1 = time.perf_counter()
    n_launch, dom_ms = r.plan.profile_read()
    r.plan.profile_disable()

    flops = gemm_flops_per_launch(dominant, r.M, cfg)
    avg_ms = dom_ms / max(n_launch, 1)
    peak = PEAK_BF16_TFLOPS if (cfg.dtype == "bf16" and dominant != "gemm_head") else PEAK_F32_TFLOPS
    achieved = flops / (avg_ms * 1e-3) / 1e12
    roofline = {"kernel": dominant, "bound": "mfma", "achieved": round(achieved, 2),
                "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": counter_traffic(w.name, dominant), "flops_per_launch": flops,
                "avg_ms": round(avg_ms, 5), "launches": n_launch,
                "timing": f"HIP events, {args.steps} direct-launch steps after the timed region",
                "ms_per_step_profiled": round((p1 - p0) * 1e3 / args.steps, 3)}

    # all GEMMs together (algorithmic flops / summed kernel time, one step)
    g_flops = sum(gemm_flops_per_launch(c, r.M, cfg) * breakdown[c]["launches"]
                  for c in GEMM_CLASSES)
    g_ms = sum(breakdown[c]["ms"] for c in GEMM_CLASSES)
    # fused affine kernel in the path: 20*C bytes per token per launch
    # (no separate launches when the affine update is fused into the head
    # GEMM's kernel, which the gemm_head class then times)
    aff = breakdown["affine"]
    aff_bytes = 20 * cfg.C * r.M
    aff_gbs = aff_bytes * aff["launches"] / (aff["ms"] * 1e-3) / 1e9 if aff["ms"] else None

    # forward pass (af_forward) time, untimed by the metric
    torch.cuda.synchronize()
    f0 = time.perf_counter()
    r.plan.forward(r.x_fwd)
    torch.cuda.synchronize()
    fwd_ms = (time.perf_counter() - f0) * 1e3

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "tokens": w.length,
                   "jacobi_block": w.jacobi_block, "tau": w.tau, "init": w.init,
                   "stack_blocks": w.n_blocks, "layers": cfg.n_layers, "d": cfg.d,
                   "heads": cfg.n_heads, "C": cfg.C, "prefix": w.prefix},
        "iters_per_block": r.iters.tolist(),
        "roofline": roofline,
        "gemm_all": {"TFLOP/s": round(g_flops / (g_ms * 1e-3) / 1e12, 2) if g_ms else None,
                     "frac": round(g_flops / (g_ms * 1e-3) / 1e12 / peak, 4) if g_ms else None},
        "affine_in_path": ({"bound": "hbm", "GB/s": round(aff_gbs, 1),
                            "frac": round(aff_gbs / PEAK_HBM_GBS, 4),
                            "bytes_per_launch": aff_bytes} if aff_gbs is not None
                           else {"fused_into": "gemm_head"}),
        "graphs": args.graphs,
        "fused_refresh": args.fused_refresh,
        "row_split": not args.no_row_split,
        "kernel_ms_per_step": breakdown,
        "forward_ms": round(fwd_ms, 3),
    }
    if not args.no_sweep:
        out["affine_hbm_sweep"] = [affine_sweep(torch, binding, t) for t in (1 << 20, 1 << 22)]
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(r, synth, args.cpu_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
