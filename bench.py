#!/usr/bin/env python3
"""Benchmark: latent tokens/s inverted by video-aware block-wise Jacobi on one
MI355X, with the roofline of the dominant kernel and the CPU oracle beside it.

    python bench.py [--steps K] [--warmup W] [--workload video21]

A step is one af_inverse_jacobi call over one batch of synthetic latents
(every kernel of the hot path: shift+embed, LayerNorm, QKV/O/MLP GEMMs,
attention over the KV cache, head, fused affine/residual kernel, host stop
test).  Inputs are resident in HBM before timing.  Prints ONE JSON line.

Workloads (autoregressive_normalizing_flow_amd.synth.WORKLOADS):
  video21        21 frames x 1560 tokens, block = frame, previous-frame warm
                 start, 8 layers d=1024                              (default)
  frame480p      one 1560-token frame, 8 layers d=1024, B=1560
  shallow_stack  T=4 alternating blocks, 2 layers d=512, 21 frames batched
  wide_prefix    4 layers d=4096, 2-frame prefix, batch 2
  tiny_f32       one 8x8 frame, fp32

Other modes: --schedule-sweep, --pipeline, --cpu-baselines (the oracle on
every workload), --affine-sweep (the fused affine kernel HBM-cold beside the
streaming copy), --copy-calibration, and --summarize-trace /
--summarize-counters (turn rocprofv3 CSV output into the summaries kept under
profiles/).
"""
import argparse
import csv
import glob
import json
import os
import statistics
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
FLOP_CLASSES = GEMM_CLASSES + ("attention", "embed")
ALL_CLASSES = GEMM_CLASSES + ("attention", "layernorm", "embed", "affine", "device_loop")
DEFAULT_WORKLOAD = "video21"
OTHER_CONFIGS = ("tiny_f32", "frame480p", "shallow_stack", "wide_prefix")


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


# ---------------------------------------------------------------------------
# the oracle on the host cores
# ---------------------------------------------------------------------------
def cpu_info():
    """CPU model, BLAS library and the threads it uses."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    from threadpoolctl import threadpool_info
    blas = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
    b = blas[0] if blas else {}
    return {"cpu": model, "host_cpus": len(os.sched_getaffinity(0)),
            "blas": f"{b.get('internal_api', '?')} {b.get('version', '')} "
                    f"{b.get('architecture', '')}".strip(),
            "threads": int(b.get("num_threads", 1))}


def oracle_sample(w, params, z, synth, max_tokens):
    """The oracle's same-schedule block-wise Jacobi on a bounded part of a
    workload: the first Jacobi block of sample 0 (for the video, frame 0 with
    its zero init; for a stack, the last stack block, which the inverse runs
    first; with a prefix, the prefix encoded first, outside the timing), cut
    to max_tokens.  Returns (seconds, tokens, iters, description)."""
    from oracle import af_oracle as O
    cfg = w.block
    S = min(max_tokens, w.jacobi_block, w.length)
    zz = np.asarray(z[:1, :S], dtype=np.float64)
    t_idx = w.n_blocks - 1
    p64 = O.to64(params[t_idx])
    kw = {}
    desc = (f"oracle fp64 block-Jacobi, same schedule: the first Jacobi block of sample 0 "
            f"({S} tokens, tau={w.tau}")
    if w.prefix:
        xp = synth.normal((1, w.prefix, cfg.C), 2).astype(np.float64)
        cache, x_last = O.prefill(p64, xp, cfg.n_heads)
        kw = dict(pos0=w.prefix, cache=cache, x_last=x_last, init="given",
                  x_init=xp[:, -w.length:][:, :S])
        desc += f", after the {w.prefix}-token prefix (encoded untimed), given init"
    if w.n_blocks > 1:
        desc += f", stack block {t_idx} of {w.n_blocks}"
    t0 = time.perf_counter()
    _, it = O.inverse_jacobi_block(p64, zz, cfg.n_heads, S, w.tau,
                                   direction=O.direction_of(t_idx), **kw)
    dt = time.perf_counter() - t0
    return dt, S, it.tolist(), desc + ")"


def cpu_baseline(w, params, z, synth, max_tokens):
    """The fp64 oracle (as it stands) timed on the host cores on a bounded
    sample of the same workload (oracle_sample); z is the workload's input on
    the host."""
    dt, S, it, desc = oracle_sample(w, params, z, synth, max_tokens)
    info = cpu_info()
    return {"value": round(S / dt, 2), "unit": "tokens/s", "cores": info["threads"],
            "kind": "oracle", "seconds": round(dt, 2), "iters": it, "sample": desc,
            "cpu": info["cpu"], "blas": info["blas"]}


def oracle_sequential_rate(w, params, z, synth, n_tokens):
    """Exact sequential inverse (token by token, 'standard AR decoding') of
    the first n_tokens of sample 0 of a workload's first Jacobi block on the
    host cores: seconds per token (after the prefix, when there is one)."""
    from oracle import af_oracle as O
    cfg = w.block
    t_idx = w.n_blocks - 1
    p64 = O.to64(params[t_idx])
    zz = np.asarray(z[:1, :n_tokens], dtype=np.float64)
    kw = {}
    if w.prefix:
        xp = synth.normal((1, w.prefix, cfg.C), 2).astype(np.float64)
        cache, x_last = O.prefill(p64, xp, cfg.n_heads)
        kw = dict(pos0=w.prefix, cache=cache, x_last=x_last)
    t0 = time.perf_counter()
    O.inverse_sequential_block(p64, zz, cfg.n_heads, O.direction_of(t_idx), **kw)
    return (time.perf_counter() - t0) / n_tokens


def cpu_baselines(torch, synth, jacobi_tokens, seq_tokens):
    """The oracle on every workload, on the host cores: the same-schedule
    Jacobi on the first Jacobi block (bounded), and the exact sequential
    inverse timed on its first seq_tokens tokens and extrapolated linearly to
    the workload's tokens (labelled)."""
    out = {"host": cpu_info()}
    for name in ("tiny_f32", "frame480p", "video21", "shallow_stack", "wide_prefix"):
        w = synth.WORKLOADS[name]
        params = synth.make_params(w.block, 0, n_blocks=w.n_blocks)
        if w.x_noise is not None:
            from oracle import af_oracle as O
            x = synth.noisy_latents((1, w.length, w.block.C), 2, w.x_noise)
            z, _ = O.forward_stack([O.to64(p) for p in params], x, w.block.n_heads)
        else:
            z = synth.normal((w.batch, w.length, w.block.C), 1)
        dt, S, it, desc = oracle_sample(w, params, z, synth, jacobi_tokens)
        row = {"jacobi": {"tokens_per_s": round(S / dt, 2), "seconds": round(dt, 2),
                          "iters": it, "sample": desc}}
        n = min(seq_tokens, w.length)
        spt = oracle_sequential_rate(w, params, z, synth, n)
        total = w.batch * w.length * w.n_blocks
        row["sequential"] = {
            "tokens_per_s": round(1.0 / spt, 3), "timed_tokens": n,
            "seconds_per_token": round(spt, 4),
            "workload_seconds": round(spt * total, 1),
            "extrapolated": n < w.length or w.batch > 1 or w.n_blocks > 1,
            "note": ("timed on the first tokens of sample 0 (one stack block), scaled "
                     "linearly to every token, sample and stack block")}
        out[name] = row
        print(json.dumps({name: row}), file=sys.stderr, flush=True)
        del params
    return out


# ---------------------------------------------------------------------------
# kernel-level measurements
# ---------------------------------------------------------------------------
def affine_sweep(torch, binding, tokens, reps=7):
    """The fused affine kernel alone (inverse mode), HBM-cold: `tokens` rows of
    C=48, buffers far larger than the 256 MB Infinity Cache.  Algorithmic
    bytes: read mu, raw, z, x_old and write x = 20*C bytes per token.  Beside
    it, the library's streaming copy moving the same number of bytes (half
    read, half written): the rate this access pattern can reach here."""
    C = 48
    head = torch.randn(tokens, 2 * C, device="cuda")
    z = torch.randn(tokens, C, device="cuda")
    x = torch.randn(tokens, C, device="cuda")
    part = torch.empty(binding.afk_affine_partials_bytes(1, tokens, C), dtype=torch.uint8,
                       device="cuda")
    res = torch.empty(1, 2, device="cuda")
    nbytes = 20 * C * tokens

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in ev:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ev]))

    ms = timed(lambda: binding.afk_affine(0, head, z, x, 1, tokens, C, res, part))
    del head, z, x, part
    src = torch.empty(nbytes // 2 // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    ms_copy = timed(lambda: binding.afk_stream_copy(src, dst))
    del src, dst
    gbs, gbs_copy = nbytes / ms / 1e6, nbytes / ms_copy / 1e6
    return {"tokens": tokens, "ms": round(ms, 4), "GB/s": round(gbs, 1),
            "frac": round(gbs / PEAK_HBM_GBS, 4), "copy_GB/s": round(gbs_copy, 1),
            "vs_copy": round(gbs / gbs_copy, 3)}


def kernel_sources_hash():
    """Short hash of the HIP kernel sources (names and contents)."""
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


# ---------------------------------------------------------------------------
# schedules
# ---------------------------------------------------------------------------
def asymmetric_schedule(vplan, zv, F, B0, B1, tau):
    """Frame 0 with blocks of B0 from zeros; every later frame n with blocks
    of B1 kept inside the frame, warm-started from frame n-1's converged
    tokens, attending to the K/V of frames 0..n-1 (关键设计 3: first frame
    B = 64, later frames B = 512).  Each frame is one af_inverse_jacobi call;
    the K/V of the frame's last Jacobi block (which that call leaves
    unrefreshed) are then recomputed from its final tokens."""
    nf = zv.shape[1] // F
    x = zv.new_empty(zv.shape)
    its = []
    for n in range(nf):
        zn = zv[:, n * F:(n + 1) * F]
        if n == 0:
            xn, it = vplan.inverse_jacobi(zn, B0, tau)
            last = (F - 1) // B0 * B0
        else:
            xn, it = vplan.inverse_jacobi(zn, B1, tau, init="given",
                                          x_init=x[:, (n - 1) * F:n * F],
                                          prefix_len=n * F,
                                          x_last=x[:, n * F - 1].contiguous())
            last = (F - 1) // B1 * B1
        x[:, n * F:(n + 1) * F].copy_(xn)
        its.append(it[0].copy())
        if n + 1 < nf:
            P = n * F + last
            vplan.refresh_kv(x[:, P:(n + 1) * F].contiguous(), prefix_len=P,
                             x_last=x[:, P - 1].contiguous() if P > 0 else None)
    return x, its


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
    vplan.workspace(1, F)
    warm = {}
    for init in ("zero", "prev_frame"):
        kw = dict(init=init, frame_len=F) if init == "prev_frame" else {}
        ms, (xv, it) = timed_call(torch, lambda: vplan.inverse_jacobi(zv, F, v.tau, **kw), 1)
        warm[init] = {"ms": round(ms, 2), "tokens_per_s": round(v.length / ms * 1e3, 1),
                      "iters": it[0].tolist()}
    ms, (_, its) = timed_call(torch, lambda: asymmetric_schedule(vplan, zv, F, 64, 512, v.tau), 1)
    asym_row = {"ms": round(ms, 2), "tokens_per_s": round(v.length / ms * 1e3, 1),
                "frame0_B64_iters_total": int(its[0].sum()),
                "frames1_B512_iters": [it.tolist() for it in its[1:]], "frames": T}
    return {"block_sweep_frame480p": rows, "warm_start_video21": warm,
            "asymmetric_video21": asym_row}


def pipeline_bench(torch, binding, synth, reps, graphs=False, fused_refresh=False,
                   row_split=False):
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


# ---------------------------------------------------------------------------
# rocprofv3 output -> the summaries kept under profiles/
# ---------------------------------------------------------------------------
def _read_csv(pattern):
    files = sorted(glob.glob(pattern, recursive=True))
    if not files:
        raise SystemExit(f"no file matches {pattern}")
    rows = []
    for fn in files:
        with open(fn, newline="") as f:
            rows.extend(csv.DictReader(f))
    return rows


def summarize_trace(d, top):
    """Markdown table of a --kernel-trace --stats run: kernel, calls, total
    ms, average us and share, from <d>/**/*kernel_stats.csv; and the busy time
    (union of the kernels' intervals) from *kernel_trace.csv."""
    stats = _read_csv(os.path.join(d, "**", "*kernel_stats.csv"))
    stats.sort(key=lambda r: -float(r["TotalDurationNs"]))
    tot = sum(float(r["TotalDurationNs"]) for r in stats)
    lines = ["| kernel | calls | total ms | avg us | % |", "|---|---:|---:|---:|---:|"]
    for r in stats[:top]:
        name = r["Name"][:110]
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.2f} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    tr = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if tr:
        iv = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]))
                    for r in _read_csv(os.path.join(d, "**", "*kernel_trace.csv")))
        busy, cur_s, cur_e = 0, None, None
        for s, e in iv:
            if cur_e is None or s > cur_e:
                if cur_e is not None:
                    busy += cur_e - cur_s
                cur_s, cur_e = s, e
            else:
                cur_e = max(cur_e, e)
        if cur_e is not None:
            busy += cur_e - cur_s
        lines.append("")
        lines.append(f"Sum of kernel durations {tot / 1e6:.1f} ms; busy (union of intervals) "
                     f"{busy / 1e6:.1f} ms.")
    print("\n".join(lines))


# kernel class of a kernel name in the inverse path (the forward's split-mode
# kernels, which carry bf16 hi + lo operands, are listed but not classed)
CLASS_PATTERNS = {
    "attention": (("attn_dma_kernel", ""), ("attn_dma2_kernel", ""), ("attn32_kernel", ""),
                  ("attn_bf16_kernel", "false>")),
    "affine": (("affine_kernel<0", ""),),
}


def _class_of(name):
    for cls, pats in CLASS_PATTERNS.items():
        for a, b in pats:
            if a in name and b in name:
                return cls
    return None


def summarize_counters(d, calib_dir, workload):
    """Per-kernel medians of the counters of one or more --pmc passes under
    <d> (FETCH_SIZE, WRITE_SIZE: KiB per dispatch, scaled by what the same
    counters read for a plain copy of known size under calib_dir), and the
    'traffic-per-launch' lines bench.py reads for the roofline."""
    rows = _read_csv(os.path.join(d, "**", "*counter_collection.csv"))
    per = {}
    for r in rows:
        key = (r["Kernel_Name"], r["Counter_Name"])
        per.setdefault(key, {}).setdefault(r["Dispatch_Id"], 0.0)
        per[key][r["Dispatch_Id"]] += float(r["Counter_Value"])
    scale = {"FETCH_SIZE": 1.0, "WRITE_SIZE": 1.0}
    if calib_dir:
        crow = _read_csv(os.path.join(calib_dir, "**", "*counter_collection.csv"))
        copy_kib = 262144.0   # 256 MiB read and 256 MiB written per dispatch
        for cn in scale:
            vals = {}
            for r in crow:
                if r["Counter_Name"] == cn and "copy" in r["Kernel_Name"].lower():
                    vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(
                        r["Counter_Value"])
            if vals:
                scale[cn] = copy_kib / statistics.median(vals.values())
    counters = sorted({k[1] for k in per})
    kernels = sorted({k[0] for k in per})
    print(f"Scale: FETCH_SIZE x {scale['FETCH_SIZE']:.3f}, WRITE_SIZE x "
          f"{scale['WRITE_SIZE']:.3f} (a plain 256 MiB copy)\n")
    print("| kernel | dispatches | " + " | ".join(f"{c} (median)" for c in counters) + " |")
    print("|---|---:|" + "---:|" * len(counters))
    cls_bytes = {}
    for k in kernels:
        vals = [per.get((k, c), {}) for c in counters]
        n = max(len(v) for v in vals)
        cells = [f"{statistics.median(v.values()):.0f}" if v else "" for v in vals]
        print(f"| `{k[:100]}` | {n} | " + " | ".join(cells) + " |")
        cls = _class_of(k)
        if cls and ("FETCH_SIZE" in counters or "WRITE_SIZE" in counters):
            for cn in ("FETCH_SIZE", "WRITE_SIZE"):
                v = per.get((k, cn), {})
                if v:
                    cls_bytes.setdefault(cls, {}).setdefault(cn, []).extend(
                        x * 1024 * scale[cn] for x in v.values())
    sha = kernel_sources_hash()
    print()
    for cls, b in cls_bytes.items():
        rd = statistics.mean(b.get("FETCH_SIZE", [0.0]))
        wr = statistics.mean(b.get("WRITE_SIZE", [0.0]))
        print(f"    traffic-per-launch {cls} {int(rd + wr)} read={int(rd)} write={int(wr)} "
              f"sources={sha}")


# ---------------------------------------------------------------------------
# the benchmark
# ---------------------------------------------------------------------------
def roofline_of(cls, n, ms, work, cfg, workload, steps):
    """The roofline entry of one kernel class from its profiled launches."""
    if n == 0 or ms <= 0:
        return {"kernel": cls, "launches": n, "achieved": None}
    avg_ms = ms / max(n, 1)
    per_launch = work / max(n, 1)
    if cls == "device_loop":
        # the whole Jacobi loop of a small fp32 block in one workgroup: vector
        # fp32 arithmetic on one CU, against the chip's fp32 vector peak
        achieved = per_launch / (avg_ms * 1e-3) / 1e12
        return {"kernel": cls, "bound": "alu", "achieved": round(achieved, 4),
                "peak": PEAK_F32_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_F32_TFLOPS, 6), "traffic": None,
                "flops_per_launch": round(per_launch), "avg_ms": round(avg_ms, 5),
                "launches": n}
    if cls == "affine":
        achieved = per_launch / (avg_ms * 1e-3) / 1e9
        return {"kernel": cls, "bound": "hbm", "achieved": round(achieved, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": counter_traffic(workload, cls), "bytes_per_launch": per_launch,
                "avg_ms": round(avg_ms, 5), "launches": n}
    peak = PEAK_BF16_TFLOPS if (cfg.dtype == "bf16" and cls not in ("gemm_head", "embed")) \
        else PEAK_F32_TFLOPS
    achieved = per_launch / (avg_ms * 1e-3) / 1e12
    return {"kernel": cls, "bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
            "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
            "traffic": counter_traffic(workload, cls), "flops_per_launch": round(per_launch),
            "avg_ms": round(avg_ms, 5), "launches": n}


def quick_config(name, torch, binding, synth, steps, warmup):
    """tokens/s and iterations of another workload (a few steps)."""
    r = Runner(name, torch, binding, synth)
    for _ in range(warmup):
        r.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        r.step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    out = {"tokens_per_s": round(r.tokens_per_step / dt, 1), "ms_per_step": round(dt * 1e3, 3),
           "iters_per_block": r.iters.tolist(), "tokens": r.tokens_per_step}
    if r.w.prefix:
        # the prefix's encoding into the KV cache, outside the metric: one
        # af_prefill of the observed tokens (median of 3 after a warm-up)
        N, C = r.w.batch, r.cfg.C
        xp = torch.from_numpy(np.ascontiguousarray(
            synth.normal((N, r.w.prefix, C), 2), np.float32)).cuda()
        times = []
        for i in range(4):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            r.plan.prefill(xp, rows=r.rows)
            torch.cuda.synchronize()
            if i:
                times.append(time.perf_counter() - t0)
        times.sort()
        out["prefill_ms"] = round(times[1] * 1e3, 3)
        out["prefill_tokens"] = N * r.w.prefix
        # the GEMMs at the prefill's shape (N x prefix rows), by event timing
        gem = {}
        for cls in ("gemm_qkv", "gemm_mlp1", "gemm_mlp2"):
            r.plan.profile_enable(cls)
            r.plan.prefill(xp, rows=r.rows)
            n, ms, work = r.plan.profile_read_work()
            r.plan.profile_disable()
            if n and ms > 0:
                tf = work / (ms * 1e-3) / 1e12
                gem[cls] = {"TFLOP/s": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                            "avg_ms": round(ms / n, 4)}
        out["prefill_gemms"] = gem
    del r
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-tokens", type=int, default=1560,
                    help="oracle sample size for the CPU baseline (tokens of the first "
                         "Jacobi block)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the short runs of the other workloads")
    ap.add_argument("--row-split", action="store_true",
                    help="run long-prefix Jacobi updates as two half passes on two streams "
                         "(af_plan_set_row_split; off by default)")
    ap.add_argument("--fused-refresh", action="store_true",
                    help="recompute an early-stopped block's K/V in the next block's "
                         "first update instead of in a pass of its own")
    ap.add_argument("--serial-refresh", action="store_true",
                    help="run an early-stopped block's K/V recomputation on the call's "
                         "stream instead of beside the next block's first update "
                         "(af_plan_set_overlap_refresh(0))")
    ap.add_argument("--graphs", action="store_true",
                    help="replay the captured Jacobi update as a HIP graph instead "
                         "of launching every kernel directly")
    ap.add_argument("--affine-sweep", action="store_true",
                    help="print only the HBM-cold sweep of the fused affine kernel and the "
                         "streaming copy beside it")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (to scale HBM counters)")
    ap.add_argument("--pipeline", action="store_true",
                    help="only run the deep o shallow end-to-end inverse (stages, "
                         "frames serial, pipelined)")
    ap.add_argument("--schedule-sweep", action="store_true",
                    help="only run the block-size / warm-start / schedule sweep "
                         "(B = 1 is the GPU sequential baseline)")
    ap.add_argument("--cpu-baselines", action="store_true",
                    help="only time the oracle on every workload (same-schedule Jacobi "
                         "and exact sequential inverse) on the host cores")
    ap.add_argument("--seq-tokens", type=int, default=32,
                    help="tokens timed per workload for the sequential oracle")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print the kernel-trace summary of a rocprofv3 output folder")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="print the counter summary of rocprofv3 --pmc output folder(s)")
    ap.add_argument("--calibration", metavar="DIR", default=None,
                    help="rocprofv3 --pmc output of --copy-calibration (counter scale)")
    ap.add_argument("--top", type=int, default=16)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: there is no multi-GPU path; the "
              "per-GPU kernels are measured at their real shape.", file=sys.stderr)
        sys.exit(2)
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.top)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.calibration, args.workload)
        return

    import torch
    if args.copy_calibration:
        # a plain copy of known size: 256 MiB read + 256 MiB written per
        # launch, by the library's streaming copy kernel
        from autoregressive_normalizing_flow_amd import binding
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            binding.afk_stream_copy(src, dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": src.numel() * 4, "launches": 5}))
        return
    from autoregressive_normalizing_flow_amd import synth
    if args.cpu_baselines:
        print(json.dumps(cpu_baselines(torch, synth, args.cpu_tokens, args.seq_tokens)),
              flush=True)
        return
    from autoregressive_normalizing_flow_amd import binding
    binding.load_library()
    assert torch.cuda.is_available(), "no GPU"
    if args.affine_sweep:
        print(json.dumps({"affine_hbm_sweep": [affine_sweep(torch, binding, t)
                                               for t in (1 << 20, 1 << 22, 1 << 24)]}),
              flush=True)
        return
    if args.pipeline:
        print(json.dumps(pipeline_bench(torch, binding, synth, max(args.steps, 1),
                                        args.graphs, args.fused_refresh,
                                        args.row_split)), flush=True)
        return
    if args.schedule_sweep:
        print(json.dumps(schedule_sweep(torch, binding, synth, max(args.steps, 1))), flush=True)
        return

    r = Runner(args.workload, torch, binding, synth)
    cfg, w = r.cfg, r.w
    r.plan.set_graphs(args.graphs)
    r.plan.set_fused_refresh(args.fused_refresh)
    r.plan.set_row_split(args.row_split)
    r.plan.set_overlap_refresh(not args.serial_refresh)
    for _ in range(args.warmup):
        r.step()
    torch.cuda.synchronize()

    # timed region: K steps as a user runs them (Jacobi updates launched
    # directly, or replayed as graphs with --graphs)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        r.step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = r.tokens_per_step / ((t1 - t0) / args.steps)
    iters = r.iters.tolist()

    # per-class breakdown: one profiled step per class (events on the launch
    # stream of every launch of the class; algorithmic work from the library).
    # With cache refreshes beside the next block's first update, launches of
    # the two streams overlap and each one's events also span the other's
    # work: the breakdown runs its steps with every refresh on the call's
    # stream, so the classes' times are the kernels' own and add up to a step.
    overlap = not args.serial_refresh and w.length > w.jacobi_block and cfg.dtype == "bf16"
    if overlap:
        r.plan.set_overlap_refresh(False)
    breakdown = {}
    for cls in ALL_CLASSES:
        r.plan.profile_enable(cls)
        r.step()
        n, ms, work = r.plan.profile_read_work()
        r.plan.profile_disable()
        breakdown[cls] = {"launches": n, "ms": round(ms, 4), "work": work}
    if overlap:
        r.plan.set_overlap_refresh(True)
    dominant = max(ALL_CLASSES, key=lambda c: breakdown[c]["ms"])
    gemm_dom = max(GEMM_CLASSES, key=lambda c: breakdown[c]["ms"])

    # the dominant kernel timed live by HIP events on the stream it is launched
    # on, over K more steps of the same workload; these launch directly, as
    # events recorded inside a graph carry no timing on this runtime.  With
    # cache refreshes beside the next block's first update (two streams), a
    # launch that overlaps the other stream's kernels shares the GPU with them
    # and its events span their work too: the roofline takes the K steps with
    # every refresh on the call's stream (the kernels alone, as the breakdown
    # and the counters see them), and `roofline_in_step` the same class over K
    # steps as the timed region runs them.
    def time_dominant(overlapped):
        if overlap:
            r.plan.set_overlap_refresh(overlapped)
        r.plan.profile_enable(dominant)
        torch.cuda.synchronize()
        p0 = time.perf_counter()
        for _ in range(args.steps):
            r.step()
        torch.cuda.synchronize()
        p1 = time.perf_counter()
        n_l, ms_l, work_l = r.plan.profile_read_work()
        r.plan.profile_disable()
        if overlap:
            r.plan.set_overlap_refresh(True)
        roof = roofline_of(dominant, n_l, ms_l, work_l, cfg, w.name, args.steps)
        roof["ms_per_step_profiled"] = round((p1 - p0) * 1e3 / args.steps, 3)
        return roof
    roofline = time_dominant(False)
    roofline["timing"] = (f"HIP events on the launch stream, {args.steps} direct-launch steps "
                          "after the timed region" +
                          (" with every cache refresh on the call's stream (the kernels alone; "
                           "in the timed steps refreshes run beside the next block's first "
                           "update)" if overlap else ""))
    roof_step = None
    if overlap:
        roof_step = time_dominant(True)
        roof_step["timing"] = (f"HIP events on the launch stream, {args.steps} steps as the timed "
                               "region runs them: launches that overlap the other stream's "
                               "kernels share the GPU with them, and their events span that "
                               "work too")
    g = breakdown[gemm_dom]
    gemm_roof = roofline_of(gemm_dom, g["launches"], g["ms"], g["work"], cfg, w.name, 1)

    # all GEMMs together (algorithmic flops / summed kernel time, one step)
    g_flops = sum(breakdown[c]["work"] for c in GEMM_CLASSES)
    g_ms = sum(breakdown[c]["ms"] for c in GEMM_CLASSES)
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    aff = breakdown["affine"]
    aff_gbs = aff["work"] / (aff["ms"] * 1e-3) / 1e9 if aff["ms"] else None

    # forward pass (af_forward) time, outside the metric
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
                   "frame_len": w.frame_len, "stack_blocks": w.n_blocks,
                   "layers": cfg.n_layers, "d": cfg.d, "heads": cfg.n_heads, "C": cfg.C,
                   "prefix": w.prefix},
        "iters_per_block": iters,
        "roofline": roofline,
        "gemm_dominant": gemm_roof,
        "gemm_all": {"TFLOP/s": round(g_flops / (g_ms * 1e-3) / 1e12, 2) if g_ms else None,
                     "frac": round(g_flops / (g_ms * 1e-3) / 1e12 / peak, 4) if g_ms else None},
        "affine_in_path": ({"bound": "hbm", "GB/s": round(aff_gbs, 1),
                            "frac": round(aff_gbs / PEAK_HBM_GBS, 4),
                            "bytes_per_launch": aff["work"] / max(aff["launches"], 1)}
                           if aff_gbs is not None else None),
        "graphs": args.graphs,
        "fused_refresh": args.fused_refresh,
        "row_split": args.row_split,
        "overlap_refresh": not args.serial_refresh,
        "roofline_in_step": roof_step,
        "kernel_ms_per_step": {c: {"launches": b["launches"], "ms": b["ms"]}
                               for c, b in breakdown.items()},
        "breakdown_timing": ("one profiled step per class" +
                             (", every cache refresh on the call's stream (kernels alone)"
                              if overlap else "")),
        "forward_ms": round(fwd_ms, 3),
    }
    if not args.no_sweep:
        out["affine_hbm_sweep"] = [affine_sweep(torch, binding, t) for t in (1 << 20, 1 << 22)]
    z_host, params = r.z.detach().cpu().numpy(), r.params
    if not args.no_other_configs:
        del r
        torch.cuda.empty_cache()
        out["other_configs"] = {}
        for name in OTHER_CONFIGS:
            if name != w.name:
                out["other_configs"][name] = quick_config(name, torch, binding, synth, 3, 1)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, params, z_host, synth, args.cpu_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
