"""Deep-shallow flow f = f_D o f_S on one GPU, with the pipelined inverse.

The shallow stack f_S (alternating-direction AF blocks) maps every frame on
its own, u_n = f_S(x_n); the deep causal block f_D maps the whole sequence,
z = f_D(u).  Sampling inverts f_D frame by frame (block-wise Jacobi with one
frame per block, the previous frame as the warm start, the finished frames'
K/V in the cache) and f_S per frame.  Because f_S^-1 of frame n only needs
u_n, it runs on a second stream, driven by a second host thread, while f_D^-1
works on frame n+1: the deep block keeps running and the shallow stack
consumes its output.  The pipelined inverse inverts f_D in one call over all
frames (the same results as one call per frame) and learns from the library's
block-done notification when each frame's tokens are final.

Method: STARFlow-V notes (papernotes.org), 整体框架 (f_theta = f_D o f_S,
u = f_S(x), z = f_D(u); f_D^-1 causal over frames, f_S^-1 per frame),
关键设计 1 (the likelihood factorises into the deep term and one shallow
Jacobian factor per frame), 关键设计 3 (block-wise Jacobi, warm start; f_D
runs without pause while f_S consumes its output in parallel, so the latency
is set by the deep block).

Every step runs through the C ABI (af_forward, af_inverse_jacobi,
af_refresh_kv, af_plan_set_block_done); this module only schedules calls and
streams.
"""
from __future__ import annotations

import queue
import threading
from typing import Optional, Tuple

import numpy as np
import torch

from .binding import AFPlan, af_inverse_jacobi


class DeepShallowFlow:
    """f = f_D o f_S over sequences of frames of ``frame_len`` tokens.

    ``deep`` is a single-block plan whose max_len covers the whole sequence;
    ``shallow`` is a stack plan whose max_len covers one frame."""

    def __init__(self, deep: AFPlan, shallow: AFPlan, frame_len: int):
        if deep.T != 1:
            raise ValueError("the deep flow is a single AF block")
        if deep.cfg.C != shallow.cfg.C:
            raise ValueError("deep and shallow flows must share C")
        if shallow.cfg.max_len < frame_len:
            raise ValueError("the shallow flow must cover one frame")
        self.deep, self.shallow, self.F = deep, shallow, frame_len

    def _split(self, t: torch.Tensor) -> int:
        N, L, C = t.shape
        if L % self.F:
            raise ValueError("sequence length must be a multiple of frame_len")
        return L // self.F

    # forward ----------------------------------------------------------------
    def forward(self, x: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
        """z = f_D(f_S(x)) and logdet[n] = log|det dz/dx| = the deep log-det
        plus the shallow log-dets of the sample's frames."""
        N, L, C = x.shape
        nf = self._split(x)
        # the shallow stack over all frames sums each sequence's frame factors
        # into logdet[n]; the deep block's forward then adds its own term
        u_f, ld = self.shallow.forward(x.reshape(N * nf, self.F, C).contiguous(),
                                       frames_per_entry=nf)
        z, ld = self.deep.forward(u_f.reshape(N, L, C).contiguous(), logdet=ld,
                                  accumulate=True)
        return z, ld

    # inverse ----------------------------------------------------------------
    def _deep_frame(self, z, u, n, tau, max_iters, stream):
        """Invert f_D on frame n (positions n*F..) after frames 0..n-1, then
        refresh the frame's K/V from its final tokens for the frames after."""
        F = self.F
        zn = z[:, n * F:(n + 1) * F]
        if n == 0:
            un, it = self.deep.inverse_jacobi(zn, F, tau, max_iters, stream=stream)
        else:
            un, it = self.deep.inverse_jacobi(
                zn, F, tau, max_iters, init="given",
                x_init=u[:, (n - 1) * F:n * F].contiguous(), prefix_len=n * F,
                x_last=u[:, n * F - 1].contiguous(), stream=stream)
        with torch.cuda.stream(stream):
            u[:, n * F:(n + 1) * F].copy_(un)
            done = torch.cuda.Event()
            done.record(stream)
            if int(it[0, 0]) < F and (n + 1) * F < u.shape[1]:
                self.deep.refresh_kv(un, prefix_len=n * F,
                                     x_last=None if n == 0 else u[:, n * F - 1].contiguous(),
                                     stream=stream)
        return int(it[0, 0]), done

    def _shallow_frame(self, u, x, n, tau, max_iters, stream):
        F = self.F
        xn, it = self.shallow.inverse_jacobi(u[:, n * F:(n + 1) * F].contiguous(), F, tau,
                                             max_iters, stream=stream)
        with torch.cuda.stream(stream):
            x[:, n * F:(n + 1) * F].copy_(xn)
        return it[:, 0].copy()

    def inverse(self, z: torch.Tensor, tau: float = 1e-3, max_iters: int = 0,
                pipelined: bool = True):
        """x = f_S^-1(f_D^-1(z)) for one sequence (z [1, n_frames*F, C]).
        Returns (x, deep updates per frame [n_frames], shallow updates per
        frame and stack block [n_frames, T]).  With pipelined=False the frames
        run one after another on the current stream (same results)."""
        if z.shape[0] != 1:
            raise ValueError("one sequence at a time")
        nf = self._split(z)
        u = torch.empty_like(z)
        x = torch.empty_like(z)
        it_d = np.zeros(nf, dtype=np.int32)
        it_s = np.zeros((nf, self.shallow.T), dtype=np.int32)
        # workspaces sized up front: a reallocation would drop the KV cache
        self.deep.workspace(1, self.F)
        self.shallow.workspace(1, self.F)
        if not pipelined:
            st = torch.cuda.current_stream()
            for n in range(nf):
                it_d[n], _ = self._deep_frame(z, u, n, tau, max_iters, st)
                it_s[n] = self._shallow_frame(u, x, n, tau, max_iters, st)
            return x, it_d, it_s

        s_deep, s_shallow = torch.cuda.Stream(), torch.cuda.Stream()
        s_deep.wait_stream(torch.cuda.current_stream())
        s_shallow.wait_stream(torch.cuda.current_stream())
        ready: "queue.Queue[Optional[Tuple[int, torch.cuda.Event]]]" = queue.Queue()
        errors = []

        # each thread allocates on its own stream, so a buffer freed by one
        # thread is never reused by the other while a copy is still queued
        def consumer():
            try:
                with torch.cuda.stream(s_shallow):
                    while True:
                        item = ready.get()
                        if item is None:
                            return
                        n, ev = item
                        s_shallow.wait_event(ev)
                        it_s[n] = self._shallow_frame(u, x, n, tau, max_iters, s_shallow)
            except BaseException as e:  # surfaced to the caller below
                errors.append(e)

        th = threading.Thread(target=consumer, daemon=True)
        th.start()

        # f_D^-1 as one call over all frames (previous-frame warm start, each
        # finished frame's cache refreshed inside the call, beside the next
        # frame's first update); the library reports each frame as soon as
        # its tokens are final on the deep stream
        def frame_done(_t, b):
            ev = torch.cuda.Event()
            ev.record(s_deep)
            ready.put((b, ev))

        iters = np.zeros((1, nf), dtype=np.int32)
        try:
            with torch.cuda.stream(s_deep):
                ws = self.deep.workspace(1, self.F)
                self.deep._use(s_deep)
                self.deep.set_block_done(frame_done)
                try:
                    af_inverse_jacobi(self.deep, z, self.F, tau, max_iters, "prev_frame", None,
                                      self.F, 0, None, u, iters, ws, s_deep)
                finally:
                    self.deep.set_block_done(None)
        finally:
            ready.put(None)
            th.join()
        if errors:
            raise errors[0]
        it_d[:] = iters[0]
        torch.cuda.current_stream().wait_stream(s_deep)
        torch.cuda.current_stream().wait_stream(s_shallow)
        return x, it_d, it_s


def stream_inverse(plan: AFPlan, z: torch.Tensor, window: int, overlap: int, B: int,
                   tau: float = 1e-3, max_iters: int = 0, frame_len: int = 0,
                   stream=None):
    """Invert a sequence longer than the block's positions by a sliding window
    (STARFlow-V notes, 一个完整示例, streaming generation): the first chunk
    inverts z[:, :window] at positions 0..window-1; each later chunk re-encodes
    the last ``overlap`` generated tokens into a fresh KV cache at positions
    0..overlap-1 (af_prefill) and inverts the next window - overlap latents
    after them.  Inside a chunk: block-wise Jacobi with blocks of B tokens,
    zero init or the previous-frame warm start (frame_len > 0).  Needs
    window <= the plan's max_len.  Returns (x, per-chunk iteration arrays)."""
    if plan.T != 1:
        raise ValueError("streaming runs on a single AF block")
    if not 0 <= overlap < window <= plan.cfg.max_len:
        raise ValueError("need 0 <= overlap < window <= max_len")
    N, L, C = z.shape
    kw = dict(init="prev_frame", frame_len=frame_len) if frame_len > 0 else {}
    x = torch.empty_like(z)
    plan.workspace(N, max(B, overlap))
    its, done = [], 0
    while done < L:
        if done == 0:
            n = min(window, L)
            xc, it = plan.inverse_jacobi(z[:, :n].contiguous(), B, tau, max_iters,
                                         stream=stream, **kw)
        else:
            n = min(window - overlap, L - done)
            ov = x[:, done - overlap:done].contiguous()
            if overlap > 0:
                plan.prefill(ov, rows=B, stream=stream)
            xc, it = plan.inverse_jacobi(
                z[:, done:done + n].contiguous(), B, tau, max_iters, prefix_len=overlap,
                x_last=ov[:, -1].contiguous() if overlap > 0 else None, stream=stream, **kw)
        x[:, done:done + n].copy_(xc)
        its.append(it[0].copy())
        done += n
    return x, its
