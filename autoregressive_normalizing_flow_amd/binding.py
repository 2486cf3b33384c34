"""Thin ctypes binding of ``libafhip.so`` (the C ABI in include/af.h).

Argument marshalling only: every step of the AF block runs in the library's
HIP kernels.  PyTorch provides device memory (tensors) and the stream.  The
functions keep the C names (``af_forward``, ``af_inverse_jacobi``, ...);
``AFPlan`` bundles a plan with its uploaded weights and a workspace.

The library must be built first (``python -m
autoregressive_normalizing_flow_amd.build``); a missing library raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Callable, Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch  # loads the HIP runtime the library then shares

from . import synth

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libafhip.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "af.h")

AF_OK, AF_ERR_ARG, AF_ERR_HIP, AF_ERR_WORKSPACE, AF_ERR_NONFINITE, AF_ERR_UNSUPPORTED = range(6)
AF_F32, AF_BF16 = 0, 1
AF_FWD_ACCUMULATE, AF_FWD_CHECK_FINITE = 1, 2
INIT = {"zero": 0, "given": 1, "prev_frame": 2}
KERNEL_CLASSES = ("embed", "layernorm", "gemm_qkv", "gemm_o", "gemm_mlp1",
                  "gemm_mlp2", "gemm_head", "attention", "affine")


class AFError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


class af_block_cfg(ctypes.Structure):
    _fields_ = [("C", ctypes.c_int), ("d", ctypes.c_int), ("n_heads", ctypes.c_int),
                ("n_layers", ctypes.c_int), ("max_len", ctypes.c_int),
                ("dtype", ctypes.c_int)]


_P = ctypes.c_void_p
_PP = ctypes.POINTER(ctypes.c_void_p)


class af_block_weights(ctypes.Structure):
    _fields_ = [(n, _P) for n in ("w_in", "b_in", "pos", "ln_f_g", "ln_f_b",
                                  "w_head", "b_head")] + \
               [(n, _PP) for n in ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_o",
                                   "b_o", "ln2_g", "ln2_b", "w_1", "b_1",
                                   "w_2", "b_2")]


_lib = None


def load_library() -> ctypes.CDLL:
    """Load libafhip.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m autoregressive_normalizing_flow_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    st = ctypes.c_int
    sz = ctypes.c_size_t
    i = ctypes.c_int
    f = ctypes.c_float
    L.af_plan_create.argtypes = [ctypes.POINTER(af_block_cfg), i,
                                 ctypes.POINTER(af_block_weights), ctypes.POINTER(_P)]
    L.af_plan_create.restype = st
    L.af_plan_destroy.argtypes = [_P]
    L.af_plan_destroy.restype = None
    L.af_workspace_bytes.argtypes = [_P, i, i]
    L.af_workspace_bytes.restype = sz
    L.af_cache_bytes.argtypes = [_P, i]
    L.af_cache_bytes.restype = sz
    L.af_forward.argtypes = [_P, _P, _P, _P, i, i, i, i, _P, sz, _P]
    L.af_forward.restype = st
    L.af_prefill.argtypes = [_P, _P, i, i, _P, sz, _P]
    L.af_prefill.restype = st
    L.af_refresh_kv.argtypes = [_P, _P, i, i, i, _P, _P, sz, _P]
    L.af_refresh_kv.restype = st
    L.af_inverse_jacobi.argtypes = [_P, _P, i, i, i, f, i, i, _P, i, i, _P, _P,
                                    ctypes.POINTER(ctypes.c_int32), _P, sz, _P]
    L.af_inverse_jacobi.restype = st
    L.af_profile_enable.argtypes = [_P, ctypes.c_char_p]
    L.af_profile_enable.restype = st
    L.af_profile_disable.argtypes = [_P]
    L.af_profile_disable.restype = st
    L.af_profile_read.argtypes = [_P, ctypes.POINTER(ctypes.c_int),
                                  ctypes.POINTER(ctypes.c_double),
                                  ctypes.POINTER(ctypes.c_double)]
    L.af_profile_read.restype = st
    L.af_plan_set_fused_refresh.argtypes = [_P, i]
    L.af_plan_set_fused_refresh.restype = st
    L.af_plan_set_graphs.argtypes = [_P, i]
    L.af_plan_set_graphs.restype = st
    L.af_plan_set_row_split.argtypes = [_P, i]
    L.af_plan_set_row_split.restype = st
    L.af_plan_set_overlap_refresh.argtypes = [_P, i]
    L.af_plan_set_overlap_refresh.restype = st
    L.af_plan_set_block_done.argtypes = [_P, _BLOCK_DONE_FN, _P]
    L.af_plan_set_block_done.restype = st
    L.af_plan_set_device_loop.argtypes = [_P, i]
    L.af_plan_set_device_loop.restype = st
    L.af_plan_graph_stats.argtypes = [_P, ctypes.POINTER(ctypes.c_longlong),
                                      ctypes.POINTER(ctypes.c_longlong)]
    L.af_plan_graph_stats.restype = st
    L.af_plan_last_residual.argtypes = [_P, i, ctypes.POINTER(ctypes.c_float)]
    L.af_plan_last_residual.restype = st
    L.afk_affine_partials_bytes.argtypes = [i, i, i]
    L.afk_affine_partials_bytes.restype = sz
    L.afk_affine.argtypes = [i, _P, _P, _P, i, i, i, _P, _P, sz, i, _P]
    L.afk_affine.restype = st
    L.afk_affine_noalloc.argtypes = [i, _P, _P, _P, i, i, i, _P, _P]
    L.afk_affine_noalloc.restype = st
    L.afk_stream_copy.argtypes = [_P, _P, sz, _P]
    L.afk_stream_copy.restype = st
    L.afk_attention_workspace_bytes.argtypes = [i, i, i, i, i]
    L.afk_attention_workspace_bytes.restype = sz
    L.afk_attention.argtypes = [_P, _P, _P, _P, i, i, i, i, i, i, _P, sz, _P]
    L.afk_attention.restype = st
    L.afk_gemm_bf16.argtypes = [_P, _P, _P, _P, i, i, i, _P]
    L.afk_gemm_bf16.restype = st
    L.af_status_str.argtypes = [st]
    L.af_status_str.restype = ctypes.c_char_p
    L.af_last_error.argtypes = []
    L.af_last_error.restype = ctypes.c_char_p
    L.af_abi_version.argtypes = []
    L.af_abi_version.restype = ctypes.c_int
    _lib = L
    return L


# af_block_done_fn: void (*)(void *user, int stack_block, int jacobi_block)
_BLOCK_DONE_FN = ctypes.CFUNCTYPE(None, ctypes.c_void_p, ctypes.c_int, ctypes.c_int)


def header_functions() -> List[str]:
    """Names of the functions declared in include/af.h."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(af[k]?_[a-z_0-9]+)\s*\(", text)))


def _check(status: int, where: str):
    if status != AF_OK:
        L = load_library()
        raise AFError(status, where, L.af_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _tok(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype != torch.float32 or not t.is_contiguous() or t.device.type != "cuda":
        raise ValueError(f"{name} must be a contiguous fp32 CUDA tensor")
    return t


# ---------------------------------------------------------------------------
# plan with uploaded weights
# ---------------------------------------------------------------------------
class AFPlan:
    """A stack of AF blocks (block t is L->R for even t, R->L for odd t) with
    its weights on the device.  ``params`` are the per-block dicts of
    ``synth.make_params`` (fp32 arrays, bf16-exact for the per-layer matrices
    on the bf16 path)."""

    def __init__(self, cfg: synth.BlockCfg, params: Sequence[Dict],
                 device: str = "cuda:0"):
        self.L = load_library()
        self.cfg = cfg
        self.device = torch.device(device)
        self.T = len(params)
        mat_dtype = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        self._keep = []
        ws_structs = (af_block_weights * self.T)()

        def up(a, dtype=torch.float32):
            t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(self.device)
            t = t.to(dtype) if dtype != torch.float32 else t
            self._keep.append(t)
            return ctypes.c_void_p(t.data_ptr())

        for bi, p in enumerate(params):
            w = ws_structs[bi]
            for n in ("w_in", "b_in", "pos", "ln_f_g", "ln_f_b", "w_head", "b_head"):
                setattr(w, n, up(p[n]))
            for n in ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o", "ln2_g",
                      "ln2_b", "w_1", "b_1", "w_2", "b_2"):
                dt = mat_dtype if n in synth.BF16_MATRICES else torch.float32
                arr = (ctypes.c_void_p * cfg.n_layers)(
                    *[up(layer[n], dt) for layer in p["layers"]])
                self._keep.append(arr)
                setattr(w, n, ctypes.cast(arr, _PP))
        c = af_block_cfg(cfg.C, cfg.d, cfg.n_heads, cfg.n_layers, cfg.max_len,
                         AF_BF16 if cfg.dtype == "bf16" else AF_F32)
        h = _P()
        with torch.cuda.device(self.device):
            _check(self.L.af_plan_create(ctypes.byref(c), self.T, ws_structs,
                                         ctypes.byref(h)), "af_plan_create")
        self.handle = h
        self._ws = None
        self._ws_key = None
        self._ws_stream = None

    def __del__(self):
        try:
            if getattr(self, "handle", None):
                self.L.af_plan_destroy(self.handle)
                self.handle = None
        except Exception:
            pass

    # workspace -------------------------------------------------------------
    def workspace_bytes(self, batch: int, rows: int) -> int:
        return int(self.L.af_workspace_bytes(self.handle, batch, rows))

    def workspace(self, batch: int, rows: int) -> torch.Tensor:
        """A workspace for (batch, rows), reused while large enough.  Its KV
        cache survives between calls with the same batch."""
        need = self.workspace_bytes(batch, rows)
        if self._ws is None or self._ws_key[0] != batch or self._ws.numel() < need:
            old, old_batch = self._ws, (self._ws_key[0] if self._ws_key else None)
            if old is not None and self._ws_stream is not None:
                # an inverse call may return with kernels still writing the
                # old workspace on the stream it used: let them finish before
                # its cache is copied and its memory handed back
                self._ws_stream.synchronize()
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
            self._ws_key = (batch, rows)
            if old is not None and old_batch == batch:
                # a larger workspace for the same batch keeps the KV cache
                cache = int(self.L.af_cache_bytes(self.handle, batch))
                self._ws[:cache].copy_(old[:cache])
        return self._ws

    def _use(self, stream):
        """Remember the stream a call runs on: later workspace growth waits
        for it."""
        self._ws_stream = stream if stream is not None else torch.cuda.current_stream()

    # entry points ----------------------------------------------------------
    def forward(self, x: torch.Tensor, stream=None, logdet: Optional[torch.Tensor] = None,
                frames_per_entry: int = 1, accumulate: bool = False,
                check_finite: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
        """z = f(x) and the log-det per entry (af_forward): one entry per
        sample, or per group of ``frames_per_entry`` consecutive samples;
        ``accumulate`` adds into the given ``logdet``."""
        _tok(x, "x")
        N, L, C = x.shape
        z = torch.empty_like(x)
        if logdet is None:
            logdet = torch.empty(N // frames_per_entry, dtype=torch.float32, device=x.device)
        ws = self.workspace(N, L)
        flags = (AF_FWD_ACCUMULATE if accumulate else 0) | \
                (AF_FWD_CHECK_FINITE if check_finite else 0)
        af_forward(self, x, z, logdet, ws, stream, frames_per_entry, flags)
        return z, logdet

    def prefill(self, x_prefix: torch.Tensor, rows: Optional[int] = None, stream=None):
        _tok(x_prefix, "x_prefix")
        N, P, C = x_prefix.shape
        ws = self.workspace(N, max(P, rows or 0))
        self._use(stream)
        af_prefill(self, x_prefix, ws, stream)

    def refresh_kv(self, x: torch.Tensor, prefix_len: int = 0,
                   x_last: Optional[torch.Tensor] = None, stream=None):
        """Recompute the cache rows prefix_len.. from their final tokens x."""
        _tok(x, "x")
        N, L, C = x.shape
        ws = self.workspace(N, max(L, self._ws_key[1] if self._ws_key else 0))
        self._use(stream)
        af_refresh_kv(self, x, prefix_len, x_last, ws, stream)

    def inverse_jacobi(self, z: torch.Tensor, B: int, tau: float = 1e-3,
                       max_iters: int = 0, init: str = "zero",
                       x_init: Optional[torch.Tensor] = None, frame_len: int = 0,
                       prefix_len: int = 0, x_last: Optional[torch.Tensor] = None,
                       stream=None) -> Tuple[torch.Tensor, np.ndarray]:
        _tok(z, "z")
        N, L, C = z.shape
        x = torch.empty_like(z)
        nb = (L + B - 1) // B
        iters = np.zeros((self.T, nb), dtype=np.int32)
        # rows for two blocks when a block's cache refresh shares the next
        # block's first pass
        rows = min(2 * B, L) if nb > 1 and getattr(self, "_fused_refresh", False) else min(B, L)
        ws = self.workspace(N, max(rows, self._ws_key[1] if self._ws_key else 0))
        self._use(stream)
        af_inverse_jacobi(self, z, B, tau, max_iters, init, x_init, frame_len,
                          prefix_len, x_last, x, iters, ws, stream)
        return x, iters

    def last_residual(self, N: int) -> np.ndarray:
        """[N, 2] (sum of squared change, sum of squares) of the last Jacobi
        update of the last inverse call, as its stop test saw them."""
        out = np.zeros((N, 2), dtype=np.float32)
        _check(self.L.af_plan_last_residual(
            self.handle, N, out.ctypes.data_as(ctypes.POINTER(ctypes.c_float))),
            "af_plan_last_residual")
        return out

    # profiling -------------------------------------------------------------
    def profile_enable(self, kernel_class: str):
        _check(self.L.af_profile_enable(self.handle, kernel_class.encode()),
               "af_profile_enable")

    def profile_disable(self):
        _check(self.L.af_profile_disable(self.handle), "af_profile_disable")

    def profile_read(self) -> Tuple[int, float]:
        """(launches, summed ms) of the profiled class since profile_enable."""
        n, ms, _ = self.profile_read_work()
        return n, ms

    def profile_read_work(self) -> Tuple[int, float, float]:
        """(launches, summed ms, summed algorithmic work: flops, or bytes for
        the affine class) of the profiled class since profile_enable."""
        n = ctypes.c_int()
        ms = ctypes.c_double()
        work = ctypes.c_double()
        _check(self.L.af_profile_read(self.handle, ctypes.byref(n), ctypes.byref(ms),
                                      ctypes.byref(work)), "af_profile_read")
        return n.value, ms.value, work.value

    def set_fused_refresh(self, enable: bool):
        _check(self.L.af_plan_set_fused_refresh(self.handle, int(bool(enable))),
               "af_plan_set_fused_refresh")
        self._fused_refresh = bool(enable)

    # graph replay of the Jacobi update ------------------------------------
    def set_row_split(self, enable: bool):
        _check(self.L.af_plan_set_row_split(self.handle, int(bool(enable))),
               "af_plan_set_row_split")

    def set_overlap_refresh(self, enable: bool):
        _check(self.L.af_plan_set_overlap_refresh(self.handle, int(bool(enable))),
               "af_plan_set_overlap_refresh")

    def set_block_done(self, fn: Optional[Callable[[int, int], None]]):
        """fn(stack_block, jacobi_block) is called on the calling thread of
        inverse_jacobi once that block's tokens are final on the call's stream
        (record an event there to wait for them from another stream); None
        turns it off.  Exceptions raised by fn are kept and re-raised by the
        next set_block_done(None)."""
        if fn is None:
            _check(self.L.af_plan_set_block_done(self.handle, _BLOCK_DONE_FN(), None),
                   "af_plan_set_block_done")
            self._done_cb = None
            errs, self._done_errors = getattr(self, "_done_errors", []), []
            if errs:
                raise errs[0]
            return
        self._done_errors = []

        def tramp(_user, t, b):
            try:
                fn(t, b)
            except BaseException as e:  # no exception may cross the C ABI
                self._done_errors.append(e)
        self._done_cb = _BLOCK_DONE_FN(tramp)   # kept alive with the plan
        _check(self.L.af_plan_set_block_done(self.handle, self._done_cb, None),
               "af_plan_set_block_done")

    def set_device_loop(self, enable: bool):
        _check(self.L.af_plan_set_device_loop(self.handle, int(bool(enable))),
               "af_plan_set_device_loop")

    def set_graphs(self, enable: bool):
        _check(self.L.af_plan_set_graphs(self.handle, int(bool(enable))), "af_plan_set_graphs")

    def graph_stats(self) -> Tuple[int, int]:
        c = ctypes.c_longlong()
        r = ctypes.c_longlong()
        _check(self.L.af_plan_graph_stats(self.handle, ctypes.byref(c), ctypes.byref(r)),
               "af_plan_graph_stats")
        return c.value, r.value


# ---------------------------------------------------------------------------
# C-named entry points (tensors in, status checked)
# ---------------------------------------------------------------------------
def af_forward(plan: AFPlan, x, z, logdet, ws, stream=None, frames_per_entry: int = 1,
               flags: int = 0):
    N, L, C = x.shape
    plan._use(stream)
    _check(plan.L.af_forward(plan.handle, _ptr(x), _ptr(z), _ptr(logdet), N, L,
                             frames_per_entry, flags, _ptr(ws), ws.numel(),
                             _stream(stream)), "af_forward")


def af_prefill(plan: AFPlan, x_prefix, ws, stream=None):
    N, P, C = x_prefix.shape
    _check(plan.L.af_prefill(plan.handle, _ptr(x_prefix), N, P, _ptr(ws),
                             ws.numel(), _stream(stream)), "af_prefill")


def af_refresh_kv(plan: AFPlan, x, prefix_len: int, x_last, ws, stream=None):
    N, L, C = x.shape
    _check(plan.L.af_refresh_kv(plan.handle, _ptr(x), N, L, prefix_len, _ptr(x_last),
                                _ptr(ws), ws.numel(), _stream(stream)), "af_refresh_kv")


def af_inverse_jacobi(plan: AFPlan, z, B, tau, max_iters, init, x_init, frame_len,
                      prefix_len, x_last, x, iters: np.ndarray, ws, stream=None):
    N, L, C = z.shape
    if x_init is not None:
        _tok(x_init, "x_init")
    if x_last is not None:
        _tok(x_last, "x_last")
    assert iters.dtype == np.int32 and iters.flags.c_contiguous
    _check(plan.L.af_inverse_jacobi(
        plan.handle, _ptr(z), N, L, B, ctypes.c_float(tau), max_iters,
        INIT[init] if isinstance(init, str) else int(init), _ptr(x_init), frame_len,
        prefix_len, _ptr(x_last), _ptr(x),
        iters.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), _ptr(ws), ws.numel(),
        _stream(stream)), "af_inverse_jacobi")


def afk_affine(mode: int, head, src, dst, N: int, rows: int, C: int, res,
               partials, check: bool = False, stream=None):
    L = load_library()
    _check(L.afk_affine(mode, _ptr(head), _ptr(src), _ptr(dst), N, rows, C,
                        _ptr(res), _ptr(partials), partials.numel(), int(check),
                        _stream(stream)), "afk_affine")


def afk_affine_noalloc(mode: int, head, src, dst, N: int, rows: int, C: int, res,
                       stream=None):
    """afk_affine with its scratch in the library's static device array."""
    L = load_library()
    _check(L.afk_affine_noalloc(mode, _ptr(head), _ptr(src), _ptr(dst), N, rows, C, _ptr(res),
                                _stream(stream)), "afk_affine_noalloc")


def afk_attention(q: torch.Tensor, kc: torch.Tensor, vt: torch.Tensor, pos_base: int,
                  stream=None) -> torch.Tensor:
    """One layer's bf16 attention over a KV cache: q [N, R, H*dh] (times
    log2(e)/sqrt(dh)), kc [N, H, Lcap, dh], vt [N, H, dh, Lcap]; returns out
    [N, R, H*dh] bf16."""
    assert q.dtype == kc.dtype == vt.dtype == torch.bfloat16
    N, R, d = q.shape
    _, H, Lcap, dh = kc.shape
    assert d == H * dh and tuple(vt.shape) == (N, H, dh, Lcap)
    L = load_library()
    nb = int(L.afk_attention_workspace_bytes(N, R, H, dh, pos_base))
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=q.device)
    out = torch.empty_like(q)
    _check(L.afk_attention(_ptr(q), _ptr(kc), _ptr(vt), _ptr(out), N, R, H, dh, Lcap, pos_base,
                           _ptr(ws), ws.numel(), _stream(stream)), "afk_attention")
    return out


def afk_stream_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """dst <- src (same byte size) with the library's streaming copy kernel."""
    nbytes = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() == nbytes
    _check(load_library().afk_stream_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)),
           "afk_stream_copy")


def afk_affine_partials_bytes(N: int, rows: int, C: int) -> int:
    return int(load_library().afk_affine_partials_bytes(N, rows, C))


def afk_gemm_bf16(a: torch.Tensor, w: torch.Tensor, bias: Optional[torch.Tensor],
                  stream=None) -> torch.Tensor:
    assert a.dtype == torch.bfloat16 and w.dtype == torch.bfloat16
    M, K = a.shape
    N = w.shape[0]
    y = torch.empty(M, N, dtype=torch.float32, device=a.device)
    _check(load_library().afk_gemm_bf16(_ptr(a), _ptr(w), _ptr(bias), _ptr(y), M, N,
                                        K, _stream(stream)), "afk_gemm_bf16")
    return y
