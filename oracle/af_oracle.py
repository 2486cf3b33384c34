"""CPU fp64 oracle of the affine autoregressive-flow (AF) block.

TEST INFRASTRUCTURE ONLY.  This module is the correctness reference for the
HIP path.  Only the test-suite, the package's smoke check and the benchmark's
CPU-baseline leg may import it; the product path never does.  It shares no
code with the HIP path: the two only receive the same seeded arrays.

Everything is plain NumPy in float64, written for a reader to check against
the STARFlow-V notes (papernotes.org, "STARFlow-V: End-to-End Video Generative
Modeling with Autoregressive Normalizing Flows"), cited below as [notes, <section>]:

* [notes, 关键设计 1, affine AF equation]   z = (x - mu(x*m)) / sigma(x*m), sigma > 0,
  m the self-exclusive causal mask; T >= 3 blocks with alternating directions.
* [notes, 整体框架]  the shallow blocks alternate left-to-right / right-to-left
  masks; inverting f_D proceeds token by token, frame by frame.
* [notes, 关键设计 3, Jacobi fixed-point equation]  x = mu(x*m) + sigma(x*m)*z is
  solved by x^(k+1) = mu(x^(k)*m) + sigma(x^(k)*m)*z from x^(0) until
  ||x^(k+1)-x^(k)||^2 / ||x^(k+1)||^2 < tau (default 1e-3); blocks of B tokens
  run one after another, tokens inside a block in parallel, finished blocks
  feed a KV cache, a new frame starts from the previous frame's solution.
* [notes, 损失函数, L_NF]  the objective carries log|det J| of the forward map.
* [notes, 一个完整示例, I2V]  observed frames are forward-encoded into the KV
  cache before autoregressive continuation.
* [notes, 一个完整示例, streaming]  beyond the trained length the deep block
  slides a window: after a chunk, the last overlap latents are re-run through
  f_D to rebuild the KV cache and the next chunk continues from them.
* [notes, 整体框架 and 关键设计 1]  the full flow is f = f_D o f_S: the shallow
  stack maps each frame on its own (u_n = f_S(x_n)), the deep causal block maps
  the whole sequence (z = f_D(u)); the likelihood factorises into the deep
  term and one shallow Jacobian factor per frame; sampling inverts f_D frame
  by frame and then f_S per frame.

Readings where the notes leave a step open (each one plain and standard):
  R1  mask m: shift the sequence by one token (zero at the start of the
      sequence), then inclusive causal attention.  mu_t, sigma_t thus see
      exactly x_<t.
  R2  network: learned input projection + learned absolute position table,
      pre-LN Transformer layers (LayerNorm eps 1e-5, attention scale
      1/sqrt(d_head), exact erf GELU, MLP width 4d), final LayerNorm and a
      linear head whose first C outputs are mu and last C are raw.  QKV
      columns are [Q | K | V], heads contiguous inside each.
  R3  sigma = exp(0.5 * tanh(raw)), so log sigma = 0.5 * tanh(raw).
  R4  logdet per sample = -sum_{t,c} log sigma = log|det dz/dx|; a stack sums.
  R5  batch residual: r_n per sample over the whole block; a block stops when
      every sample has r_n < tau (strict).  0/0 -> 0, x/0 -> inf.
  R6  iters counts the updates made, including the one that passes the test;
      at most Bb (the block length), after which the block is exact.
  R7  a finished block's K/V are recomputed from its final x (refresh).
  R8  positions are global token indices in processing order; R->L blocks
      process flip(x) and return flip of the result.
  R9  tau <= 0 forces exactly min(max_iters, Bb) updates per block.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

try:  # exact erf for GELU; scipy is a library primitive here
    from scipy.special import erf as _erf
except ImportError:  # pragma: no cover - scipy is present in this image
    _erf = np.vectorize(math.erf)

LN_EPS = 1e-5

__all__ = [
    "to64", "layernorm", "gelu", "attention", "net_rows", "shift",
    "forward_block", "forward_stack", "inverse_sequential_block",
    "inverse_sequential_stack", "inverse_jacobi_block", "inverse_jacobi_stack",
    "prefill", "jacobian_bruteforce", "direction_of", "forward_deep_shallow",
    "inverse_deep_shallow", "inverse_streaming",
]


# --------------------------------------------------------------------------
# parameters
# --------------------------------------------------------------------------
def to64(p: Dict) -> Dict:
    """Upcast one block's parameters (fp32 arrays holding the stored values)
    to float64.  The oracle computes with the stored values exactly."""
    out = {k: np.asarray(v, dtype=np.float64) for k, v in p.items() if k != "layers"}
    out["layers"] = [{k: np.asarray(v, dtype=np.float64) for k, v in l.items()}
                     for l in p["layers"]]
    return out


# --------------------------------------------------------------------------
# textbook pieces of the causal Transformer (reading R2)
# --------------------------------------------------------------------------
def layernorm(h: np.ndarray, g: np.ndarray, b: np.ndarray) -> np.ndarray:
    """LayerNorm over the last axis: (h - mean) / sqrt(var + eps) * g + b,
    with the biased variance."""
    mean = h.mean(axis=-1, keepdims=True)
    var = ((h - mean) ** 2).mean(axis=-1, keepdims=True)
    return (h - mean) / np.sqrt(var + LN_EPS) * g + b


def gelu(u: np.ndarray) -> np.ndarray:
    """Exact GELU: u * Phi(u) = 0.5 u (1 + erf(u / sqrt 2))."""
    return 0.5 * u * (1.0 + _erf(u / math.sqrt(2.0)))


def attention(q, k, v, q_pos, k_pos):
    """Causal multi-head attention.  q [N,H,R,dh], k/v [N,H,S,dh]; query at
    position q_pos[i] may attend key j iff k_pos[j] <= q_pos[i] (inclusive)."""
    dh = q.shape[-1]
    scores = q @ np.swapaxes(k, -1, -2) / math.sqrt(dh)          # [N,H,R,S]
    allowed = k_pos[None, :] <= q_pos[:, None]                   # [R,S]
    scores = np.where(allowed, scores, -np.inf)
    scores = scores - scores.max(axis=-1, keepdims=True)
    w = np.exp(scores)
    w = w / w.sum(axis=-1, keepdims=True)
    return w @ v                                                  # [N,H,R,dh]


def _split_heads(a: np.ndarray, n_heads: int) -> np.ndarray:
    N, R, d = a.shape
    return a.reshape(N, R, n_heads, d // n_heads).transpose(0, 2, 1, 3)


def _merge_heads(a: np.ndarray) -> np.ndarray:
    N, H, R, dh = a.shape
    return a.transpose(0, 2, 1, 3).reshape(N, R, H * dh)


def net_rows(p: Dict, inp: np.ndarray, pos: np.ndarray, n_heads: int,
             cache: Optional[List[Tuple[np.ndarray, np.ndarray]]] = None):
    """The network that maps shifted tokens to (mu, raw)  [notes, 关键设计 1;
    reading R2].

    inp   [N, R, C] shifted inputs of R consecutive rows
    pos   [R] their positions (consecutive, all after the cached ones)
    cache per layer (K, V) of earlier positions 0..S-1, [N, H, S, dh] each
    Returns mu [N,R,C], raw [N,R,C] and the rows' per-layer (K, V).
    """
    C = p["w_in"].shape[1]
    h = inp @ p["w_in"].T + p["b_in"] + p["pos"][pos]
    new_kv = []
    for li, L in enumerate(p["layers"]):
        a = layernorm(h, L["ln1_g"], L["ln1_b"])
        qkv = a @ L["w_qkv"].T + L["b_qkv"]
        d = qkv.shape[-1] // 3
        q = _split_heads(qkv[..., :d], n_heads)
        k = _split_heads(qkv[..., d:2 * d], n_heads)
        v = _split_heads(qkv[..., 2 * d:], n_heads)
        if cache is not None and cache[li][0].shape[2] > 0:
            kc, vc = cache[li]
            k_all = np.concatenate([kc, k], axis=2)
            v_all = np.concatenate([vc, v], axis=2)
            k_pos = np.concatenate([np.arange(kc.shape[2]), pos])
        else:
            k_all, v_all, k_pos = k, v, pos
        att = _merge_heads(attention(q, k_all, v_all, pos, k_pos))
        h = h + att @ L["w_o"].T + L["b_o"]
        a = layernorm(h, L["ln2_g"], L["ln2_b"])
        h = h + gelu(a @ L["w_1"].T + L["b_1"]) @ L["w_2"].T + L["b_2"]
        new_kv.append((k, v))
    hf = layernorm(h, p["ln_f_g"], p["ln_f_b"])
    out = hf @ p["w_head"].T + p["b_head"]
    return out[..., :C], out[..., C:], new_kv


def _empty_cache(p: Dict, N: int, n_heads: int):
    d = p["w_in"].shape[0]
    e = np.zeros((N, n_heads, 0, d // n_heads))
    return [(e.copy(), e.copy()) for _ in p["layers"]]


def _append(cache, kv):
    return [(np.concatenate([kc, k], axis=2), np.concatenate([vc, v], axis=2))
            for (kc, vc), (k, v) in zip(cache, kv)]


def log_sigma(raw: np.ndarray) -> np.ndarray:
    """log sigma = 0.5 * tanh(raw)  (reading R3; sigma > 0 as the affine
    equation of [notes, 关键设计 1] requires)."""
    return 0.5 * np.tanh(raw)


def shift(x: np.ndarray, x_last: Optional[np.ndarray] = None) -> np.ndarray:
    """The self-exclusive mask as a one-token shift (reading R1): row t gets
    x[t-1]; row 0 gets x_last (the token before the sequence) or zeros."""
    out = np.zeros_like(x)
    out[:, 1:] = x[:, :-1]
    if x_last is not None:
        out[:, 0] = x_last
    return out


def direction_of(t: int) -> str:
    """Block t of a stack: even -> left-to-right, odd -> right-to-left
    [notes, 整体框架: alternating masks]."""
    return "l2r" if t % 2 == 0 else "r2l"


def _flip(a: np.ndarray) -> np.ndarray:
    return a[:, ::-1].copy()


# --------------------------------------------------------------------------
# forward  [notes, 关键设计 1, affine AF equation; 损失函数, log|det J|]
# --------------------------------------------------------------------------
def forward_block(p: Dict, x: np.ndarray, n_heads: int, direction: str = "l2r",
                  pos0: int = 0, cache=None, x_last=None):
    """z = (x - mu) / sigma with mu, sigma from the shifted x; returns
    (z [N,L,C], logdet [N]) where logdet = -sum log sigma  (reading R4).
    ``cache``/``pos0``/``x_last`` continue a sequence after a prefix."""
    x = np.asarray(x, dtype=np.float64)
    if direction == "r2l":
        z, ld = forward_block(p, _flip(x), n_heads, "l2r", pos0, cache, x_last)
        return _flip(z), ld
    L = x.shape[1]
    mu, raw, _ = net_rows(p, shift(x, x_last), pos0 + np.arange(L), n_heads, cache)
    ls = log_sigma(raw)
    z = (x - mu) * np.exp(-ls)
    return z, -ls.sum(axis=(1, 2))


def forward_stack(ps: Sequence[Dict], x: np.ndarray, n_heads: int):
    """f = f_{T-1} o ... o f_0 with alternating directions; log-dets add."""
    z = np.asarray(x, dtype=np.float64)
    ld = np.zeros(z.shape[0])
    for t, p in enumerate(ps):
        z, l = forward_block(p, z, n_heads, direction_of(t))
        ld = ld + l
    return z, ld


def prefill(p: Dict, x_prefix: np.ndarray, n_heads: int):
    """Forward-encode observed tokens into the KV cache [notes, 一个完整示例,
    I2V]: returns the per-layer cache of positions 0..P-1 and the last
    observed token (the shifted input of position P)."""
    x_prefix = np.asarray(x_prefix, dtype=np.float64)
    P = x_prefix.shape[1]
    _, _, kv = net_rows(p, shift(x_prefix), np.arange(P), n_heads, None)
    return kv, x_prefix[:, -1].copy()


# --------------------------------------------------------------------------
# exact inverse: token by token  [notes, 整体框架 / 关键设计 3: sequential decode]
# --------------------------------------------------------------------------
def inverse_sequential_block(p: Dict, z: np.ndarray, n_heads: int,
                             direction: str = "l2r", pos0: int = 0,
                             cache=None, x_last=None):
    """The unique solution of the triangular system z_t = (x_t - mu_t)/sigma_t,
    x_t = mu_t(x_<t) + sigma_t(x_<t) * z_t for t = 0, 1, ..."""
    z = np.asarray(z, dtype=np.float64)
    if direction == "r2l":
        return _flip(inverse_sequential_block(p, _flip(z), n_heads, "l2r",
                                              pos0, cache, x_last))
    N, L, C = z.shape
    cache = _empty_cache(p, N, n_heads) if cache is None else cache
    x = np.zeros_like(z)
    prev = np.zeros((N, C)) if x_last is None else np.asarray(x_last, np.float64)
    for t in range(L):
        mu, raw, kv = net_rows(p, prev[:, None, :], np.array([pos0 + t]),
                               n_heads, cache)
        x[:, t] = mu[:, 0] + np.exp(log_sigma(raw[:, 0])) * z[:, t]
        cache = _append(cache, kv)
        prev = x[:, t]
    return x


def inverse_sequential_stack(ps: Sequence[Dict], z: np.ndarray, n_heads: int):
    x = np.asarray(z, dtype=np.float64)
    for t in reversed(range(len(ps))):
        x = inverse_sequential_block(ps[t], x, n_heads, direction_of(t))
    return x


# --------------------------------------------------------------------------
# block-wise Jacobi  [notes, 关键设计 3, Jacobi fixed-point equation]
# --------------------------------------------------------------------------
def block_residual(x_new: np.ndarray, x_old: np.ndarray) -> np.ndarray:
    """Per-sample ||x_new - x_old||^2 / ||x_new||^2 over the block (R5)."""
    num = ((x_new - x_old) ** 2).sum(axis=(1, 2))
    den = (x_new ** 2).sum(axis=(1, 2))
    r = np.empty_like(num)
    for n in range(num.shape[0]):
        if den[n] > 0:
            r[n] = num[n] / den[n]
        else:
            r[n] = 0.0 if num[n] == 0 else np.inf
    return r


def inverse_jacobi_block(p: Dict, z: np.ndarray, n_heads: int, B: int,
                         tau: float = 1e-3, max_iters: int = 0,
                         init: str = "zero", x_init: Optional[np.ndarray] = None,
                         frame_len: int = 0, direction: str = "l2r",
                         pos0: int = 0, cache=None, x_last=None,
                         forced_iters: Optional[Sequence[int]] = None,
                         trace: Optional[list] = None):
    """Video-aware block-wise Jacobi inversion of one AF block.

    Blocks [s, e) of B tokens (the last may be shorter) are solved one after
    another.  Block b starts from x^(0):
      zero        zeros
      given       x_init[:, s:e]
      prev_frame  the already-solved x[:, s-F:e-F] if s >= F, else zeros
    and repeats x^(k) = mu(shift(x[:s] ++ x^(k-1))) + sigma(...) * z[s:e]
    (rows s..e-1, the finished rows' K/V from the cache) until every sample's
    residual is below tau, at most min(max_iters, Bb) times (R6, R9).  The
    finished block's K/V then enter the cache, recomputed from its final x (R7).

    ``forced_iters`` (one count per block) replaces the stop test by a fixed
    number of updates; ``trace`` (a list) receives (block, k, r) per update.
    Returns (x [N,L,C], iters [nb]).
    """
    z = np.asarray(z, dtype=np.float64)
    if direction == "r2l":
        xi = None if x_init is None else _flip(np.asarray(x_init, np.float64))
        x, it = inverse_jacobi_block(p, _flip(z), n_heads, B, tau, max_iters,
                                     init, xi, frame_len, "l2r", pos0, cache,
                                     x_last, forced_iters, trace)
        return _flip(x), it
    N, L, C = z.shape
    cache = _empty_cache(p, N, n_heads) if cache is None else cache
    x = np.zeros_like(z)
    nb = (L + B - 1) // B
    iters = np.zeros(nb, dtype=np.int64)
    first = np.zeros((N, C)) if x_last is None else np.asarray(x_last, np.float64)
    for b in range(nb):
        s, e = b * B, min(L, (b + 1) * B)
        Bb = e - s
        if init == "zero":
            xk = np.zeros((N, Bb, C))
        elif init == "given":
            xk = np.asarray(x_init, np.float64)[:, s:e].copy()
        elif init == "prev_frame":
            xk = x[:, s - frame_len:e - frame_len].copy() if s >= frame_len \
                else np.zeros((N, Bb, C))
        else:
            raise ValueError(init)
        kmax = Bb if max_iters <= 0 else min(max_iters, Bb)
        if forced_iters is not None:
            kmax = min(int(forced_iters[b]), Bb)
        before = first if s == 0 else x[:, s - 1]
        k = 0
        for k in range(1, kmax + 1):
            inp = shift(xk, before)
            mu, raw, _ = net_rows(p, inp, pos0 + np.arange(s, e), n_heads, cache)
            x_new = mu + np.exp(log_sigma(raw)) * z[:, s:e]
            r = block_residual(x_new, xk)
            xk = x_new
            if trace is not None:
                trace.append((b, k, r.copy()))
            if forced_iters is None and tau > 0 and np.all(r < tau):
                break
        x[:, s:e] = xk
        iters[b] = k
        _, _, kv = net_rows(p, shift(xk, before), pos0 + np.arange(s, e),
                            n_heads, cache)
        cache = _append(cache, kv)
    return x, iters


def inverse_jacobi_stack(ps: Sequence[Dict], z: np.ndarray, n_heads: int,
                         B: int, tau: float = 1e-3, max_iters: int = 0,
                         forced_iters: Optional[Sequence[Sequence[int]]] = None):
    """Invert the stack t = T-1 .. 0, each block by Jacobi from zero init.
    Returns (x, iters [T][nb]) with iters indexed by block t."""
    x = np.asarray(z, dtype=np.float64)
    all_iters = [None] * len(ps)
    for t in reversed(range(len(ps))):
        f = None if forced_iters is None else forced_iters[t]
        x, it = inverse_jacobi_block(ps[t], x, n_heads, B, tau, max_iters,
                                     "zero", None, 0, direction_of(t),
                                     forced_iters=f)
        all_iters[t] = it
    return x, np.stack(all_iters)


# --------------------------------------------------------------------------
# deep o shallow composition  [notes, 整体框架; 关键设计 1, frame factorisation]
# --------------------------------------------------------------------------
def _frames(a: np.ndarray, frame_len: int) -> np.ndarray:
    N, L, C = a.shape
    return a.reshape(N * (L // frame_len), frame_len, C)


def forward_deep_shallow(p_deep: Dict, ps_shallow: Sequence[Dict], x: np.ndarray,
                         h_deep: int, h_shallow: int, frame_len: int):
    """z = f_D(f_S(x)) with f_S applied to every frame of F = frame_len tokens
    on its own and f_D to the whole sequence; returns (z, logdet) with
    logdet[n] = log|det dz/dx| = logdet_D(u) + sum over frames of logdet_S."""
    x = np.asarray(x, dtype=np.float64)
    N, L, C = x.shape
    u_f, ld_s = forward_stack(ps_shallow, _frames(x, frame_len), h_shallow)
    z, ld_d = forward_block(p_deep, u_f.reshape(N, L, C), h_deep)
    return z, ld_d + ld_s.reshape(N, L // frame_len).sum(axis=1)


def inverse_deep_shallow(p_deep: Dict, ps_shallow: Sequence[Dict], z: np.ndarray,
                         h_deep: int, h_shallow: int, frame_len: int,
                         tau: float = 1e-3, max_iters: int = 0,
                         deep_forced: Optional[Sequence[int]] = None,
                         shallow_forced: Optional[Sequence] = None):
    """x = f_S^-1(f_D^-1(z)).  f_D^-1 by block-wise Jacobi with one frame per
    block and the previous-frame warm start; then f_S^-1 of every frame on its
    own (its own stop test), each stack block by Jacobi over the frame.
    Returns (x, deep iters [n_frames], shallow iters [N*n_frames][T][1])."""
    z = np.asarray(z, dtype=np.float64)
    N, L, C = z.shape
    u, it_d = inverse_jacobi_block(p_deep, z, h_deep, frame_len, tau, max_iters,
                                   "prev_frame", None, frame_len,
                                   forced_iters=deep_forced)
    u_f = _frames(u, frame_len)
    xs, its = [], []
    for i in range(u_f.shape[0]):
        f = None if shallow_forced is None else shallow_forced[i]
        x_i, it_i = inverse_jacobi_stack(ps_shallow, u_f[i:i + 1], h_shallow, frame_len,
                                         tau, max_iters, forced_iters=f)
        xs.append(x_i)
        its.append(it_i)
    return np.concatenate(xs, axis=0).reshape(N, L, C), it_d, np.stack(its)


# --------------------------------------------------------------------------
# streaming: sliding window over the deep block  [notes, 一个完整示例, 流式生成]
# --------------------------------------------------------------------------
def inverse_streaming(p: Dict, z: np.ndarray, n_heads: int, window: int, overlap: int,
                      B: int, tau: float = 1e-3, max_iters: int = 0, frame_len: int = 0,
                      forced_iters: Optional[Sequence[Sequence[int]]] = None):
    """Generate a sequence longer than the block's positions chunk by chunk.
    The first chunk inverts z[:, :window] at positions 0..window-1.  Each later
    chunk re-encodes the last `overlap` generated tokens into the KV cache at
    positions 0..overlap-1 (a fresh cache) and inverts the next
    window - overlap latents at positions overlap.. conditioned on them.
    Inside a chunk: block-wise Jacobi with blocks of B tokens, zero init, or
    the previous-frame warm start when frame_len > 0 (frames of the chunk).
    Returns (x, per-chunk iteration arrays)."""
    z = np.asarray(z, dtype=np.float64)
    N, L, C = z.shape
    if not 0 <= overlap < window:
        raise ValueError("need 0 <= overlap < window")
    init = "prev_frame" if frame_len > 0 else "zero"
    xs, its = [], []
    done, c = 0, 0
    while done < L:
        f = None if forced_iters is None else forced_iters[c]
        if done == 0:
            n = min(window, L)
            x_c, it = inverse_jacobi_block(p, z[:, :n], n_heads, B, tau, max_iters, init,
                                           None, frame_len, forced_iters=f)
        else:
            n = min(window - overlap, L - done)
            ov = np.concatenate(xs, axis=1)[:, done - overlap:done]
            cache, x_last = prefill(p, ov, n_heads) if overlap > 0 else (None, None)
            x_c, it = inverse_jacobi_block(p, z[:, done:done + n], n_heads, B, tau, max_iters,
                                           init, None, frame_len, pos0=overlap, cache=cache,
                                           x_last=x_last, forced_iters=f)
        xs.append(x_c)
        its.append(it)
        done += n
        c += 1
    return np.concatenate(xs, axis=1), its


# --------------------------------------------------------------------------
# brute-force Jacobian (tiny inputs only)
# --------------------------------------------------------------------------
def jacobian_bruteforce(f, x: np.ndarray, h: float = 1e-6) -> np.ndarray:
    """Central-difference Jacobian of f: R^{n} -> R^{n} at x (any shape);
    returns J[i, j] = d f_i / d x_j over the flattened arrays."""
    x = np.asarray(x, dtype=np.float64)
    n = x.size
    cols = []
    for j in range(n):
        e = np.zeros(n)
        e[j] = h
        fp = f((x.ravel() + e).reshape(x.shape)).ravel()
        fm = f((x.ravel() - e).reshape(x.shape)).ravel()
        cols.append((fp - fm) / (2 * h))
    return np.stack(cols, axis=1)
