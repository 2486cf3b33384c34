"""Shared helpers of the GPU parity tests: seeded problems, oracle runs and
error metrics.  The oracle and the HIP path receive the same seeded arrays
(from autoregressive_normalizing_flow_amd.synth) and share nothing else."""
import sys

import numpy as np

from autoregressive_normalizing_flow_amd import synth
from oracle import af_oracle as O

# tolerances: relative L2 on the fp32 path / on the bf16 path, log-det
# relative error (both paths)
TOL_F32 = 1e-4
TOL_BF16 = 2e-2
TOL_LOGDET = 1e-3
# Per-token bound beside the whole-tensor one: no single token's relative
# error (its error norm over the C channels against its own norm) may exceed
# five times the tensor bar.  The tensor bar bounds the root-mean-square of
# the tokens' errors; tokens see rounding errors of the same kind, so their
# largest relative error exceeds the mean by a small factor, while one wrong
# token (an error of its own size) fails at once.
TOL_BF16_TOKEN = 5 * TOL_BF16


def say(*a):
    """Name the case on stdout before a GPU step (flushed)."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def token_rel_max(a, b) -> float:
    """Largest per-token relative error: max over (sample, token) of
    ||a_t - b_t|| / ||b_t|| over the channel axis (token tensors [N, L, C])."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    num = np.linalg.norm(a - b, axis=-1)
    den = np.maximum(np.linalg.norm(b, axis=-1), 1e-300)
    return float((num / den).max())


class Progress(list):
    """A trace list for the oracle's Jacobi loop that prints each update as
    it is appended (long oracle runs stay visibly alive)."""

    def __init__(self, tag):
        super().__init__()
        self.tag = tag

    def append(self, item):
        b, k, r = item
        print(f"  [oracle {self.tag}] block {b} update {k} r {np.max(r):.3e}", flush=True)
        super().append(item)


def layer0_cache(p64, x, H, chunk=1560):
    """K/V of positions 0..P-1 for a ONE-layer block: layer 0's K and V of a
    row depend only on that row's shifted token and position (they are
    computed before its attention), so the oracle's network run on row chunks
    without a cache gives exactly those rows' cache entries."""
    assert len(p64["layers"]) == 1
    sh = O.shift(np.asarray(x, np.float64))
    P = sh.shape[1]
    ks, vs = [], []
    for c0 in range(0, P, chunk):
        c1 = min(P, c0 + chunk)
        _, _, kv = O.net_rows(p64, sh[:, c0:c1], np.arange(c0, c1), H, None)
        ks.append(kv[0][0])
        vs.append(kv[0][1])
    return [(np.concatenate(ks, axis=2), np.concatenate(vs, axis=2))]


def chunked_prefill(p64, x, H, chunk=520):
    """The oracle's prefill over row chunks, each attending to the cache of
    the chunks before it (equal to one pass over all rows: the cache
    equivalence the oracle's pins check), so that no chunk's score matrix
    spans the whole prefix."""
    x = np.asarray(x, np.float64)
    N, P, C = x.shape
    d = p64["w_in"].shape[0]
    sh = O.shift(x)
    e = np.zeros((N, H, 0, d // H))
    cache = [(e.copy(), e.copy()) for _ in p64["layers"]]
    for c0 in range(0, P, chunk):
        c1 = min(P, c0 + chunk)
        _, _, kv = O.net_rows(p64, sh[:, c0:c1], np.arange(c0, c1), H, cache)
        cache = [(np.concatenate([kc, k], axis=2), np.concatenate([vc, v], axis=2))
                 for (kc, vc), (k, v) in zip(cache, kv)]
    return cache, x[:, -1].copy()


def rel_err(a, b) -> np.ndarray:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.abs(a - b) / np.maximum(np.abs(b), 1e-300)


def problem(C, d, H, layers, max_len, dtype, seed=0, aux=True, n_blocks=1):
    cfg = synth.BlockCfg(C=C, d=d, n_heads=H, n_layers=layers, max_len=max_len,
                         dtype=dtype)
    params = synth.make_params(cfg, seed, randomize_aux=aux, n_blocks=n_blocks)
    return cfg, params, [O.to64(p) for p in params]


def to_dev(a, device="cuda:0"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def to_np(t):
    return t.detach().cpu().numpy().astype(np.float64)


def oracle_jacobi_like(p64, z, H, B, tau, gpu_iters, **kw):
    """The oracle's Jacobi with the same tau, and — when its iteration counts
    differ from the GPU's — the oracle run forced to the GPU's counts, which
    is the result to compare element by element.  Returns
    (x_compare, oracle_iters_tau)."""
    x_t, it_t = O.inverse_jacobi_block(p64, z, H, B, tau, **kw)
    if np.array_equal(it_t, gpu_iters):
        return x_t, it_t
    x_f, _ = O.inverse_jacobi_block(p64, z, H, B, tau, forced_iters=list(gpu_iters), **kw)
    return x_f, it_t
