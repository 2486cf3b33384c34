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


def say(*a):
    """Name the case on stdout before a GPU step (flushed)."""
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


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
