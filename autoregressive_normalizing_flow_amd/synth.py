"""Seeded synthetic inputs and parameters for the affine autoregressive-flow block.

This module holds no arithmetic of the method itself: it only draws random
numbers, rounds stored weights to their storage format, and names the
workload shapes.  Both the CPU oracle and the HIP path receive the arrays it
produces, so the two sides always see bit-identical weights and inputs.

Workload shapes follow the STARFlow-V notes (papernotes.org, "STARFlow-V:
End-to-End Video Generative Modeling with Autoregressive Normalizing Flows"),
section 整体框架: latents of a 3D causal VAE with 16x spatial / 4x temporal
compression and 48 channels.  A 480x832 frame is 30x52 = 1560 latent tokens,
and an 81-frame clip is 1 + 80/4 = 21 latent frames (an inference: the notes
give the factors, not the counts).

Random-number recipe (numpy PCG64 via ``default_rng``):
  * parameters from seed s, drawn in parameter-list order (see PARAM_ORDER),
    one standard-normal array per parameter whether or not it is used,
  * z from seed s+1, x / noise / prefix from seed s+2.
Weight matrices, the position table and the head get N(0, 0.02^2); biases are
0 and LayerNorm gains 1 unless ``randomize_aux`` (then N(0, 0.02^2) biases and
1 + N(0, 0.02^2) gains, so those code paths are exercised).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

INIT_STD = 0.02

# Matrices that the bf16 path stores in bf16 (the dense contractions).  All
# other parameters (input projection, position table, head, biases, norms)
# are stored in fp32 on every path.
BF16_MATRICES = ("w_qkv", "w_o", "w_1", "w_2")

LAYER_PARAMS = ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o",
                "ln2_g", "ln2_b", "w_1", "b_1", "w_2", "b_2")
TOP_PARAMS_PRE = ("w_in", "b_in", "pos")
TOP_PARAMS_POST = ("ln_f_g", "ln_f_b", "w_head", "b_head")


@dataclasses.dataclass(frozen=True)
class BlockCfg:
    """Shape of one affine AF block: a causal Transformer that maps the
    shifted tokens to (mu, raw) per token."""
    C: int            # latent channels per token
    d: int            # model width
    n_heads: int
    n_layers: int
    max_len: int      # position-table length (positions 0..max_len-1)
    dtype: str = "bf16"   # "bf16" or "f32": storage/operand type of BF16_MATRICES

    @property
    def d_mlp(self) -> int:
        return 4 * self.d

    @property
    def d_head(self) -> int:
        return self.d // self.n_heads


def param_shapes(cfg: BlockCfg) -> Dict[str, tuple]:
    d, C, F = cfg.d, cfg.C, cfg.d_mlp
    shapes = {"w_in": (d, C), "b_in": (d,), "pos": (cfg.max_len, d)}
    for name, shp in (("ln1_g", (d,)), ("ln1_b", (d,)), ("w_qkv", (3 * d, d)),
                      ("b_qkv", (3 * d,)), ("w_o", (d, d)), ("b_o", (d,)),
                      ("ln2_g", (d,)), ("ln2_b", (d,)), ("w_1", (F, d)),
                      ("b_1", (F,)), ("w_2", (d, F)), ("b_2", (d,))):
        shapes[name] = shp
    shapes.update({"ln_f_g": (d,), "ln_f_b": (d,), "w_head": (2 * C, d),
                   "b_head": (2 * C,)})
    return shapes


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returned as fp32
    arrays that hold exactly the bf16 values.  Storage-format conversion only."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = (r & 0xFFFFFFFF).astype(np.uint32).view(np.float32)
    return out.reshape(a.shape)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """The uint16 bit patterns of fp32 arrays that already hold bf16 values."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> 16).astype(np.uint16)


def _draw(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape)  # fp64 draws, cast by the caller


def _block_params(cfg: BlockCfg, rng: np.random.Generator,
                  randomize_aux: bool) -> Dict:
    shapes = param_shapes(cfg)
    p: Dict = {"layers": []}

    def make(name):
        g = _draw(rng, shapes[name])
        if name.startswith("w_") or name == "pos":
            v = INIT_STD * g
        elif name.endswith("_g"):
            v = 1.0 + INIT_STD * g if randomize_aux else np.ones(shapes[name])
        else:  # biases and LayerNorm shifts
            v = INIT_STD * g if randomize_aux else np.zeros(shapes[name])
        v = v.astype(np.float32)
        if cfg.dtype == "bf16" and name in BF16_MATRICES:
            v = bf16_round(v)
        return v

    for name in TOP_PARAMS_PRE:
        p[name] = make(name)
    for _ in range(cfg.n_layers):
        p["layers"].append({name: make(name) for name in LAYER_PARAMS})
    for name in TOP_PARAMS_POST:
        p[name] = make(name)
    return p


def make_params(cfg: BlockCfg, seed: int = 0, randomize_aux: bool = False,
                n_blocks: int = 1) -> List[Dict]:
    """Parameters of ``n_blocks`` AF blocks (a stack), drawn in block order
    from one generator.  Every value is fp32 (bf16-exact for BF16_MATRICES on
    the bf16 path)."""
    rng = np.random.default_rng(seed)
    return [_block_params(cfg, rng, randomize_aux) for _ in range(n_blocks)]


def normal(shape, seed: int, scale: float = 1.0) -> np.ndarray:
    """fp32 N(0, scale^2) array from ``default_rng(seed)``."""
    rng = np.random.default_rng(seed)
    return (scale * rng.standard_normal(shape)).astype(np.float32)


def noisy_latents(shape, seed: int, noise_std: float) -> np.ndarray:
    """x = eps1 + noise_std * eps2 with eps ~ N(0, 1), both drawn from one
    generator (first eps1, then eps2).  Stands in for noise-augmented VAE
    latents (STARFlow-V notes, 关键设计 2: training data carries additive
    Gaussian noise)."""
    rng = np.random.default_rng(seed)
    e1 = rng.standard_normal(shape)
    e2 = rng.standard_normal(shape)
    return (e1 + noise_std * e2).astype(np.float32)


# ---------------------------------------------------------------------------
# Named workloads.  Frame = 30x52 latent tokens of a 480x832 clip, C = 48.
# ---------------------------------------------------------------------------
FRAME_TOKENS = 30 * 52
LATENT_C = 48


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    block: BlockCfg
    n_blocks: int          # AF blocks in the stack (alternating L->R / R->L)
    batch: int
    length: int            # tokens inverted per sample
    jacobi_block: int      # B
    tau: float
    init: str              # "zero" | "prev_frame" | "given"
    frame_len: int = 0     # F for "prev_frame"
    prefix: int = 0        # positions pre-filled from observed tokens
    x_noise: Optional[float] = None   # forward input = eps1 + x_noise*eps2
    description: str = ""


WORKLOADS = {
    "tiny_f32": Workload(
        "tiny_f32", BlockCfg(C=16, d=64, n_heads=2, n_layers=1, max_len=64,
                             dtype="f32"),
        n_blocks=1, batch=1, length=64, jacobi_block=16, tau=1e-3, init="zero",
        description="one 8x8 latent frame, C=16, 1 layer d=64, fp32"),
    "frame480p": Workload(
        "frame480p", BlockCfg(C=LATENT_C, d=1024, n_heads=16, n_layers=8,
                              max_len=FRAME_TOKENS),
        n_blocks=1, batch=1, length=FRAME_TOKENS, jacobi_block=FRAME_TOKENS,
        tau=1e-3, init="zero",
        description="one 480p latent frame (1560 tokens), 8-layer d=1024 deep block"),
    "video21": Workload(
        "video21", BlockCfg(C=LATENT_C, d=1024, n_heads=16, n_layers=8,
                            max_len=21 * FRAME_TOKENS),
        n_blocks=1, batch=1, length=21 * FRAME_TOKENS, jacobi_block=FRAME_TOKENS,
        tau=1e-3, init="prev_frame", frame_len=FRAME_TOKENS,
        description="21 latent frames (32760 tokens), block = frame, warm start"),
    "shallow_stack": Workload(
        "shallow_stack", BlockCfg(C=LATENT_C, d=512, n_heads=8, n_layers=2,
                                  max_len=FRAME_TOKENS),
        n_blocks=4, batch=21, length=FRAME_TOKENS, jacobi_block=FRAME_TOKENS,
        tau=1e-3, init="zero", x_noise=0.3,
        description="T=4 alternating blocks, 2 layers d=512, 21 frames batched"),
    "wide_prefix": Workload(
        "wide_prefix", BlockCfg(C=LATENT_C, d=4096, n_heads=32, n_layers=4,
                                max_len=3 * FRAME_TOKENS),
        n_blocks=1, batch=2, length=FRAME_TOKENS, jacobi_block=FRAME_TOKENS,
        tau=1e-3, init="given", prefix=2 * FRAME_TOKENS,
        description="4 layers d=4096, 2-frame prefix then one frame, batch 2"),
}
