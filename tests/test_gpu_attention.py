"""GPU parity of one layer's bf16 attention over a KV cache (afk_attention,
the kernel the Jacobi path runs) against the oracle's exact causal softmax
attention, at shapes that take each kernel the library routes to: the DMA
kernel at d_h 64 (past 256 query tiles with a short prefix, with several key
chunks merged in the kernel) and at d_h 128 (one chunk, and several merged),
its two-key-group form at d_h 64 (at most 256 query tiles over at most 100
key tiles: with and without a cached prefix, one key tile per unit so that
the second group has none, the first frames of the 1560-token video), the
16 x 16 kernel (no prefix, under 64 sample-head pairs, past 256 query tiles)
and the d_h 32 kernel; ragged query and key tails everywhere.  Cache rows past the last query's position hold NaN: the
kernels must not let them into the result.

"Extreme" inputs put the first 64 keys some 300 (log2 units) above the query
and every later key 300 below: the softmax reference must move up on the
first tile and must not move down by 600 on the next (2^600 overflows).

Method: STARFlow-V notes (papernotes.org), 关键设计 3 (causal attention of
the block's queries over the KV cache).  Bars: relative L2 <= 2e-2 (bf16),
and no token worse than 5 x that."""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from autoregressive_normalizing_flow_amd import synth  # noqa: E402
from oracle import af_oracle as O  # noqa: E402
from parity_util import TOL_BF16, TOL_BF16_TOKEN, rel_l2, say, token_rel_max  # noqa: E402

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from autoregressive_normalizing_flow_amd import binding
    binding.load_library()
    return binding


def inputs(N, H, dh, R, P, extreme, seed):
    """q as stored (times log2(e)/sqrt(dh)), keys and values by position, all
    bf16-exact; cache rows past P + R are NaN."""
    rng = np.random.default_rng(seed)
    S = P + R
    Lcap = (S + 63) // 64 * 64 + 64
    qs = synth.bf16_round(rng.standard_normal((N, R, H, dh)).astype(np.float32))
    k = synth.bf16_round(rng.standard_normal((N, H, S, dh)).astype(np.float32))
    v = synth.bf16_round(rng.standard_normal((N, H, S, dh)).astype(np.float32))
    if extreme:
        # dimension 0 carries +-2^5 * 2^4: score 2^9 +- the rest, keys 0..63 up,
        # the rest down (powers of two: exact in bf16)
        qs[..., 0] = 32.0
        k[..., :64, 0] = 16.0
        k[..., 64:, 0] = -16.0
    kc = np.full((N, H, Lcap, dh), np.nan, np.float32)
    kc[:, :, :S] = k
    vt = np.full((N, H, dh, Lcap), np.nan, np.float32)
    vt[:, :, :, :S] = np.swapaxes(v, -1, -2)
    return qs, k, v, kc, vt, Lcap


def oracle_out(qs, k, v, P):
    N, R, H, dh = qs.shape
    # the stored q is Q * log2(e) / sqrt(dh): the oracle's Q is that divided
    q = qs.astype(np.float64).transpose(0, 2, 1, 3) / (LOG2E / math.sqrt(dh))
    o = O.attention(q, k.astype(np.float64), v.astype(np.float64),
                    P + np.arange(R), np.arange(k.shape[2]))
    return o.transpose(0, 2, 1, 3).reshape(N, R, H * dh)


def bf16_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda().to(torch.bfloat16)


@pytest.mark.parametrize("N,H,dh,R,P", [
    (1, 16, 64, 300, 2000),    # prefix, ragged tails: two key groups
    (8, 8, 64, 200, 0),        # no prefix, 64 sample-head pairs: two key groups
    (1, 4, 64, 200, 0),        # no prefix, few heads: two key groups
    (3, 5, 64, 64, 0),         # one key tile per unit: the second group idle
    (1, 16, 64, 130, 14000),   # long prefix: DMA kernel, several key chunks per query tile
    (2, 16, 64, 1100, 2000),   # 288 query tiles, short prefix: DMA kernel
    (1, 32, 64, 1200, 0),      # no prefix, 32 pairs, 320 query tiles: 16 x 16 kernel
    (1, 8, 32, 200, 700),      # d_h 32
    (2, 4, 128, 150, 600),     # d_h 128
    (1, 4, 128, 200, 8000),    # d_h 128, key chunks merged in the kernel
])
@pytest.mark.parametrize("extreme", [False, True])
def test_attention_layer(B, N, H, dh, R, P, extreme):
    say("attention", N, H, dh, R, P, "extreme" if extreme else "normal")
    qs, k, v, kc, vt, Lcap = inputs(N, H, dh, R, P, extreme, seed=R + P + dh)
    out = B.afk_attention(bf16_dev(qs.reshape(N, R, H * dh)), bf16_dev(kc), bf16_dev(vt), P)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all()
    ref = oracle_out(qs, k, v, P)
    e = rel_l2(got, ref)
    t = token_rel_max(got, ref)
    say("   rel_l2", e, "worst token", t)
    assert e < TOL_BF16 and t < TOL_BF16_TOKEN


def oracle_rows(qs, k, v, P, rows):
    """The oracle's output at the given query rows only (positions P + row)."""
    N, R, H, dh = qs.shape
    q = qs[:, rows].astype(np.float64).transpose(0, 2, 1, 3) / (LOG2E / math.sqrt(dh))
    o = O.attention(q, k.astype(np.float64), v.astype(np.float64),
                    P + np.asarray(rows), np.arange(k.shape[2]))
    return o.transpose(0, 2, 1, 3).reshape(N, len(rows), H * dh)


@pytest.mark.parametrize("R,P", [(1560, 0), (1560, 4680), (1560, 12480), (1000, 31000)])
@pytest.mark.parametrize("extreme", [False, True])
def test_attention_long_prefix_sampled(B, R, P, extreme):
    """Frames of the 21-frame video at 16 heads of 64: the first and the 4th
    (two key groups over whole key ranges, the 4th at their 98-tile limit),
    the 9th and 1000 queries after 31 000 keys (a ragged last query tile;
    several key chunks per query tile, dispatched chunk-major and merged in
    key order).  Sampled query rows (both ends of every 128-row query tile and
    every 11th row) against the oracle."""
    N, H, dh = 1, 16, 64
    say("attention long prefix", R, P, "extreme" if extreme else "normal")
    qs, k, v, kc, vt, Lcap = inputs(N, H, dh, R, P, extreme, seed=R + P + 7)
    out = B.afk_attention(bf16_dev(qs.reshape(N, R, H * dh)), bf16_dev(kc), bf16_dev(vt), P)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all()
    rows = sorted(set(range(0, R, 11)) | {min(R - 1, t) for q in range(0, R, 128)
                                          for t in (q, q + 127)})
    ref = oracle_rows(qs, k, v, P, rows)
    e = rel_l2(got[:, rows], ref)
    t = token_rel_max(got[:, rows], ref)
    say("   rows", len(rows), "rel_l2", e, "worst token", t)
    assert e < TOL_BF16 and t < TOL_BF16_TOKEN
