"""CPU checks of the GPU tests' oracle helpers: the layer-0 cache of a
one-layer block built row chunk by row chunk, and the chunked prefill, equal
the oracle's own one-pass prefill (STARFlow-V notes, 一个完整示例: observed
frames forward-encoded into the KV cache)."""
import numpy as np

from autoregressive_normalizing_flow_amd import synth
from oracle import af_oracle as O
from parity_util import chunked_prefill, layer0_cache, token_rel_max


def _block(layers, seed):
    cfg = synth.BlockCfg(C=3, d=16, n_heads=2, n_layers=layers, max_len=40, dtype="f32")
    return O.to64(synth.make_params(cfg, seed, randomize_aux=True)[0])


def test_layer0_cache_equals_prefill():
    p = _block(1, 3)
    x = np.random.default_rng(1).standard_normal((2, 37, 3))
    ref, _ = O.prefill(p, x, 2)
    got = layer0_cache(p, x, 2, chunk=8)
    np.testing.assert_allclose(got[0][0], ref[0][0], rtol=0, atol=1e-13)
    np.testing.assert_allclose(got[0][1], ref[0][1], rtol=0, atol=1e-13)


def test_chunked_prefill_equals_prefill():
    p = _block(3, 4)
    x = np.random.default_rng(2).standard_normal((2, 37, 3))
    ref, last = O.prefill(p, x, 2)
    got, last2 = chunked_prefill(p, x, 2, chunk=10)
    for (k, v), (kr, vr) in zip(got, ref):
        np.testing.assert_allclose(k, kr, rtol=0, atol=1e-12)
        np.testing.assert_allclose(v, vr, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(last, last2)


def test_token_rel_max_sees_one_bad_token():
    b = np.ones((1, 100, 4))
    a = b.copy()
    a[0, 57] = -1.0
    assert token_rel_max(a, b) == 2.0
    assert token_rel_max(b, b) == 0.0
