"""Parity at the benchmark workloads' full sizes, in the launch configuration
bench.py times, against the oracle element by element.  Where the oracle
cannot run a case whole it runs an exact part of it:

  * the whole 1560-token frame, and the first two frames of the 21-frame
    video (frame 1 with frame 0's K/V as its cache and frame 0 as its warm
    start), with the oracle forced to the GPU's iteration counts;
  * late frames at the video's attention shape (a 31 200-token prefix, and a
    12 480-token prefix where the two-stream row split starts) with a
    one-layer block of the deep block's width, teacher-forced: both sides
    encode the same observed prefix, then invert the next frame.  Causality
    makes the first S tokens of a Jacobi block depend only on the first S
    tokens of every iterate, so the oracle runs on a prefix of the block,
    forced to the GPU's count, and reproduces the GPU's prefix exactly;
  * the wide block (4 layers, d = 4096) after its 3120-token prefix, the same
    way on the first 256 tokens of both samples;
  * frames of the shallow stack run alone (frames are independent).

Every comparison reports the whole-tensor relative L2 and the largest
per-token relative error; the log-det is asserted at full size.

Method: STARFlow-V notes (papernotes.org), 关键设计 1 (affine AF block, log
sigma, alternating directions), 关键设计 3 (block-wise Jacobi: KV cache,
warm start from the previous frame, residual stop), 一个完整示例 (I2V: the
observed frames are forward-encoded into the KV cache)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from autoregressive_normalizing_flow_amd import synth  # noqa: E402
from oracle import af_oracle as O  # noqa: E402
from parity_util import (TOL_BF16, TOL_BF16_TOKEN, TOL_LOGDET, Progress,  # noqa: E402
                         chunked_prefill, layer0_cache, problem, rel_l2, say, to_dev,
                         to_np, token_rel_max)

pytestmark = pytest.mark.gpu
F = 1560       # tokens per latent frame
PREFIX = 256   # tokens of a late-frame block compared element by element


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from autoregressive_normalizing_flow_amd import binding
    binding.load_library()
    return binding


def check(tag, xg, xo):
    e, et = rel_l2(xg, xo), token_rel_max(xg, xo)
    print(f"{tag}: rel_l2 {e:.2e}, max per-token {et:.2e}", flush=True)
    assert e < TOL_BF16, tag
    assert et < TOL_BF16_TOKEN, tag


def test_bf16_long_sequence_multichunk_attention(B):
    """Key ranges long enough to be split into chunks (and merged)."""
    say("bf16 long multichunk")
    cfg = synth.BlockCfg(C=48, d=256, n_heads=4, n_layers=1, max_len=1100, dtype="bf16")
    params = synth.make_params(cfg, 40, randomize_aux=True)
    p64 = O.to64(params[0])
    plan = B.AFPlan(cfg, params)
    x = synth.normal((1, 1100, 48), 42)
    zg, _ = plan.forward(to_dev(x))
    zo, _ = O.forward_block(p64, x, 4)
    check("forward", to_np(zg), zo)
    z = synth.normal((1, 1100, 48), 41)
    xg, itg = plan.inverse_jacobi(to_dev(z), 550, 1e-3)
    xo, _ = O.inverse_jacobi_block(p64, z, 4, 550, 1e-3, forced_iters=list(itg[0]))
    print("iters", itg.tolist())
    check("inverse", to_np(xg), xo)


@pytest.mark.parametrize("H", [4, 2], ids=["dh64", "dh128"])
def test_bf16_long_prefix_many_chunks(B, H):
    """A 2600-token prefix and a 200-token block, one or two samples' worth of
    heads: every query tile's keys span six 512-key chunks, so the merge runs
    over more than one group of slots (in the prefill as well as in the
    Jacobi updates), checked against the oracle."""
    say("bf16 long prefix, many chunks", H)
    P, Fb = 2600, 200
    cfg, params, p64 = problem(C=48, d=256, H=H, layers=2, max_len=P + Fb, dtype="bf16",
                               seed=60 + H)
    plan = B.AFPlan(cfg, params)
    xp = synth.normal((1, P, 48), 61)
    z = synth.normal((1, Fb, 48), 62)
    plan.prefill(to_dev(xp), rows=Fb)
    xg, itg = plan.inverse_jacobi(to_dev(z), Fb, 1e-3, prefix_len=P, x_last=to_dev(xp[:, -1]))
    cache, x_last = O.prefill(p64[0], xp, H)
    x_t, it_t = O.inverse_jacobi_block(p64[0], z, H, Fb, 1e-3, pos0=P, cache=cache,
                                       x_last=x_last)
    xo = x_t
    if not np.array_equal(it_t, itg[0]):
        xo, _ = O.inverse_jacobi_block(p64[0], z, H, Fb, 1e-3, pos0=P, cache=cache,
                                       x_last=x_last, forced_iters=list(itg[0]))
    print("iters gpu", itg.tolist(), "oracle", it_t.tolist())
    check("inverse", to_np(xg), xo)
    # the merge adds the chunks in a fixed order whichever chunk finishes
    # last, so a second run is bit for bit the same
    plan.prefill(to_dev(xp), rows=Fb)
    xg2, itg2 = plan.inverse_jacobi(to_dev(z), Fb, 1e-3, prefix_len=P, x_last=to_dev(xp[:, -1]))
    assert np.array_equal(itg2, itg) and torch.equal(xg2, xg)


def oracle_pair(p64, z, H, B_, k, **kw):
    """The oracle forced to k-1 and to k updates: (x^(k), num, den) with the
    residual sums of update k, sum (x^(k) - x^(k-1))^2 and sum (x^(k))^2."""
    xa, _ = O.inverse_jacobi_block(p64, z, H, B_, 0.0, forced_iters=[k - 1], **kw)
    xb, _ = O.inverse_jacobi_block(p64, z, H, B_, 0.0, forced_iters=[k], **kw)
    return xb, ((xb - xa) ** 2).sum(axis=(1, 2)), (xb ** 2).sum(axis=(1, 2))


def test_row_split_matches_single_pass_and_oracle(B):
    """Row split of the Jacobi update (two streams: a 1024-row block after an
    8192-token prefix, so the split applies).  A forced count of 3 updates:
    x against the oracle and against the single pass, and the residual sums
    the stop test sees (both halves added) against the oracle's sums of
    update 3 and against the single pass's.  The tau stop: x against the
    oracle forced to the GPU's count, whichever count each mode reaches."""
    say("row split")
    P, R = 8192, 1024
    cfg, params, p64 = problem(C=48, d=256, H=4, layers=1, max_len=P + R, dtype="bf16",
                               seed=70)
    plan = B.AFPlan(cfg, params)
    xp = synth.normal((1, P, 48), 71)
    z = synth.normal((1, R, 48), 72)
    cache, x_last = O.prefill(p64[0], xp, 4)
    kw = dict(pos0=P, cache=cache, x_last=x_last)
    xo3, num3, den3 = oracle_pair(p64[0], z, 4, R, 3, **kw)
    out = {}
    for split in (True, False):
        plan.set_row_split(split)
        plan.prefill(to_dev(xp), rows=R)
        plan.profile_enable("affine")
        xf, itf = plan.inverse_jacobi(to_dev(z), R, 0.0, 3, prefix_len=P,
                                      x_last=to_dev(xp[:, -1]))
        n_aff, _ = plan.profile_read()
        plan.profile_disable()
        assert n_aff == (6 if split else 3)   # one affine update per half and update
        assert itf[0][0] == 3
        res = plan.last_residual(1)
        plan.prefill(to_dev(xp), rows=R)
        xt, itt = plan.inverse_jacobi(to_dev(z), R, 1e-3, prefix_len=P,
                                      x_last=to_dev(xp[:, -1]))
        out[split] = (to_np(xf), res, to_np(xt), itt)
        check(f"split={split} forced 3 vs oracle", to_np(xf), xo3)
        e_num = abs(float(res[0, 0]) - num3[0]) / num3[0]
        e_den = abs(float(res[0, 1]) - den3[0]) / den3[0]
        print(f"split={split}: residual sums {res[0].tolist()} oracle "
              f"({num3[0]:.6e}, {den3[0]:.6e}): rel {e_num:.2e}, {e_den:.2e}")
        # the change between bf16 iterates carries more relative error than x
        # itself; a half dropped or counted twice moves num by about 2x
        assert e_num < 0.25 and e_den < 1e-2
        xo_t, _ = O.inverse_jacobi_block(p64[0], z, 4, R, 1e-3, forced_iters=list(itt[0]),
                                         **kw)
        print(f"split={split}: tau iters {itt.tolist()}")
        check(f"split={split} tau vs oracle", to_np(xt), xo_t)
    (fa, ra, ta, ja), (fb, rb, tb, jb) = out[True], out[False]
    assert rel_l2(fa, fb) < 2e-3
    # both halves' sums reach the stop test: equal to the single pass's sums
    # up to summation order (one half dropped or counted twice would move
    # them by tens of percent)
    assert np.all(np.abs(ra - rb) / rb < 1e-2)


def test_row_split_batch_of_two(B):
    """The row split with two samples (each sample's rows halved, residual
    pairs per sample and half): against the single pass and the oracle, forced
    count and tau stop, the two samples' counts shared."""
    say("row split, batch 2")
    P, R, N = 8192, 1024, 2
    cfg, params, p64 = problem(C=48, d=256, H=4, layers=1, max_len=P + R, dtype="bf16",
                               seed=73)
    plan = B.AFPlan(cfg, params)
    xp_np = synth.normal((N, P, 48), 74)
    z_np = synth.normal((N, R, 48), 75)
    xp, z = to_dev(xp_np), to_dev(z_np)
    cache, x_last = O.prefill(p64[0], xp_np, 4)
    kw = dict(pos0=P, cache=cache, x_last=x_last)
    out = {}
    for split in (True, False):
        plan.set_row_split(split)
        plan.prefill(xp, rows=R)
        plan.profile_enable("affine")
        xf, itf = plan.inverse_jacobi(z, R, 0.0, 2, prefix_len=P, x_last=xp[:, -1].contiguous())
        n_aff, _ = plan.profile_read()
        plan.profile_disable()
        assert n_aff == (4 if split else 2) and itf[0][0] == 2
        res = plan.last_residual(N)
        plan.prefill(xp, rows=R)
        xt, itt = plan.inverse_jacobi(z, R, 1e-3, prefix_len=P, x_last=xp[:, -1].contiguous())
        out[split] = (to_np(xf), res, to_np(xt), itt)
    (fa, ra, ta, ja), (fb, rb, tb, jb) = out[True], out[False]
    xo2, num2, den2 = oracle_pair(p64[0], z_np, 4, R, 2, **kw)
    check("forced 2, split vs oracle", fa, xo2)
    assert rel_l2(fa, fb) < 2e-3
    assert np.all(np.abs(ra[:, 0] - num2) / num2 < 0.25)
    assert np.all(np.abs(ra[:, 1] - den2) / den2 < 1e-2)
    assert np.all(np.abs(ra - rb) / rb < 1e-2)
    xo_t, _ = O.inverse_jacobi_block(p64[0], z_np, 4, R, 1e-3, forced_iters=list(ja[0]), **kw)
    print(f"tau iters split {ja.tolist()} single pass {jb.tolist()}")
    check("tau, split vs oracle", ta, xo_t)


def test_frame480p_fullsize(B):
    """One 1560-token frame, 8 layers d=1024, B=1560, zero init, tau=1e-3:
    the whole frame against the oracle forced to the GPU's count, and the
    forward (z and log-det) of a random x."""
    w = synth.WORKLOADS["frame480p"]
    say("frame480p full size")
    params = synth.make_params(w.block, 0)
    p64 = O.to64(params[0])
    plan = B.AFPlan(w.block, params)
    x = synth.normal((1, F, 48), 2)
    zgf, ldg = plan.forward(to_dev(x))
    zof, ldo = O.forward_block(p64, x, 16)
    check("forward z", to_np(zgf), zof)
    e_ld = abs(float(to_np(ldg)[0]) - ldo[0]) / abs(ldo[0])
    print(f"log-det gpu {float(to_np(ldg)[0]):.6f} oracle {ldo[0]:.6f} rel {e_ld:.2e}")
    assert e_ld < TOL_LOGDET
    z = synth.normal((1, F, 48), 1)
    xg, itg = plan.inverse_jacobi(to_dev(z), F, 1e-3)
    print("iters", itg.tolist(), flush=True)
    xo, _ = O.inverse_jacobi_block(p64, z, 16, F, 1e-3, forced_iters=[int(itg[0, 0])],
                                   trace=Progress("frame480p"))
    check("inverse, whole frame", to_np(xg), xo)


def test_video21_first_frames_fullsize(B):
    """21 frames x 1560 tokens, block = frame, previous-frame warm start, as
    the benchmark runs it: frames 0 and 1 (frame 1 warm-started from frame 0
    and attending to frame 0's refreshed K/V) against the oracle forced to
    the GPU's counts, every token."""
    w = synth.WORKLOADS["video21"]
    say("video21 full size")
    params = synth.make_params(w.block, 0)
    p64 = O.to64(params[0])
    plan = B.AFPlan(w.block, params)
    z = synth.normal((1, 21 * F, 48), 1)
    xg, itg = plan.inverse_jacobi(to_dev(z), F, 1e-3, init="prev_frame", frame_len=F)
    xg_np = to_np(xg)
    print("iters per frame", itg.tolist(), flush=True)
    assert itg.shape == (1, 21) and np.all(itg >= 1) and np.all(itg <= F)
    assert np.isfinite(xg_np).all()
    xo, _ = O.inverse_jacobi_block(p64, z[:, :2 * F], 16, F, 1e-3, init="prev_frame",
                                   frame_len=F, forced_iters=[int(k) for k in itg[0, :2]],
                                   trace=Progress("video21"))
    check("frame 0", xg_np[:, :F], xo[:, :F])
    check("frame 1", xg_np[:, F:2 * F], xo[:, F:])


def late_frame(B, P, split, seed):
    """One layer of the deep block's width (d=1024, 16 heads), teacher-forced
    after a P-token observed prefix: af_prefill on both sides, then one
    1560-token Jacobi block from the last prefix frame (warm start, tau=1e-3)
    on the GPU; the oracle reruns its first PREFIX tokens forced to the GPU's
    count."""
    cfg, params, (p64,) = problem(C=48, d=1024, H=16, layers=1, max_len=P + F,
                                  dtype="bf16", seed=seed, aux=False)
    plan = B.AFPlan(cfg, params)
    plan.set_row_split(split)
    xp = synth.normal((1, P, 48), seed + 1)
    z = synth.normal((1, F, 48), seed + 2)
    x_init = np.ascontiguousarray(xp[:, P - F:])
    plan.prefill(to_dev(xp), rows=F)
    plan.profile_enable("affine")
    xg, itg = plan.inverse_jacobi(to_dev(z), F, 1e-3, init="given", x_init=to_dev(x_init),
                                  prefix_len=P, x_last=to_dev(xp[:, -1]))
    n_aff, _ = plan.profile_read()
    plan.profile_disable()
    k = int(itg[0, 0])
    print(f"prefix {P} split={split}: iters {k}, affine launches {n_aff}", flush=True)
    return plan, xp, z, x_init, to_np(xg), k, n_aff, p64


@pytest.mark.parametrize("split", [True, False], ids=["row_split", "one_pass"])
def test_video_last_frame_attention_shape(B, split):
    """The 21st frame's attention shape: 1560 queries over a 31 200-token
    prefix plus their own keys.  In one pass the key range of every query
    tile is cut into 8192-key chunks; with the row split each half's into
    4096-key chunks.  First 256 tokens against the oracle."""
    say("video last frame, split", split)
    P = 20 * F
    plan, xp, z, x_init, xg, k, n_aff, p64 = late_frame(B, P, split, 80)
    assert n_aff == (2 * k if split else k)
    cache = layer0_cache(p64, xp, 16)
    xo, _ = O.inverse_jacobi_block(p64, z[:, :PREFIX], 16, PREFIX, 0.0, init="given",
                                   x_init=x_init[:, :PREFIX], pos0=P, cache=cache,
                                   x_last=xp[:, -1], forced_iters=[k],
                                   trace=Progress("last frame"))
    check(f"last frame, first {PREFIX} tokens", xg[:, :PREFIX], xo)


def test_video_frame_at_split_threshold(B):
    """A frame after 8 frames of prefix (12 480 tokens: the first shape the
    row split takes), the whole 1560-token block against the oracle forced to
    the GPU's count, so both halves' rows are compared."""
    say("video frame 8, whole block")
    P = 8 * F
    plan, xp, z, x_init, xg, k, n_aff, p64 = late_frame(B, P, True, 90)
    assert n_aff == 2 * k
    cache = layer0_cache(p64, xp, 16)
    xo, _ = O.inverse_jacobi_block(p64, z, 16, F, 0.0, init="given", x_init=x_init, pos0=P,
                                   cache=cache, x_last=xp[:, -1], forced_iters=[k],
                                   trace=Progress("frame 8"))
    check("frame 8, first half", xg[:, :F // 2], xo[:, :F // 2])
    check("frame 8, second half", xg[:, F // 2:], xo[:, F // 2:])


def test_shallow_stack_fullsize(B):
    """T=4 alternating blocks, 2 layers d=512, 21 frames batched: z, log-det
    and the Jacobi inverse of sampled frames, run alone by the oracle."""
    w = synth.WORKLOADS["shallow_stack"]
    say("shallow_stack full size")
    params = synth.make_params(w.block, 0, n_blocks=4)
    ps64 = [O.to64(p) for p in params]
    plan = B.AFPlan(w.block, params)
    x = synth.noisy_latents((21, F, 48), 2, 0.3)
    zg, ldg = plan.forward(to_dev(x))
    xg, itg = plan.inverse_jacobi(zg, F, 1e-3)
    print("iters per stack block", itg.tolist())
    zg_np, xg_np, ldg_np = to_np(zg), to_np(xg), to_np(ldg)
    for n in (0, 20):   # sampled frames, run alone by the oracle
        zo, ldo = O.forward_stack(ps64, x[n:n + 1], 8)
        check(f"frame {n} z", zg_np[n:n + 1], zo)
        e_ld = abs(ldg_np[n] - ldo[0]) / abs(ldo[0])
        print(f"frame {n}: log-det gpu {ldg_np[n]:.6f} oracle {ldo[0]:.6f} rel {e_ld:.2e}")
        assert e_ld < TOL_LOGDET
        xo, _ = O.inverse_jacobi_stack(ps64, zg_np[n:n + 1], 8, F, 1e-3, forced_iters=itg)
        check(f"frame {n} x", xg_np[n:n + 1], xo)


def test_wide_prefix_fullsize(B):
    """4 layers d=4096 (dh=128), batch 2: the 2-frame prefix encoded on both
    sides, then one frame by Jacobi from the last prefix frame; the first 256
    tokens of both samples against the oracle forced to the GPU's count."""
    w = synth.WORKLOADS["wide_prefix"]
    say("wide_prefix full size")
    params = synth.make_params(w.block, 0)
    p64 = O.to64(params[0])
    plan = B.AFPlan(w.block, params)
    xp = synth.normal((2, 2 * F, 48), 2)
    z = synth.normal((2, F, 48), 1)
    x_init = np.ascontiguousarray(xp[:, F:])
    plan.prefill(to_dev(xp), rows=F)
    xg, itg = plan.inverse_jacobi(to_dev(z), F, 1e-3, init="given", x_init=to_dev(x_init),
                                  prefix_len=2 * F, x_last=to_dev(xp[:, -1]))
    k = int(itg[0, 0])
    print("iters", itg.tolist(), flush=True)
    cache, x_last = chunked_prefill(p64, xp, 32)
    xo, _ = O.inverse_jacobi_block(p64, z[:, :PREFIX], 32, PREFIX, 0.0, init="given",
                                   x_init=x_init[:, :PREFIX], pos0=2 * F, cache=cache,
                                   x_last=x_last, forced_iters=[k], trace=Progress("wide"))
    check(f"wide prefix, first {PREFIX} tokens", to_np(xg)[:, :PREFIX], xo)


def test_wide_width_prefix_vs_oracle(B):
    """Full width d=4096, dh=128, one layer, short frames: prefix + GIVEN init
    against the oracle element by element."""
    say("wide width prefix vs oracle")
    Fs = 96
    cfg = synth.BlockCfg(C=48, d=4096, n_heads=32, n_layers=1, max_len=3 * Fs, dtype="bf16")
    params = synth.make_params(cfg, 0)
    p64 = O.to64(params[0])
    plan = B.AFPlan(cfg, params)
    xp = synth.normal((2, 2 * Fs, 48), 2)
    z = synth.normal((2, Fs, 48), 1)
    plan.prefill(to_dev(xp), rows=Fs)
    x_init = np.ascontiguousarray(xp[:, Fs:])
    xg, itg = plan.inverse_jacobi(to_dev(z), Fs, 1e-3, init="given", x_init=to_dev(x_init),
                                  prefix_len=2 * Fs, x_last=to_dev(xp[:, -1]))
    cache, x_last = O.prefill(p64, xp, 32)
    xo, _ = O.inverse_jacobi_block(p64, z, 32, Fs, 1e-3, init="given", x_init=x_init,
                                   pos0=2 * Fs, cache=cache, x_last=x_last,
                                   forced_iters=list(itg[0]))
    print("iters", itg.tolist())
    check("wide width", to_np(xg), xo)
