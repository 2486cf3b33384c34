"""Parity at the benchmark workloads' full sizes, in the launch configuration
bench.py times.  The oracle cannot run every full-size case whole, so each
test compares outputs it can compute exactly:

  * causality: the first S tokens of a Jacobi block depend only on the first
    S tokens of every iterate, so the oracle run on a prefix of the block,
    forced to the GPU's iteration count, reproduces the GPU's prefix exactly;
  * frames are independent in the shallow stack, so sampled frames are run
    alone;
  * the fixed-point defect ||forward(x) - z|| / ||z|| of the GPU's x, with the
    oracle's forward on a prefix of frames and the GPU's own forward on all.

Method: STARFlow-V notes (papernotes.org), 关键设计 1 and 3, 一个完整示例."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from autoregressive_normalizing_flow_amd import synth  # noqa: E402
from oracle import af_oracle as O  # noqa: E402
from parity_util import TOL_BF16, problem, rel_l2, say, to_dev, to_np  # noqa: E402

pytestmark = pytest.mark.gpu
PREFIX = 256   # tokens of a block compared element by element


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from autoregressive_normalizing_flow_amd import binding
    binding.load_library()
    return binding


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
    assert rel_l2(to_np(zg), zo) < TOL_BF16
    z = synth.normal((1, 1100, 48), 41)
    xg, itg = plan.inverse_jacobi(to_dev(z), 550, 1e-3)
    xo, _ = O.inverse_jacobi_block(p64, z, 4, 550, 1e-3, forced_iters=list(itg[0]))
    print("iters", itg.tolist(), "x rel_l2", rel_l2(to_np(xg), xo))
    assert rel_l2(to_np(xg), xo) < TOL_BF16


@pytest.mark.parametrize("H", [4, 2], ids=["dh64", "dh128"])
def test_bf16_long_prefix_many_chunks(B, H):
    """A 2600-token prefix and a 200-token block, one or two samples' worth of
    heads: every query tile's keys span six 512-key chunks, so the merge runs
    over more than one group of slots (in the prefill as well as in the
    Jacobi updates), checked against the oracle."""
    say("bf16 long prefix, many chunks", H)
    P, F = 2600, 200
    cfg, params, p64 = problem(C=48, d=256, H=H, layers=2, max_len=P + F, dtype="bf16",
                               seed=60 + H)
    plan = B.AFPlan(cfg, params)
    xp = synth.normal((1, P, 48), 61)
    z = synth.normal((1, F, 48), 62)
    plan.prefill(to_dev(xp), rows=F)
    xg, itg = plan.inverse_jacobi(to_dev(z), F, 1e-3, prefix_len=P, x_last=to_dev(xp[:, -1]))
    cache, x_last = O.prefill(p64[0], xp, H)
    x_t, it_t = O.inverse_jacobi_block(p64[0], z, H, F, 1e-3, pos0=P, cache=cache,
                                       x_last=x_last)
    xo = x_t
    if not np.array_equal(it_t, itg[0]):
        xo, _ = O.inverse_jacobi_block(p64[0], z, H, F, 1e-3, pos0=P, cache=cache,
                                       x_last=x_last, forced_iters=list(itg[0]))
    print("iters gpu", itg.tolist(), "oracle", it_t.tolist(), "x rel_l2", rel_l2(to_np(xg), xo))
    assert rel_l2(to_np(xg), xo) < TOL_BF16
    # the merge adds the chunks in a fixed order whichever chunk finishes
    # last, so a second run is bit for bit the same
    plan.prefill(to_dev(xp), rows=F)
    xg2, itg2 = plan.inverse_jacobi(to_dev(z), F, 1e-3, prefix_len=P, x_last=to_dev(xp[:, -1]))
    assert np.array_equal(itg2, itg) and torch.equal(xg2, xg)


def test_row_split_matches_single_pass_and_oracle(B):
    """Row split of the Jacobi update (two streams: a 1024-row block after an
    8192-token prefix, so the split applies): a forced count of 3 updates
    against the oracle and against the single pass, and the tau stop against
    the single pass (same count within one update)."""
    say("row split")
    P, R = 8192, 1024
    cfg, params, p64 = problem(C=48, d=256, H=4, layers=1, max_len=P + R, dtype="bf16",
                               seed=70)
    plan = B.AFPlan(cfg, params)
    xp = synth.normal((1, P, 48), 71)
    z = synth.normal((1, R, 48), 72)
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
        plan.prefill(to_dev(xp), rows=R)
        xt, itt = plan.inverse_jacobi(to_dev(z), R, 1e-3, prefix_len=P,
                                      x_last=to_dev(xp[:, -1]))
        out[split] = (to_np(xf), itf, to_np(xt), itt)
    (fa, ia, ta, ja), (fb, ib, tb, jb) = out[True], out[False]
    cache, x_last = O.prefill(p64[0], xp, 4)
    xo, _ = O.inverse_jacobi_block(p64[0], z, 4, R, 0.0, forced_iters=[3], pos0=P,
                                   cache=cache, x_last=x_last)
    e_or, e_ss = rel_l2(fa, xo), rel_l2(fa, fb)
    print(f"forced 3: split vs oracle {e_or:.2e}, split vs single pass {e_ss:.2e}; "
          f"tau: iters {ja.tolist()} / {jb.tolist()}")
    assert ia[0][0] == 3 and ib[0][0] == 3
    assert e_or < TOL_BF16 and rel_l2(fb, xo) < TOL_BF16
    assert e_ss < 2e-3
    assert abs(int(ja[0][0]) - int(jb[0][0])) <= 1
    if ja[0][0] == jb[0][0]:
        assert rel_l2(ta, tb) < 2e-3


def test_row_split_batch_of_two(B):
    """The row split with two samples (each sample's rows halved, residual
    pairs per sample and half): the same as the single pass, forced count and
    tau stop, the two samples' counts shared."""
    say("row split, batch 2")
    P, R, N = 8192, 1024, 2
    cfg, params, _ = problem(C=48, d=256, H=4, layers=1, max_len=P + R, dtype="bf16", seed=73)
    plan = B.AFPlan(cfg, params)
    xp = to_dev(synth.normal((N, P, 48), 74))
    z = to_dev(synth.normal((N, R, 48), 75))
    out = {}
    for split in (True, False):
        plan.set_row_split(split)
        plan.prefill(xp, rows=R)
        plan.profile_enable("affine")
        xf, itf = plan.inverse_jacobi(z, R, 0.0, 2, prefix_len=P, x_last=xp[:, -1].contiguous())
        n_aff, _ = plan.profile_read()
        plan.profile_disable()
        assert n_aff == (4 if split else 2)
        plan.prefill(xp, rows=R)
        xt, itt = plan.inverse_jacobi(z, R, 1e-3, prefix_len=P, x_last=xp[:, -1].contiguous())
        out[split] = (to_np(xf), itf, to_np(xt), itt)
    (fa, ia, ta, ja), (fb, ib, tb, jb) = out[True], out[False]
    print(f"forced: rel {rel_l2(fa, fb):.2e}; tau: iters {ja.tolist()} / {jb.tolist()}, "
          f"rel {rel_l2(ta, tb):.2e}")
    assert ia[0][0] == 2 and ib[0][0] == 2 and rel_l2(fa, fb) < 2e-3
    assert abs(int(ja[0][0]) - int(jb[0][0])) <= 1
    if ja[0][0] == jb[0][0]:
        assert rel_l2(ta, tb) < 2e-3
    assert np.isfinite(ta).all()


def test_frame480p_fullsize(B):
    """One 1560-token frame, 8 layers d=1024, B=1560, zero init, tau=1e-3."""
    w = synth.WORKLOADS["frame480p"]
    say("frame480p full size")
    params = synth.make_params(w.block, 0)
    p64 = O.to64(params[0])
    plan = B.AFPlan(w.block, params)
    z = synth.normal((1, 1560, 48), 1)
    xg, itg = plan.inverse_jacobi(to_dev(z), 1560, 1e-3)
    xg_np = to_np(xg)
    # prefix of the block, oracle forced to the GPU's count
    xo, _ = O.inverse_jacobi_block(p64, z[:, :PREFIX], 16, PREFIX, 1e-3,
                                   forced_iters=[int(itg[0, 0])])
    e_pre = rel_l2(xg_np[:, :PREFIX], xo)
    # fixed-point defect of the whole frame under the oracle's forward
    zf, _ = O.forward_block(p64, xg_np, 16)
    defect = rel_l2(zf, z)
    # and the GPU's forward of a random x against the oracle's
    xin = synth.normal((1, 1560, 48), 2)
    zgf, ldg = plan.forward(to_dev(xin))
    zof, ldo = O.forward_block(p64, xin, 16)
    e_fwd = rel_l2(to_np(zgf), zof)
    e_ld = abs(float(to_np(ldg)[0]) - ldo[0]) / abs(ldo[0])
    print(f"iters {itg.tolist()} prefix rel_l2 {e_pre:.2e} defect {defect:.2e} "
          f"forward rel_l2 {e_fwd:.2e} logdet rel {e_ld:.2e}")
    assert e_pre < TOL_BF16
    assert defect < 0.05
    assert e_fwd < TOL_BF16


def test_video21_fullsize(B):
    """21 frames x 1560 tokens, block = frame, previous-frame warm start."""
    w = synth.WORKLOADS["video21"]
    say("video21 full size")
    params = synth.make_params(w.block, 0)
    p64 = O.to64(params[0])
    plan = B.AFPlan(w.block, params)
    F = 1560
    z = synth.normal((1, 21 * F, 48), 1)
    zd = to_dev(z)
    xg, itg = plan.inverse_jacobi(zd, F, 1e-3, init="prev_frame", frame_len=F)
    xg_np = to_np(xg)
    print("iters per frame", itg.tolist())
    assert itg.shape == (1, 21) and np.all(itg >= 1) and np.all(itg <= F)
    # frame 0: prefix equality with the oracle forced to the GPU's count
    xo, _ = O.inverse_jacobi_block(p64, z[:, :PREFIX], 16, PREFIX, 1e-3,
                                   forced_iters=[int(itg[0, 0])])
    e_pre = rel_l2(xg_np[:, :PREFIX], xo)
    # frames 0-1: fixed-point defect under the oracle's forward
    zf, _ = O.forward_block(p64, xg_np[:, :2 * F], 16)
    d01 = rel_l2(zf, z[:, :2 * F])
    # all 21 frames: defect under the GPU's own forward
    zg, _ = plan.forward(xg)
    d_all = rel_l2(to_np(zg), z)
    print(f"frame0 prefix rel_l2 {e_pre:.2e}; defect frames0-1 {d01:.2e}; "
          f"defect all (GPU forward) {d_all:.2e}")
    assert e_pre < TOL_BF16
    assert d01 < 0.05 and d_all < 0.05


def test_shallow_stack_fullsize(B):
    """T=4 alternating blocks, 2 layers d=512, 21 frames batched."""
    w = synth.WORKLOADS["shallow_stack"]
    say("shallow_stack full size")
    params = synth.make_params(w.block, 0, n_blocks=4)
    ps64 = [O.to64(p) for p in params]
    plan = B.AFPlan(w.block, params)
    x = synth.noisy_latents((21, 1560, 48), 2, 0.3)
    zg, ldg = plan.forward(to_dev(x))
    xg, itg = plan.inverse_jacobi(zg, 1560, 1e-3)
    print("iters per stack block", itg.tolist())
    zg_np, xg_np = to_np(zg), to_np(xg)
    for n in (0, 20):   # sampled frames, run alone by the oracle
        zo, ldo = O.forward_stack(ps64, x[n:n + 1], 8)
        e_z = rel_l2(zg_np[n:n + 1], zo)
        e_ld = abs(float(to_np(ldg)[n]) - ldo[0]) / abs(ldo[0])
        xo, _ = O.inverse_jacobi_stack(ps64, zg_np[n:n + 1], 8, 1560, 1e-3,
                                       forced_iters=itg)
        e_x = rel_l2(xg_np[n:n + 1], xo)
        print(f"frame {n}: z rel_l2 {e_z:.2e} logdet rel {e_ld:.2e} x rel_l2 {e_x:.2e}")
        assert e_z < TOL_BF16 and e_x < TOL_BF16
    assert rel_l2(xg_np, x) < 0.1


def test_wide_prefix_fullsize(B):
    """4 layers d=4096 (dh=128), 2-frame prefix, one frame, batch 2: checked by
    the fixed-point defect under the GPU forward of prefix ++ x, and the
    prefix structure against the oracle at full width with a short frame."""
    w = synth.WORKLOADS["wide_prefix"]
    say("wide_prefix full size")
    params = synth.make_params(w.block, 0)
    plan = B.AFPlan(w.block, params)
    F = 1560
    xp = synth.normal((2, 2 * F, 48), 2)
    z = synth.normal((2, F, 48), 1)
    plan.prefill(to_dev(xp), rows=F)
    xg, itg = plan.inverse_jacobi(to_dev(z), F, 1e-3, init="given",
                                  x_init=to_dev(np.ascontiguousarray(xp[:, F:])),
                                  prefix_len=2 * F, x_last=to_dev(xp[:, -1]))
    print("iters", itg.tolist())
    full = torch.cat([to_dev(xp), xg], dim=1).contiguous()
    zg, _ = plan.forward(full)
    d = rel_l2(to_np(zg)[:, 2 * F:], z)
    print(f"defect (GPU forward of prefix ++ x) {d:.2e}")
    assert d < 0.05


def test_wide_width_prefix_vs_oracle(B):
    """Full width d=4096, dh=128, one layer, short frames: prefix + GIVEN init
    against the oracle element by element."""
    say("wide width prefix vs oracle")
    F = 96
    cfg = synth.BlockCfg(C=48, d=4096, n_heads=32, n_layers=1, max_len=3 * F, dtype="bf16")
    params = synth.make_params(cfg, 0)
    p64 = O.to64(params[0])
    plan = B.AFPlan(cfg, params)
    xp = synth.normal((2, 2 * F, 48), 2)
    z = synth.normal((2, F, 48), 1)
    plan.prefill(to_dev(xp), rows=F)
    x_init = np.ascontiguousarray(xp[:, F:])
    xg, itg = plan.inverse_jacobi(to_dev(z), F, 1e-3, init="given", x_init=to_dev(x_init),
                                  prefix_len=2 * F, x_last=to_dev(xp[:, -1]))
    cache, x_last = O.prefill(p64, xp, 32)
    xo, _ = O.inverse_jacobi_block(p64, z, 32, F, 1e-3, init="given", x_init=x_init,
                                   pos0=2 * F, cache=cache, x_last=x_last,
                                   forced_iters=list(itg[0]))
    e = rel_l2(to_np(xg), xo)
    print("iters", itg.tolist(), f"x rel_l2 {e:.2e}")
    assert e < TOL_BF16
