"""GPU parity: the HIP path (through the C ABI) against the CPU fp64 oracle on
the same seeded inputs.  Bars: relative L2 <= 1e-4 on the fp32 path and
<= 2e-2 on the bf16 path, log-det relative error <= 1e-3; Jacobi iteration
counts reported side by side (equal on the fp32 path; on the bf16 path the
oracle is re-run forced to the GPU's counts when they differ).

Method: STARFlow-V notes (papernotes.org), 关键设计 1 (affine AF block,
alternating directions), 关键设计 3 (block-wise Jacobi with KV cache, warm
start, residual stop), 一个完整示例 (prefix encoding into the KV cache)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from autoregressive_normalizing_flow_amd import synth  # noqa: E402
from oracle import af_oracle as O  # noqa: E402
from parity_util import (TOL_BF16, TOL_BF16_TOKEN, TOL_F32, TOL_LOGDET,  # noqa: E402
                         oracle_jacobi_like, problem, rel_err, rel_l2, say, to_dev, to_np,
                         token_rel_max)

pytestmark = pytest.mark.gpu

# fp32 end-to-end cases run on both inverse paths: the device loop (the
# default for the shapes it covers) and the launch-per-kernel path
PATHS = pytest.mark.parametrize("dl", [True, False], ids=["device_loop", "launches"])


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from autoregressive_normalizing_flow_amd import binding
    binding.load_library()
    return binding


# ---------------------------------------------------------------------------
# kernel units
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,N,K", [(200, 192, 128), (1560, 384, 256), (1, 128, 64),
                                   (333, 1024, 512)])
def test_gemm_bf16_unit(B, M, N, K):
    say("gemm_bf16", M, N, K)
    rng = np.random.default_rng(M + N + K)
    a = synth.bf16_round(rng.standard_normal((M, K)).astype(np.float32))
    w = synth.bf16_round(rng.standard_normal((N, K)).astype(np.float32))
    bias = rng.standard_normal(N).astype(np.float32)
    y = B.afk_gemm_bf16(to_dev(a).to(torch.bfloat16), to_dev(w).to(torch.bfloat16),
                        to_dev(bias))
    torch.cuda.synchronize()
    ref = a.astype(np.float64) @ w.astype(np.float64).T + bias
    assert rel_l2(to_np(y), ref) < 1e-6


# (2, 349531, 48): above the size where the kernel streams (four rows in
# flight per thread, non-temporal access), with a ragged last pass
@pytest.mark.parametrize("N,rows,C", [(3, 77, 48), (1, 1560, 48), (2, 5, 16),
                                      (2, 349531, 48)])
def test_affine_unit_both_modes(B, N, rows, C):
    say("affine", N, rows, C)
    rng = np.random.default_rng(rows)
    head = rng.standard_normal((N * rows, 2 * C)).astype(np.float32)
    z = rng.standard_normal((N, rows, C)).astype(np.float32)
    x_old = rng.standard_normal((N, rows, C)).astype(np.float32)
    mu = head[:, :C].reshape(N, rows, C).astype(np.float64)
    ls = 0.5 * np.tanh(head[:, C:].reshape(N, rows, C).astype(np.float64))
    part = torch.empty(B.afk_affine_partials_bytes(N, rows, C), dtype=torch.uint8,
                       device="cuda")
    res = torch.empty(N, 2, device="cuda")
    # inverse mode: x <- mu + sigma z in place, residual sums
    x = to_dev(x_old)
    B.afk_affine(0, to_dev(head), to_dev(z), x, N, rows, C, res, part, check=True)
    x_ref = mu + np.exp(ls) * z
    assert rel_l2(to_np(x), x_ref) < 1e-6
    num = ((x_ref - x_old) ** 2).sum(axis=(1, 2))
    den = (x_ref ** 2).sum(axis=(1, 2))
    r = to_np(res)
    assert np.all(rel_err(r[:, 0], num) < 1e-5) and np.all(rel_err(r[:, 1], den) < 1e-5)
    # forward mode: z = (x - mu) / sigma and -sum log sigma
    zo = torch.empty_like(x)
    B.afk_affine(1, to_dev(head), to_dev(x_old), zo, N, rows, C, res, part, check=True)
    assert rel_l2(to_np(zo), (x_old - mu) * np.exp(-ls)) < 1e-6
    r = to_np(res)
    assert np.all(rel_err(r[:, 0], -ls.sum(axis=(1, 2))) < 1e-4)
    assert np.all(r[:, 1] == 0)


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, (1 << 26) + 48])
def test_stream_copy_exact(B, nbytes):
    say("stream copy", nbytes)
    src = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    B.afk_stream_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_affine_flags_nonfinite(B):
    say("affine nonfinite")
    N, rows, C = 2, 33, 8
    head = torch.zeros(N * rows, 2 * C, device="cuda")
    z = torch.ones(N, rows, C, device="cuda")
    z[1, 7, 3] = float("nan")
    x = torch.zeros_like(z)
    part = torch.empty(B.afk_affine_partials_bytes(N, rows, C), dtype=torch.uint8,
                       device="cuda")
    res = torch.empty(N, 2, device="cuda")
    with pytest.raises(B.AFError) as ei:
        B.afk_affine(0, head, z, x, N, rows, C, res, part, check=True)
    assert ei.value.status == B.AF_ERR_NONFINITE


def test_forward_flags_and_grouped_logdet(B):
    """af_forward on a stack of two blocks over six frames: with
    frames_per_entry = 3 the two log-det entries are the sums of the oracle's
    per-frame log-dets (关键设计 1: one shallow factor per frame); with
    AF_FWD_ACCUMULATE they add to what the buffer held; a NaN in frame 4 is
    reported (AF_ERR_NONFINITE, stack block 0) only when the check is asked
    for."""
    say("forward flags")
    cfg, params, ps64 = problem(C=16, d=256, H=4, layers=1, max_len=40, dtype="bf16",
                                seed=19, n_blocks=2)
    plan = B.AFPlan(cfg, params)
    x = synth.normal((6, 40, 16), 20)
    zo, ldo = O.forward_stack(ps64, x, 4)
    zg, ldg = plan.forward(to_dev(x), frames_per_entry=3, check_finite=True)
    assert ldg.shape == (2,)
    assert rel_l2(to_np(zg), zo) < TOL_BF16
    sums = ldo.reshape(2, 3).sum(axis=1)
    assert np.all(rel_err(to_np(ldg), sums) < TOL_LOGDET)
    base = torch.tensor([1.5, -2.0], device="cuda")
    _, lda = plan.forward(to_dev(x), logdet=base.clone(), frames_per_entry=3,
                          accumulate=True)
    assert np.all(rel_err(to_np(lda), sums + np.array([1.5, -2.0])) < TOL_LOGDET)
    xb = x.copy()
    xb[4, 9, 2] = np.nan
    with pytest.raises(B.AFError) as ei:
        plan.forward(to_dev(xb), check_finite=True)
    assert ei.value.status == B.AF_ERR_NONFINITE and "stack block 0" in str(ei.value)
    zn, _ = plan.forward(to_dev(xb))   # stream-ordered: no check, no error
    torch.cuda.synchronize()
    assert not np.isfinite(to_np(zn)[4]).all() and np.isfinite(to_np(zn)[:4]).all()
    # a clean call afterwards passes the check (the tag starts at zero per call)
    plan.forward(to_dev(x), check_finite=True)


@PATHS
@pytest.mark.parametrize("tau", [1e-3, 0.0])
def test_inverse_flags_nonfinite(B, tau, dl):
    """A NaN latent in the second Jacobi block: reported as AF_ERR_NONFINITE
    whether the residual is read back every iteration (tau > 0) or only the
    sticky tag at the end (forced count)."""
    say("inverse nonfinite", tau)
    w = synth.WORKLOADS["tiny_f32"]
    params = synth.make_params(w.block, 0)
    plan = B.AFPlan(w.block, params)
    plan.set_device_loop(dl)
    z = synth.normal((1, 64, 16), 1)
    z[0, 20, 5] = np.nan
    with pytest.raises(B.AFError) as ei:
        plan.inverse_jacobi(to_dev(z), 16, tau, max_iters=3)
    assert ei.value.status == B.AF_ERR_NONFINITE
    assert "Jacobi block 1" in str(ei.value)
    # the plan stays usable: a clean call after the failure equals a fresh plan's
    z[0, 20, 5] = 0.0
    xa, ia = plan.inverse_jacobi(to_dev(z), 16, tau, max_iters=3)
    fresh = B.AFPlan(w.block, params)
    fresh.set_device_loop(dl)
    xb, ib = fresh.inverse_jacobi(to_dev(z), 16, tau, max_iters=3)
    torch.cuda.synchronize()
    assert np.array_equal(ia, ib) and torch.equal(xa, xb)


def test_back_to_back_calls_without_sync(B):
    """An inverse call returns once its last update has published its
    residual, possibly with kernels still queued: three calls in a row on one
    plan and stream, with no synchronisation between them (and the plan
    destroyed right after the last), equal the same calls made one at a
    time."""
    say("back-to-back inverse calls")
    cfg, params, _ = problem(C=48, d=256, H=4, layers=2, max_len=96, dtype="bf16", seed=21)
    plan = B.AFPlan(cfg, params)
    zs = [to_dev(synth.normal((2, 96, 48), 22 + i)) for i in range(3)]
    ref = []
    for z in zs:
        x, it = plan.inverse_jacobi(z, 32, 1e-3)
        torch.cuda.synchronize()
        ref.append((x.clone(), it.copy()))
    out = [plan.inverse_jacobi(z, 32, 1e-3) for z in zs]
    del plan   # destroyed with the last call's kernels possibly still queued
    torch.cuda.synchronize()
    for (x, it), (xr, itr) in zip(out, ref):
        assert np.array_equal(it, itr) and torch.equal(x, xr)


# ---------------------------------------------------------------------------
# fp32 path, end to end
# ---------------------------------------------------------------------------
@PATHS
def test_tiny_f32_forward_and_inverse(B, dl):
    """One 8x8 latent frame, C=16, 1 layer d=64, 2 heads, fp32, B=16, tau=1e-3."""
    w = synth.WORKLOADS["tiny_f32"]
    say("tiny_f32")
    params = synth.make_params(w.block, 0)
    p64 = O.to64(params[0])
    plan = B.AFPlan(w.block, params)
    plan.set_device_loop(dl)
    z = synth.normal((1, 64, 16), 1)
    x_in = synth.normal((1, 64, 16), 2)
    # forward of x
    zg, ldg = plan.forward(to_dev(x_in))
    zo, ldo = O.forward_block(p64, x_in, 2)
    assert rel_l2(to_np(zg), zo) < TOL_F32
    assert np.all(rel_err(to_np(ldg), ldo) < TOL_LOGDET)
    # Jacobi inverse of z ~ N(0, 1)
    xg, itg = plan.inverse_jacobi(to_dev(z), 16, 1e-3)
    xo, ito = O.inverse_jacobi_block(p64, z, 2, 16, 1e-3)
    print("iters gpu", itg.tolist(), "oracle", ito.tolist())
    assert np.array_equal(itg[0], ito)
    assert rel_l2(to_np(xg), xo) < TOL_F32
    # forward then inverse recovers x up to the stop threshold, and the GPU's
    # round trip equals the oracle's
    xr, itr = plan.inverse_jacobi(zg, 16, 1e-3)
    xor_, itor = O.inverse_jacobi_block(p64, zo, 2, 16, 1e-3)
    assert np.array_equal(itr[0], itor)
    assert rel_l2(to_np(xr), xor_) < TOL_F32
    assert rel_l2(to_np(xr), x_in) < 0.05


@PATHS
def test_f32_stack_ragged_r2l(B, dl):
    """T=2 (L->R, R->L), ragged last Jacobi block, batch 3, dh=32."""
    say("f32 stack ragged")
    cfg, params, p64 = problem(C=5, d=64, H=2, layers=2, max_len=60, dtype="f32",
                               seed=3, n_blocks=2)
    plan = B.AFPlan(cfg, params)
    plan.set_device_loop(dl)
    x_in = synth.normal((3, 60, 5), 4)
    zg, ldg = plan.forward(to_dev(x_in))
    zo, ldo = O.forward_stack(p64, x_in, 2)
    assert rel_l2(to_np(zg), zo) < TOL_F32
    assert np.all(rel_err(to_np(ldg), ldo) < TOL_LOGDET)
    xg, itg = plan.inverse_jacobi(zg, 16, 1e-3)
    xo, ito = O.inverse_jacobi_stack(p64, zo, 2, 16, 1e-3)
    print("iters gpu", itg.tolist(), "oracle", ito.tolist())
    assert np.array_equal(itg, ito)
    assert rel_l2(to_np(xg), xo) < TOL_F32


@pytest.mark.parametrize("C,d,N,L,Bj", [(24, 128, 2, 70, 32), (64, 256, 1, 50, 50),
                                         (8, 512, 3, 33, 16)])
@PATHS
def test_f32_head_mfma_shapes(B, C, d, N, L, Bj, dl):
    """The fp32-MFMA head at other channel counts (2C = 48, 128, 16 columns),
    K split over 1..8 ranges, ragged 16-row tiles, batch."""
    say("f32 head mfma", C, d, N, L, Bj)
    H = d // 64
    cfg, params, (p64,) = problem(C=C, d=d, H=H, layers=1, max_len=L, dtype="f32",
                                  seed=C + d)
    plan = B.AFPlan(cfg, params)
    plan.set_device_loop(dl)
    x_in = synth.normal((N, L, C), C + 1)
    zg, ldg = plan.forward(to_dev(x_in))
    zo, ldo = O.forward_block(p64, x_in, H)
    assert rel_l2(to_np(zg), zo) < TOL_F32
    assert np.all(rel_err(to_np(ldg), ldo) < TOL_LOGDET)
    z = synth.normal((N, L, C), C + 2)
    xg, itg = plan.inverse_jacobi(to_dev(z), Bj, 1e-3)
    xo, ito = O.inverse_jacobi_block(p64, z, H, Bj, 1e-3)
    print("iters gpu", itg.tolist(), "oracle", ito.tolist())
    assert np.array_equal(itg[0], ito)
    assert rel_l2(to_np(xg), xo) < TOL_F32


def test_bf16_head_vector_path(B):
    """C = 20 (2C not a multiple of 16): the head runs on the vector-ALU fp32
    GEMM, and block refreshes run as separate passes."""
    say("bf16 C=20 L=150 B=64")
    _bf16_block_case(B, d=256, H=4, layers=1, L=150, Bj=64, N=2, seed=23, C=20)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fused_refresh_matches_separate_pass(B, dtype):
    """A block that stops early has its K/V recomputed from its final tokens;
    merged into the next block's first update (one pass over both blocks'
    rows) the result equals the separate pass: bit for bit on the fp32 path,
    to summation order on the bf16 path; both match the oracle."""
    say("fused refresh", dtype)
    if dtype == "f32":
        cfg, params, (p64,) = problem(C=8, d=64, H=2, layers=2, max_len=100, dtype="f32",
                                      seed=60)
        N, L, Bj, C, H = 2, 100, 32, 8, 2
    else:
        cfg, params, (p64,) = problem(C=48, d=256, H=4, layers=2, max_len=300, dtype="bf16",
                                      seed=61)
        N, L, Bj, C, H = 2, 300, 96, 48, 4
    plan = B.AFPlan(cfg, params)
    # both runs on the launch-per-kernel path (the fused refresh is one of
    # its options; the device loop refreshes inside its own kernel)
    plan.set_device_loop(False)
    z = to_dev(synth.normal((N, L, C), 62))
    ws = plan.workspace(N, min(2 * Bj, L))
    out = {}
    for fused in (False, True):
        plan.set_fused_refresh(fused)
        x = torch.empty_like(z)
        it = np.zeros((1, -(-L // Bj)), np.int32)
        B.af_inverse_jacobi(plan, z, Bj, 1e-3, 0, "zero", None, 0, 0, None, x, it, ws)
        torch.cuda.synchronize()
        out[fused] = (x, it)
    (x0, it0), (x1, it1) = out[False], out[True]
    print("iters separate", it0.tolist(), "fused", it1.tolist())
    assert np.all(it0[0][:-1] < Bj)                 # early stops: refreshes happen
    xo, ito = oracle_jacobi_like(p64, to_np(z), H, Bj, 1e-3, it1[0])
    if dtype == "f32":
        assert np.array_equal(it0, it1) and torch.equal(x0, x1)
        assert np.array_equal(it1[0], ito)
        assert rel_l2(to_np(x1), xo) < TOL_F32
    else:
        assert np.all(np.abs(it0 - it1) <= 1)
        assert rel_l2(to_np(x1), to_np(x0)) < 1e-2
        assert rel_l2(to_np(x1), xo) < TOL_BF16


@pytest.mark.parametrize("prefix", [0, 192])
def test_refresh_beside_next_block_matches_serial(B, prefix):
    """A block that stops early has its K/V recomputed from its final tokens;
    run on the plan's second stream beside the next block's first update
    (whose attention waits for it layer by layer) the result equals the
    refresh on the call's stream bit for bit, blocks and iteration counts
    alike, and matches the oracle.  Two samples, three layers, blocks of 96
    rows with a ragged last block, after an encoded prefix or none."""
    say("refresh beside the next block, prefix", prefix)
    N, L, Bj, C, H = 2, 300, 96, 48, 4
    cfg, params, (p64,) = problem(C=C, d=256, H=H, layers=3, max_len=prefix + L,
                                  dtype="bf16", seed=63)
    plan = B.AFPlan(cfg, params)
    z = synth.normal((N, L, C), 64)
    xp = synth.normal((N, prefix, C), 65) if prefix else None
    kw = {}
    if prefix:
        cache, x_last = O.prefill(p64, xp, H)
        kw = dict(pos0=prefix, cache=cache, x_last=x_last)
    out = {}
    for overlap in (False, True):
        plan.set_overlap_refresh(overlap)
        if prefix:
            plan.prefill(to_dev(xp))
            x, it = plan.inverse_jacobi(to_dev(z), Bj, 1e-3, prefix_len=prefix,
                                        x_last=to_dev(xp[:, -1]))
        else:
            x, it = plan.inverse_jacobi(to_dev(z), Bj, 1e-3)
        torch.cuda.synchronize()
        out[overlap] = (x, it)
    (x0, it0), (x1, it1) = out[False], out[True]
    print("iters serial", it0.tolist(), "beside", it1.tolist())
    assert np.all(it0[0][:-1] < Bj)                 # early stops: refreshes happen
    assert np.array_equal(it0, it1) and torch.equal(x0, x1)
    xo, _ = oracle_jacobi_like(p64, z, H, Bj, 1e-3, it1[0], **kw)
    e, et = rel_l2(to_np(x1), xo), token_rel_max(to_np(x1), xo)
    print(f"beside, prefix {prefix}: rel_l2 {e:.2e}, max per-token {et:.2e}")
    assert e < TOL_BF16 and et < TOL_BF16_TOKEN


def test_refresh_beside_next_block_in_a_stack(B):
    """A bf16 stack of two alternating AF blocks (two layers each) with three
    Jacobi blocks per AF block: refreshes run beside the next Jacobi block
    inside each AF block, and the next AF block (which rewrites the same cache
    rows with its own K/V) starts only after them.  Equal to every refresh on
    the call's stream, bit for bit, and to the oracle's stack inverse forced to
    the GPU's counts."""
    say("refresh beside the next block: stack T=2")
    N, L, Bj, C, H = 2, 240, 80, 48, 4
    cfg, params, p64 = problem(C=C, d=256, H=H, layers=2, max_len=L, dtype="bf16",
                               seed=68, n_blocks=2)
    plan = B.AFPlan(cfg, params)
    z = synth.normal((N, L, C), 69)
    out = {}
    for overlap in (False, True):
        plan.set_overlap_refresh(overlap)
        x, it = plan.inverse_jacobi(to_dev(z), Bj, 1e-3)
        torch.cuda.synchronize()
        out[overlap] = (x, it)
    (x0, it0), (x1, it1) = out[False], out[True]
    print("iters serial", it0.tolist(), "beside", it1.tolist())
    assert np.all(it1[:, :-1] < Bj)                 # early stops in both AF blocks
    assert np.array_equal(it0, it1) and torch.equal(x0, x1)
    xo, _ = O.inverse_jacobi_stack(p64, z, H, Bj, 1e-3, forced_iters=it1)
    e, et = rel_l2(to_np(x1), xo), token_rel_max(to_np(x1), xo)
    print(f"stack beside: rel_l2 {e:.2e}, max per-token {et:.2e}")
    assert e < TOL_BF16 and et < TOL_BF16_TOKEN


def test_refresh_beside_next_block_needs_its_workspace(B):
    """With a workspace one byte short of af_workspace_bytes (room for the
    main layout but not for the refresh's scratch) every refresh runs on the
    call's stream: the same result, bit for bit, as with the full workspace."""
    say("refresh beside the next block: small workspace")
    N, L, Bj, C, H = 1, 288, 96, 48, 4
    cfg, params, _ = problem(C=C, d=256, H=H, layers=2, max_len=L, dtype="bf16", seed=70)
    plan = B.AFPlan(cfg, params)
    z = to_dev(synth.normal((N, L, C), 71))
    ws = plan.workspace(N, Bj)
    assert ws.numel() == plan.workspace_bytes(N, Bj)
    out = []
    for w in (ws, ws[:-1]):
        x = torch.empty_like(z)
        it = np.zeros((1, -(-L // Bj)), np.int32)
        B.af_inverse_jacobi(plan, z, Bj, 1e-3, 0, "zero", None, 0, 0, None, x, it, w)
        torch.cuda.synchronize()
        out.append((x, it))
    (xa, ia), (xb, ib) = out
    print("iters", ia.tolist())
    assert np.all(ia[0][:-1] < Bj)
    assert np.array_equal(ia, ib) and torch.equal(xa, xb)


def test_refresh_beside_next_block_error_path(B):
    """A non-finite value in a later block while an earlier block's refresh
    may still run on the plan's second stream: the call reports
    AF_ERR_NONFINITE for that block (with the calling stream ordered after
    the second stream's work), and a clean call on the same plan afterwards
    equals a fresh plan's, bit for bit."""
    say("refresh beside the next block: error path")
    N, L, Bj, C, H = 1, 288, 96, 48, 4
    cfg, params, _ = problem(C=C, d=256, H=H, layers=2, max_len=L, dtype="bf16", seed=66)
    plan = B.AFPlan(cfg, params)
    z = synth.normal((N, L, C), 67)
    z[0, 2 * Bj + 5, 3] = np.nan                     # in the third block
    with pytest.raises(B.AFError) as ei:
        plan.inverse_jacobi(to_dev(z), Bj, 1e-3)
    assert ei.value.status == B.AF_ERR_NONFINITE
    assert "Jacobi block 2" in str(ei.value)
    z[0, 2 * Bj + 5, 3] = 0.0
    xa, ia = plan.inverse_jacobi(to_dev(z), Bj, 1e-3)
    fresh = B.AFPlan(cfg, params)
    xb, ib = fresh.inverse_jacobi(to_dev(z), Bj, 1e-3)
    torch.cuda.synchronize()
    print("iters", ia.tolist())
    assert np.all(ia[0][:-1] < Bj)                  # early stops: refreshes ran beside
    assert np.array_equal(ia, ib) and torch.equal(xa, xb)


@PATHS
def test_f32_forced_count_and_sequential(B, dl):
    say("f32 forced + B=1")
    cfg, params, (p64,) = problem(C=4, d=64, H=1, layers=1, max_len=20, dtype="f32", seed=5)
    plan = B.AFPlan(cfg, params)
    plan.set_device_loop(dl)
    z = synth.normal((2, 20, 4), 6)
    xg, itg = plan.inverse_jacobi(to_dev(z), 8, 0.0, max_iters=3)
    assert np.all(itg == 3)
    xo, _ = O.inverse_jacobi_block(p64, z, 1, 8, 0.0, max_iters=3)
    assert rel_l2(to_np(xg), xo) < TOL_F32
    # B = 1: one update per token is sequential decoding
    x1, it1 = plan.inverse_jacobi(to_dev(z), 1, 1e-3)
    assert np.all(it1 == 1)
    assert rel_l2(to_np(x1), O.inverse_sequential_block(p64, z, 1)) < TOL_F32
    # tau <= 0 with no cap runs Bb updates and reaches the sequential solution
    xf, itf = plan.inverse_jacobi(to_dev(z), 8, 0.0)
    assert itf.tolist() == [[8, 8, 4]]
    assert rel_l2(to_np(xf), O.inverse_sequential_block(p64, z, 1)) < TOL_F32


@PATHS
def test_f32_prefill_given_prevframe(B, dl):
    say("f32 prefill/given/prev_frame")
    cfg, params, (p64,) = problem(C=6, d=128, H=2, layers=2, max_len=96, dtype="f32", seed=7)
    plan = B.AFPlan(cfg, params)
    plan.set_device_loop(dl)
    xp = synth.normal((2, 32, 6), 8)
    z = synth.normal((2, 64, 6), 9)
    xinit = synth.normal((2, 64, 6), 10)
    plan.prefill(to_dev(xp), rows=64)
    xg, itg = plan.inverse_jacobi(to_dev(z), 32, 1e-3, init="given", x_init=to_dev(xinit),
                                  prefix_len=32, x_last=to_dev(xp[:, -1]))
    cache, x_last = O.prefill(p64, xp, 2)
    xo, ito = O.inverse_jacobi_block(p64, z, 2, 32, 1e-3, init="given", x_init=xinit,
                                     pos0=32, cache=cache, x_last=x_last)
    print("iters gpu", itg.tolist(), "oracle", ito.tolist())
    assert np.array_equal(itg[0], ito)
    assert rel_l2(to_np(xg), xo) < TOL_F32
    # previous-frame warm start, frames of 16 tokens = one block each
    z2 = synth.normal((1, 48, 6), 11)
    xg2, itg2 = plan.inverse_jacobi(to_dev(z2), 16, 1e-3, init="prev_frame", frame_len=16)
    xo2, ito2 = O.inverse_jacobi_block(p64, z2, 2, 16, 1e-3, init="prev_frame", frame_len=16)
    print("iters gpu", itg2.tolist(), "oracle", ito2.tolist())
    assert np.array_equal(itg2[0], ito2)
    assert rel_l2(to_np(xg2), xo2) < TOL_F32


@PATHS
def test_f32_run_twice_bitwise(B, dl):
    say("f32 determinism")
    cfg, params, _ = problem(C=8, d=64, H=2, layers=2, max_len=80, dtype="f32", seed=12)
    plan = B.AFPlan(cfg, params)
    plan.set_device_loop(dl)
    z = to_dev(synth.normal((2, 80, 8), 13))
    a, ia = plan.inverse_jacobi(z, 32, 1e-3)
    b, ib = plan.inverse_jacobi(z, 32, 1e-3)
    assert np.array_equal(ia, ib) and torch.equal(a, b)


# ---------------------------------------------------------------------------
# bf16 path, end to end at reduced sizes (several tiles, ragged tails)
# ---------------------------------------------------------------------------
def _bf16_block_case(B, d, H, layers, L, Bj, N, seed, C=48):
    cfg, params, p64 = problem(C=C, d=d, H=H, layers=layers, max_len=L, dtype="bf16",
                               seed=seed)
    p = p64[0]
    plan = B.AFPlan(cfg, params)
    x_in = synth.normal((N, L, C), seed + 2)
    zg, ldg = plan.forward(to_dev(x_in))
    zo, ldo = O.forward_block(p, x_in, H)
    e_z, e_ld = rel_l2(to_np(zg), zo), rel_err(to_np(ldg), ldo)
    print(f"forward rel_l2 {e_z:.2e} logdet rel {e_ld.max():.2e}")
    assert e_z < TOL_BF16
    assert np.all(e_ld < TOL_LOGDET)
    z = synth.normal((N, L, C), seed + 1)
    xg, itg = plan.inverse_jacobi(to_dev(z), Bj, 1e-3)
    xo, ito = oracle_jacobi_like(p, z, H, Bj, 1e-3, itg[0])
    e_x = rel_l2(to_np(xg), xo)
    print("iters gpu", itg.tolist(), "oracle(tau)", ito.tolist(), f"x rel_l2 {e_x:.2e}")
    assert np.all(np.abs(itg[0] - ito) <= 2)
    assert e_x < TOL_BF16


def test_bf16_block_dh64(B):
    say("bf16 d=256 H=4 L=300 B=128")
    _bf16_block_case(B, d=256, H=4, layers=2, L=300, Bj=128, N=2, seed=20)


def test_bf16_block_dh128(B):
    say("bf16 d=256 H=2 L=200 B=100")
    _bf16_block_case(B, d=256, H=2, layers=1, L=200, Bj=100, N=1, seed=21)


def test_bf16_stack_alternating(B):
    """Shallow-stack structure: T=4 alternating blocks, frames batched."""
    say("bf16 stack T=4")
    cfg, params, p64 = problem(C=48, d=256, H=4, layers=1, max_len=130, dtype="bf16",
                               seed=22, n_blocks=4)
    plan = B.AFPlan(cfg, params)
    x_in = synth.noisy_latents((3, 130, 48), 24, 0.3)
    zg, ldg = plan.forward(to_dev(x_in))
    zo, ldo = O.forward_stack(p64, x_in, 4)
    print("forward", rel_l2(to_np(zg), zo), rel_err(to_np(ldg), ldo))
    assert rel_l2(to_np(zg), zo) < TOL_BF16
    assert np.all(rel_err(to_np(ldg), ldo) < TOL_LOGDET)
    xg, itg = plan.inverse_jacobi(zg, 130, 1e-3)
    xo, ito = O.inverse_jacobi_stack(p64, to_np(zg), 4, 130, 1e-3, forced_iters=itg)
    print("iters gpu", itg.tolist())
    assert rel_l2(to_np(xg), xo) < TOL_BF16
    assert rel_l2(to_np(xg), x_in) < 0.1


def test_bf16_prefill_given(B):
    """Prefix-conditioning structure: 2-frame prefix, then one frame warm-started
    from the last prefix frame, batch 2, dh=128."""
    say("bf16 prefill")
    F = 64
    cfg, params, p64 = problem(C=48, d=256, H=2, layers=2, max_len=3 * F, dtype="bf16",
                               seed=25)
    plan = B.AFPlan(cfg, params)
    xp = synth.normal((2, 2 * F, 48), 27)
    z = synth.normal((2, F, 48), 26)
    plan.prefill(to_dev(xp), rows=F)
    x_init = np.ascontiguousarray(xp[:, F:])
    xg, itg = plan.inverse_jacobi(to_dev(z), F, 1e-3, init="given", x_init=to_dev(x_init),
                                  prefix_len=2 * F, x_last=to_dev(xp[:, -1]))
    cache, x_last = O.prefill(p64[0], xp, 2)
    xo, ito = oracle_jacobi_like(p64[0], z, 2, F, 1e-3, itg[0], init="given",
                                 x_init=x_init, pos0=2 * F, cache=cache, x_last=x_last)
    print("iters gpu", itg.tolist(), "oracle", ito.tolist())
    assert rel_l2(to_np(xg), xo) < TOL_BF16


def test_bf16_video_prev_frame(B):
    """Multi-frame structure: 3 frames of 96 tokens, block = frame, warm start."""
    say("bf16 video prev_frame")
    F = 96
    cfg, params, p64 = problem(C=48, d=256, H=4, layers=2, max_len=3 * F, dtype="bf16",
                               seed=28)
    plan = B.AFPlan(cfg, params)
    z = synth.normal((1, 3 * F, 48), 29)
    xg, itg = plan.inverse_jacobi(to_dev(z), F, 1e-3, init="prev_frame", frame_len=F)
    xo, ito = oracle_jacobi_like(p64[0], z, 4, F, 1e-3, itg[0], init="prev_frame",
                                 frame_len=F)
    print("iters gpu", itg.tolist(), "oracle", ito.tolist())
    assert rel_l2(to_np(xg), xo) < TOL_BF16


def test_bf16_run_twice_bitwise(B):
    say("bf16 determinism")
    cfg, params, _ = problem(C=48, d=256, H=4, layers=2, max_len=200, dtype="bf16", seed=30)
    plan = B.AFPlan(cfg, params)
    z = to_dev(synth.normal((2, 200, 48), 31))
    a, ia = plan.inverse_jacobi(z, 128, 1e-3)
    b, ib = plan.inverse_jacobi(z, 128, 1e-3)
    assert np.array_equal(ia, ib) and torch.equal(a, b)
