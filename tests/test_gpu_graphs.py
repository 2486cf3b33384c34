"""Graph replay of the Jacobi update against direct launches.

af_inverse_jacobi captures one update of a Jacobi block (network pass +
affine update; STARFlow-V notes, 关键设计 3) into a HIP graph and replays it
per iteration.  Each case runs the same inverse with graphs off (every kernel
launched directly) and then several times with graphs on, with direct-launch
work (a forward pass, a direct inverse, torch ops) and synchronisations
between the replays; every replay must match the direct result bit for bit,
iteration counts included, and after the first graph call the cached graphs
must be reused (no new captures).  Parity of the direct path (the default)
with the oracle is covered by the other GPU tests."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from autoregressive_normalizing_flow_amd import synth  # noqa: E402
from parity_util import problem, say, to_dev  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from autoregressive_normalizing_flow_amd import binding
    binding.load_library()
    return binding


def _inverse(B, plan, z, Bj, x, ws, tau=1e-3, max_iters=0, init="zero", frame_len=0):
    N, L, C = z.shape
    iters = np.zeros((plan.T, -(-L // Bj)), np.int32)
    B.af_inverse_jacobi(plan, z, Bj, tau, max_iters, init, None, frame_len, 0, None, x,
                        iters, ws)
    torch.cuda.synchronize()
    return iters


CASES = [
    # dtype, C, d, H, layers, L, Bj, N, T, tau, max_iters, init, frame_len
    ("f32", 8, 64, 2, 2, 100, 32, 2, 1, 1e-3, 0, "zero", 0),
    ("f32", 8, 64, 2, 1, 64, 16, 1, 1, 0.0, 3, "zero", 0),
    ("bf16", 48, 256, 4, 2, 300, 128, 2, 1, 1e-3, 0, "zero", 0),
    ("bf16", 48, 256, 4, 2, 288, 96, 1, 1, 1e-3, 0, "prev_frame", 96),
    ("bf16", 48, 256, 4, 1, 130, 130, 3, 2, 1e-3, 0, "zero", 0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-L{c[5]}-B{c[6]}-T{c[8]}-{c[11]}")
def test_graph_replays_match_direct_launches(B, case):
    dtype, C, d, H, layers, L, Bj, N, T, tau, mi, init, F = case
    say("graph replay", case)
    cfg, params, _ = problem(C=C, d=d, H=H, layers=layers, max_len=L, dtype=dtype,
                             seed=40 + L, n_blocks=T)
    plan = B.AFPlan(cfg, params)
    # graph replay against direct launches of the same kernels (small fp32
    # blocks would otherwise run the Jacobi loop on the device when graphs
    # are off)
    plan.set_device_loop(False)
    z = to_dev(synth.normal((N, L, C), 41 + L))
    ws = plan.workspace(N, min(Bj, L))
    x_d = torch.empty_like(z)
    x_g = torch.empty_like(z)
    kw = dict(tau=tau, max_iters=mi, init=init, frame_len=F)

    plan.set_graphs(False)
    it_d = _inverse(B, plan, z, Bj, x_d, ws, **kw)
    ref = x_d.clone()
    assert plan.graph_stats() == (0, 0)

    n_blocks = T * (-(-L // Bj))
    for r in range(4):
        plan.set_graphs(True)
        x_g.fill_(float("nan"))
        c0, r0 = plan.graph_stats()
        it_g = _inverse(B, plan, z, Bj, x_g, ws, **kw)
        c1, r1 = plan.graph_stats()
        print(f"round {r}: iters {it_g.tolist()} captures {c1} replays {r1}")
        assert np.array_equal(it_g, it_d), f"round {r}"
        assert torch.equal(x_g, ref), f"round {r}: max |diff| {(x_g - ref).abs().max().item()}"
        assert c1 == n_blocks                       # captured on the first call only
        assert r1 - r0 == int(it_d.sum())           # one replay per update
        # direct-launch work between the replays: torch ops, a forward pass and
        # a direct inverse into another buffer, each synchronised
        plan.set_graphs(False)
        zf, _ = plan.forward(ref)
        torch.cuda.synchronize()
        y = torch.empty_like(z)
        it_y = _inverse(B, plan, (z * 1.0).contiguous(), Bj, y, ws, **kw)
        assert np.array_equal(it_y, it_d) and torch.equal(y, ref)
        assert torch.isfinite(zf).all()


def test_profiled_calls_launch_directly(B):
    """While a kernel class is profiled, updates are launched directly (the
    runtime gives no timing for events recorded inside a graph): no captures
    or replays, the same launch count and the same result as a graph call."""
    say("profiled call without graphs")
    cfg, params, _ = problem(C=48, d=256, H=4, layers=2, max_len=300, dtype="bf16", seed=50)
    plan = B.AFPlan(cfg, params)
    z = to_dev(synth.normal((2, 300, 48), 51))
    ws = plan.workspace(2, 128)
    x_g = torch.empty_like(z)
    plan.set_graphs(True)
    it_g = _inverse(B, plan, z, 128, x_g, ws)
    stats = plan.graph_stats()
    assert stats[0] == 3 and stats[1] == int(it_g.sum())
    counts = []
    for graphs in (False, True):
        plan.set_graphs(graphs)
        plan.profile_enable("gemm_qkv")
        x = torch.empty_like(z)
        it = _inverse(B, plan, z, 128, x, ws)
        n, ms = plan.profile_read()
        plan.profile_disable()
        print("graphs", graphs, "launches", n, "ms", ms, "iters", it.tolist())
        assert plan.graph_stats() == stats
        assert np.array_equal(it, it_g) and torch.equal(x, x_g)
        assert n >= 2 * int(it.sum()) and ms > 0      # two layers: a QKV launch each
        counts.append(n)
    assert counts[0] == counts[1]
