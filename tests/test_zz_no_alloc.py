"""afk_affine_noalloc (scratch in the library's static device array) against
afk_affine (scratch in a caller buffer) through the C ABI: identical x / z and
residual sums, bit for bit (the same kernel and reduction order), on two calls
in a row, the second with a smaller input, in both modes; a request larger
than the static scratch is refused.

Method: STARFlow-V notes (papernotes.org), 关键设计 1 (affine update) and
关键设计 3 (Jacobi residual)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from parity_util import say  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from autoregressive_normalizing_flow_amd import binding
    binding.load_library()
    return binding


def _case(N, rows, C, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    head = torch.randn(N * rows, 2 * C, generator=g).cuda()
    src = torch.randn(N, rows, C, generator=g).cuda()
    old = torch.randn(N, rows, C, generator=g).cuda()
    return head, src, old


@pytest.mark.parametrize("mode", [0, 1], ids=["inverse", "forward"])
def test_noalloc_matches_workspace_call(B, mode):
    for N, rows, C, seed in ((3, 777, 48, 1), (2, 130, 16, 2)):   # second call smaller
        say("affine noalloc", mode, N, rows, C)
        head, src, old = _case(N, rows, C, seed)
        part = torch.empty(B.afk_affine_partials_bytes(N, rows, C), dtype=torch.uint8,
                           device="cuda")
        res_a = torch.full((N, 2), float("nan"), device="cuda")
        res_b = torch.full((N, 2), float("nan"), device="cuda")
        if mode == 0:   # x updated in place: both start from the same x_old
            xa, xb = old.clone(), old.clone()
            B.afk_affine(0, head, src, xa, N, rows, C, res_a, part)
            B.afk_affine_noalloc(0, head, src, xb, N, rows, C, res_b)
        else:           # z written from x = src
            xa, xb = torch.empty_like(src), torch.empty_like(src)
            B.afk_affine(1, head, src, xa, N, rows, C, res_a, part)
            B.afk_affine_noalloc(1, head, src, xb, N, rows, C, res_b)
        torch.cuda.synchronize()
        assert torch.equal(xa, xb)
        assert torch.equal(res_a, res_b)
        assert torch.isfinite(res_b).all()


def test_noalloc_refuses_more_than_its_scratch(B):
    say("affine noalloc limit")
    N, rows, C = 40000, 1, 4   # 40000 partial pairs: above 256 KiB
    head = torch.zeros(N * rows, 2 * C, device="cuda")
    src = torch.zeros(N, rows, C, device="cuda")
    dst = torch.zeros_like(src)
    res = torch.zeros(N, 2, device="cuda")
    assert B.afk_affine_partials_bytes(N, rows, C) > 256 * 1024
    with pytest.raises(B.AFError) as ei:
        B.afk_affine_noalloc(0, head, src, dst, N, rows, C, res)
    assert ei.value.status == B.AF_ERR_WORKSPACE
