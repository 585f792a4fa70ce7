"""The Python binding refuses tensors a plan cannot use, before any launch:
host tensors, non-contiguous ones, and ones shorter than the description
(including batch strides) implies.  Raw integer addresses pass through, as
the C header documents."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tcg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import tensor_core_gemm_amd as t
    t.check_runtime()
    return t


def test_short_strided_and_host_tensors_are_refused(tcg):
    M, N, K = 256, 136, 96
    g = torch.Generator(device="cpu").manual_seed(3)
    A = torch.randn(M, K, generator=g).to(torch.bfloat16).cuda()
    B = torch.randn(K, N, generator=g).to(torch.bfloat16).cuda()
    C = torch.zeros(M, N, dtype=torch.bfloat16, device="cuda")
    p = tcg.gemm_plan(tcg.make_desc(M, N, K, tcg.BF16, tcg.BF16, tcg.EPI_RELU))
    with pytest.raises(ValueError, match="A holds"):
        tcg.gemm_run(p, A.view(-1)[:M * K - 1], B, C)
    with pytest.raises(ValueError, match="C holds"):
        tcg.gemm_run(p, A, B, C.view(-1)[:M * N - 1])
    with pytest.raises(ValueError, match="not contiguous"):
        tcg.gemm_run(p, A, B.t().contiguous().t(), C)
    with pytest.raises(ValueError, match="not a GPU tensor"):
        tcg.gemm_run(p, A.cpu(), B, C)
    pb = tcg.gemm_plan(tcg.make_desc(M, N, K, tcg.BF16, tcg.BF16, tcg.EPI_RELU, tcg.FLAG_BIAS))
    with pytest.raises(ValueError, match="bias holds"):
        tcg.gemm_run_ex(pb, A, B, C, bias=torch.zeros(N - 1, device="cuda"))
    torch.cuda.synchronize()
    assert not torch.any(C != 0)  # nothing was launched
    tcg.gemm_run(p, A, B, C)
    torch.cuda.synchronize()
    ref = torch.relu(A.float() @ B.float())
    assert torch.allclose(C.float(), ref, rtol=1e-2, atol=1e-2)


def test_batched_extent_is_checked(tcg):
    M, N, K, batch = 64, 72, 40, 3
    sa, sb, sc = M * K + 8, K * N + 16, M * N + 24
    ext_a, ext_b, ext_c = (batch - 1) * sa + M * K, (batch - 1) * sb + K * N, (batch - 1) * sc + M * N
    d = tcg.make_desc(M, N, K, tcg.F16, tcg.F32, tcg.EPI_NONE, 0, batch, sa, sb, sc)
    p = tcg.gemm_plan(d)
    A = torch.randn(ext_a, device="cuda").to(torch.float16)
    B = torch.randn(ext_b, device="cuda").to(torch.float16)
    C = torch.zeros(ext_c, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="A holds"):
        tcg.gemm_run(p, A[:-1], B, C)
    with pytest.raises(ValueError, match="C holds"):
        tcg.gemm_run(p, A, B, C[:-1])
    tcg.gemm_run(p, A, B, C)  # exactly the extent: accepted
    torch.cuda.synchronize()
    for b in range(batch):
        a = A[b * sa:b * sa + M * K].view(M, K).float()
        bb = B[b * sb:b * sb + K * N].view(K, N).float()
        assert torch.allclose(C[b * sc:b * sc + M * N].view(M, N), a @ bb, rtol=1e-4, atol=1e-3)
        if b + 1 < batch:
            assert not torch.any(C[b * sc + M * N:(b + 1) * sc] != 0)  # gaps untouched
