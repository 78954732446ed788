"""q4_gemv_noalloc through the C ABI against q4_gemv with a caller's
workspace: the same kernels and plan, so the outputs must be identical bit for
bit.  Two calls in a row on the library's shared scratch array, the second on
a smaller problem, then a shape that needs no scratch at all."""
import pytest
import torch

from bit_quantized_matmul_q4_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _case(q4, seed, M, N, K):
    W, x = wl.gemv_case(seed, M, N, K)
    qs, sm = q4.q4_pack(W.cuda())
    return x.cuda(), qs, sm


def _reference(q4, x, qs, sm):
    M, N = x.shape[0], qs.shape[0]
    need = q4.q4_gemv_workspace_bytes(M, N, x.shape[1])
    # a workspace that starts with garbage, like the scratch array would
    ws = torch.full((max(need, 1),), 0x7F, dtype=torch.uint8, device="cuda")
    return q4.q4_gemv(x, qs, sm, workspace=ws)


def test_gemv_noalloc_matches_q4_gemv(q4):
    cases = [(81, 8, 1000, 4096), (82, 5, 300, 2560), (83, 1, 4096, 4096)]
    for i, (seed, M, N, K) in enumerate(cases):
        need = q4.q4_gemv_workspace_bytes(M, N, K)
        print("noalloc call %d: M=%d N=%d K=%d scratch bytes %d" % (i, M, N, K, need), flush=True)
        assert need <= q4.NOALLOC_SCRATCH_BYTES
        if i < 2:
            assert need > 0  # these two use the scratch array (K split)
        x, qs, sm = _case(q4, seed, M, N, K)
        y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        q4.q4_gemv_noalloc(x, qs, sm, y)
        ref = _reference(q4, x, qs, sm)
        torch.cuda.synchronize()
        assert torch.equal(y, ref), "call %d differs from q4_gemv" % i
    # the first shape again after the smaller one: the array keeps the last
    # call's contents, which must not matter
    x, qs, sm = _case(q4, 81, 8, 1000, 4096)
    y = torch.empty((8, 1000), dtype=torch.float32, device="cuda")
    q4.q4_gemv_noalloc(x, qs, sm, y)
    assert torch.equal(y, _reference(q4, x, qs, sm))


def test_gemv_noalloc_refuses_shapes_beyond_the_scratch(q4):
    # 16 rows x 151936 x 65536 would need 16 K splits of partials (155 MB)
    M, N, K = 16, 151936, 65536
    assert q4.q4_gemv_workspace_bytes(M, N, K) > q4.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M, K), dtype=torch.float32, device="cuda")
    qs = torch.zeros((N, K // 2), dtype=torch.uint8, device="cuda")
    sm = torch.zeros((N, K // 256, 2), dtype=torch.float16, device="cuda")
    y = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    with pytest.raises(q4.Q4Error) as e:
        q4.q4_gemv_noalloc(x, qs, sm, y)
    assert e.value.code == -3
