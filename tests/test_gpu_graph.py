"""The library's calls inside a captured HIP graph.

Every kernel family is captured once (Q8_1 quantize, MMQ with a K split and
its sum pass, MMQ producing Q8_1, the one- and two-row VALU GEMV, the
matrix-core GEMV with a K split and its sum pass) and the graph is replayed
three times with new inputs written eagerly in place between replays; every
replay must equal the eager calls on the same inputs bit for bit (all kernels
have fixed reduction orders).  The library allocates and synchronises nothing,
so capture needs only the caller's preallocated outputs and workspaces.
"""
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager(q4):
    dev = torch.device("cuda")
    g = torch.Generator(device="cuda").manual_seed(41)

    def w(n, k):
        return (0.02 * torch.randn((n, k), generator=g, device=dev)).contiguous()

    qs1, sm1 = q4.q4_pack(w(6144, 2560))
    qs2, sm2 = q4.q4_pack(w(512, 4096))
    qs3, sm3 = q4.q4_pack(w(224, 2048))
    xa = torch.empty((100, 2048), device=dev)
    x1 = torch.empty((1, 2560), device=dev)
    x2 = torch.empty((2, 2560), device=dev)
    x8 = torch.empty((8, 4096), device=dev)
    qa = torch.empty((100, 2048), dtype=torch.int8, device=dev)
    ds = torch.empty((100, 64, 2), dtype=torch.float16, device=dev)
    ym = torch.empty((100, 224), device=dev)
    qo = torch.empty((100, 224), dtype=torch.int8, device=dev)
    dso = torch.empty((100, 7, 2), dtype=torch.float16, device=dev)
    y1 = torch.empty((1, 6144), device=dev)
    y2 = torch.empty((2, 6144), device=dev)
    y8 = torch.empty((8, 512), device=dev)
    ws_m = torch.empty((max(q4.q4_mmq_workspace_bytes(100, 224, 2048), 1),), dtype=torch.uint8, device=dev)
    ws_8 = torch.empty((max(q4.q4_gemv_workspace_bytes(8, 512, 4096), 1),), dtype=torch.uint8, device=dev)
    # the shapes take the K-split paths (partials and a second, summing kernel)
    assert q4.q4_mmq_workspace_bytes(100, 224, 2048) > 0
    assert q4.q4_gemv_workspace_bytes(8, 512, 4096) > 0

    def inputs():
        for t in (xa, x1, x2, x8):
            t.copy_(torch.randn(t.shape, generator=g, device=dev))

    def run():
        q4.q8_1_quantize(xa, qa, ds)
        q4.q4_mmq_gemm(qa, ds, qs3, sm3, y=ym, workspace=ws_m)
        q4.q4_mmq_gemm_q8_1(qa, ds, qs3, sm3, qa_out=qo, ds_out=dso, workspace=ws_m)
        q4.q4_gemv(x1, qs1, sm1, y=y1)
        q4.q4_gemv(x2, qs1, sm1, y=y2)
        q4.q4_gemv(x8, qs2, sm2, y=y8, workspace=ws_8)

    outs = (qa, ds, ym, qo, dso, y1, y2, y8)
    inputs()
    run()  # warm: per-device state is set up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        inputs()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outs]
        run()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(got, outs)):
            assert torch.equal(a.view(torch.uint8) if a.dtype == torch.float16 else a,
                               b.view(torch.uint8) if b.dtype == torch.float16 else b), (rep, i)
