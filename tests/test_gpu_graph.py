"""The library's calls inside a captured HIP graph.

Every kernel family is captured once (Q8_1 quantize, MMQ with a K split and
its sum pass, MMQ producing Q8_1, the one- and two-row VALU GEMV, the
matrix-core GEMV with a K split and its sum pass; the fp16 MMQ design with
its fused and its separate row-factor pass, fp32 and Q8_1 output; the int8
design through its own entry point; the group-32 GEMV on both arms and the
group-32 MMQ on both designs) and the graph is replayed three times with new
inputs written eagerly in place between replays; every replay must equal
the eager calls on the same inputs bit for bit (all kernels have fixed
reduction orders).  The library allocates and synchronises nothing, so
capture needs only the caller's preallocated outputs and workspaces.
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
    qs4, sm4 = q4.q4_pack(w(12288, 512))      # fp16 design, fused row factors
    qs5, sm5 = q4.q4_pack(w(9216, 4096))      # fp16 design, separate row-factor pass
    g1, gs1 = q4.q4_pack_g32(w(6144, 2560))
    g4, gs4 = q4.q4_pack_g32(w(12288, 512))
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
    xf = torch.empty((300, 512), device=dev)
    x8g = torch.empty((8, 2560), device=dev)
    xf5 = torch.empty((512, 4096), device=dev)
    qaf = torch.empty((300, 512), dtype=torch.int8, device=dev)
    dsf = torch.empty((300, 16, 2), dtype=torch.float16, device=dev)
    qaf5 = torch.empty((512, 4096), dtype=torch.int8, device=dev)
    dsf5 = torch.empty((512, 128, 2), dtype=torch.float16, device=dev)
    yf = torch.empty((300, 12288), device=dev)
    yf5 = torch.empty((512, 9216), device=dev)
    xi5 = torch.empty((1024, 4096), device=dev)
    qai5 = torch.empty((1024, 4096), dtype=torch.int8, device=dev)
    dsi5 = torch.empty((1024, 128, 2), dtype=torch.float16, device=dev)
    yi5 = torch.empty((1024, 9216), device=dev)
    qof = torch.empty((300, 12288), dtype=torch.int8, device=dev)
    dsof = torch.empty((300, 384, 2), dtype=torch.float16, device=dev)
    yg1 = torch.empty((1, 6144), device=dev)
    yg8 = torch.empty((8, 6144), device=dev)
    ygm = torch.empty((100, 224), device=dev)
    ygf = torch.empty((300, 12288), device=dev)
    qs3g, sm3g = q4.q4_pack_g32(w(224, 2048))
    ws_f = torch.empty((q4.q4_mmq_workspace_bytes(300, 12288, 512),), dtype=torch.uint8, device=dev)
    ws_f5 = torch.empty((q4.q4_mmq_workspace_bytes(512, 9216, 4096),), dtype=torch.uint8, device=dev)
    ws_i5 = torch.empty((max(q4.q4_mmq_int8_workspace_bytes(1024, 9216, 4096), 1),), dtype=torch.uint8, device=dev)
    ws_g8 = torch.empty((max(q4.q4_gemv_g32_workspace_bytes(8, 6144, 2560), 1),), dtype=torch.uint8, device=dev)
    # the fp16 design's workspace holds its activation image (2 K bytes per
    # row, rows padded to whole tiles, plus 4 bytes per row) and 8 bytes per
    # weight row, and covers the K-split partials of the Q8_1-output and
    # group-32 int8 kernels where those exceed it; q4_mmq_gemm_int8 has its
    # own (the per-row and per-weight-row records of its pipelined kernel,
    # which 576 tiles of 128 x 128 take)
    assert q4.q4_mmq_workspace_bytes(300, 12288, 512) == 384 * (2 * 512 + 4) + 12288 * 8  # two 192-row tiles
    assert q4.q4_mmq_workspace_bytes(512, 9216, 4096) == 576 * (2 * 4096 + 4) + 9216 * 8  # three 192-row tiles
    assert q4.q4_mmq_int8_workspace_bytes(1024, 9216, 4096) == 1024 * 16 * 32 + 9216 * 16 * 8
    # the shapes take the K-split paths (partials and a second, summing kernel)
    assert q4.q4_mmq_workspace_bytes(100, 224, 2048) > 0
    assert q4.q4_gemv_workspace_bytes(8, 512, 4096) > 0

    def inputs():
        for t in (xa, x1, x2, x8, x8g, xf, xf5, xi5):
            t.copy_(torch.randn(t.shape, generator=g, device=dev))

    def run():
        q4.q8_1_quantize(xa, qa, ds)
        q4.q4_mmq_gemm(qa, ds, qs3, sm3, y=ym, workspace=ws_m)
        q4.q4_mmq_gemm_q8_1(qa, ds, qs3, sm3, qa_out=qo, ds_out=dso, workspace=ws_m)
        q4.q4_gemv(x1, qs1, sm1, y=y1)
        q4.q4_gemv(x2, qs1, sm1, y=y2)
        q4.q4_gemv(x8, qs2, sm2, y=y8, workspace=ws_8)
        q4.q8_1_quantize(xf, qaf, dsf)
        q4.q4_mmq_gemm(qaf, dsf, qs4, sm4, y=yf, workspace=ws_f)
        q4.q4_mmq_gemm_q8_1(qaf, dsf, qs4, sm4, qa_out=qof, ds_out=dsof, workspace=ws_f)
        q4.q8_1_quantize(xf5, qaf5, dsf5)
        q4.q4_mmq_gemm(qaf5, dsf5, qs5, sm5, y=yf5, workspace=ws_f5)
        q4.q8_1_quantize(xi5, qai5, dsi5)
        q4.q4_mmq_gemm_int8(qai5, dsi5, qs5, sm5, y=yi5, workspace=ws_i5)
        q4.q4_gemv_g32(x1, g1, gs1, y=yg1)
        q4.q4_gemv_g32(x8g, g1, gs1, y=yg8, workspace=ws_g8)
        q4.q4_mmq_gemm_g32(qa, ds, qs3g, sm3g, y=ygm, workspace=ws_m)
        q4.q4_mmq_gemm_g32(qaf, dsf, g4, gs4, y=ygf, workspace=ws_f)

    outs = (qa, ds, ym, qo, dso, y1, y2, y8, qaf, dsf, yf, qof, dsof, qaf5, dsf5, yf5, qai5, dsi5, yi5, yg1, yg8, ygm, ygf)
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
