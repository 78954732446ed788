"""GPU parity of the group-32 variant (one fp16 scale/minimum pair per 32
weights) against the CPU oracle: packing bit-exact, GEMV and MMQ within the
fp32 tolerance.  Same seeded inputs as the group-256 tests."""
import numpy as np
import pytest
import torch

from bit_quantized_matmul_q4_amd import workloads as wl
from test_gpu_parity import MAX_NMSE, MAX_REL, close, dev, f16_workspace, say  # noqa: F401

pytestmark = pytest.mark.gpu

G32 = 32


def pack_g32_check(q4, orc, W, what):
    qs_o, sm_o = orc.q4_pack(W.numpy(), group=G32)
    qs_g, sm_g = q4.q4_pack_g32(dev(W))
    torch.cuda.synchronize()
    qg = qs_g.cpu().numpy()
    sg = sm_g.cpu().view(torch.int16).numpy().view(np.uint16)
    assert sg.shape == sm_o.shape
    bad = np.flatnonzero(qg.reshape(-1) != qs_o.reshape(-1))
    assert bad.size == 0, "%s: %d qs bytes differ, first at %s" % (what, bad.size, bad[:5])
    bad = np.flatnonzero(sg.reshape(-1) != sm_o.reshape(-1))
    assert bad.size == 0, "%s: %d sm entries differ, first at %s" % (what, bad.size, bad[:5])
    return qs_g, sm_g, qs_o, sm_o


@pytest.mark.parametrize("N,K", [(1, 256), (3, 512), (129, 768), (1000, 2560), (257, 9216)])
def test_pack_g32_bitexact(q4, orc, N, K):
    say("pack g32 N=%d K=%d" % (N, K))
    W, _ = wl.small_case(N, 1, N, K)
    pack_g32_check(q4, orc, W, "pack g32 %dx%d" % (N, K))


def test_pack_g32_edge_values(q4, orc):
    say("pack g32 edge values")
    rng = np.random.default_rng(31)
    W = (rng.standard_normal((8, 512)) * 0.02).astype(np.float32)
    W[0, :32] = 0.25                                      # constant run: scale 0
    W[1, 32:64] = 0.0
    W[1, 33:64:2] = -0.0                                  # zeros of both signs
    W[2, 64:96] = rng.standard_normal(32) * 1e-7          # scale in fp16 subnormals
    W[3, :32] = np.where(np.arange(32) % 2, 3.0, -2.0)    # two values: codes 0/15
    W[4] = np.linspace(-1, 1, 512)                        # many exact ties
    W[5, :32] = 60000.0 * np.sign(rng.standard_normal(32))
    pack_g32_check(q4, orc, torch.from_numpy(W), "pack g32 edges")


def gemv_g32_check(q4, orc, M, N, K, seed, what, rows=None):
    W, x = wl.gemv_case(seed, M, N, K)
    qs, sm = q4.q4_pack_g32(dev(W))
    y = q4.q4_gemv_g32(dev(x), qs, sm)
    torch.cuda.synchronize()
    qs_h = qs.cpu().numpy()
    sm_h = sm.cpu().view(torch.int16).numpy().view(np.uint16)
    yh = y.cpu().numpy()
    if rows is None:
        ref = orc.q4_gemv(x.numpy(), qs_h, sm_h, K, group=G32)
        close(yh, ref, what)
    else:
        qs_o, sm_o = orc.q4_pack(W.numpy()[rows], group=G32)
        assert np.array_equal(qs_o, qs_h[rows]) and np.array_equal(sm_o, sm_h[rows])
        ref = orc.q4_gemv(x.numpy(), qs_o, sm_o, K, group=G32)
        close(yh[:, rows], ref, what)
    return y


@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (1, 300, 768), (2, 129, 2560), (3, 77, 4096),
                                   (1, 1000, 9216), (2, 513, 12288), (5, 64, 2560), (16, 260, 1024),
                                   (8, 40, 256 * 17), (16, 1000, 3584)])
def test_gemv_g32_parity(q4, orc, M, N, K):
    say("gemv g32 M=%d N=%d K=%d" % (M, N, K))
    gemv_g32_check(q4, orc, M, N, K, N + K + 1, "gemv g32 %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("idx", range(len(wl.DECODE_PROJECTIONS)))
def test_gemv_g32_decode_projection(q4, orc, idx):
    name, K, N = wl.DECODE_PROJECTIONS[idx]
    say("gemv g32 decode %s K=%d N=%d" % (name, K, N))
    gemv_g32_check(q4, orc, 1, N, K, idx, "g32 decode " + name)


@pytest.mark.parametrize("M", [2, 16])
def test_gemv_g32_tiny_m(q4, orc, M):
    c = wl.TINY_M
    say("gemv g32 tiny-M M=%d (sampled rows)" % M)
    rows = np.sort(np.random.default_rng(M + 100).choice(c["N"], size=2048, replace=False))
    rows = np.unique(np.concatenate([[0, c["N"] - 1], rows]))
    gemv_g32_check(q4, orc, M, c["N"], c["K"], c["seed"], "g32 tiny-M %d" % M, rows=rows)


def test_gemv_g32_long_k(q4, orc):
    # M = 1 beyond one workgroup's LDS: the matrix-core arm with a K split
    K = 65792
    for M in (1, 2):
        say("gemv g32 M=%d N=100 K=%d" % (M, K))
        gemv_g32_check(q4, orc, M, 100, K, 90 + M, "g32 long K M=%d" % M)


def test_gemv_g32_equal_pairs_match_g256(q4, orc):
    # group-32 pairs that repeat over each run of 256 give the group-256 product
    say("gemv g32 with repeated pairs vs g256")
    W, x = wl.gemv_case(8, 3, 500, 2560)
    qs, sm = q4.q4_pack(dev(W))
    sm32 = sm.repeat_interleave(8, dim=1).contiguous()
    y32 = q4.q4_gemv_g32(dev(x), qs, sm32).cpu().numpy()
    y256 = q4.q4_gemv(dev(x), qs, sm).cpu().numpy()
    close(y32, y256, "g32 repeated vs g256")


def mmq_g32_check(q4, orc, M, N, K, seed, outliers, what, mrows=None):
    W, x = wl.mmq_case(seed, M, N, K, outliers)
    qs, sm = q4.q4_pack_g32(dev(W))
    qa, ds = q4.q8_1_quantize(dev(x))
    y = q4.q4_mmq_gemm_g32(qa, ds, qs, sm)
    torch.cuda.synchronize()
    qs_h = qs.cpu().numpy()
    sm_h = sm.cpu().view(torch.int16).numpy().view(np.uint16)
    qa_h = qa.cpu().numpy()
    ds_h = ds.cpu().view(torch.int16).numpy().view(np.uint16)
    yh = y.cpu().numpy()
    sel = slice(None) if mrows is None else mrows
    ref = orc.q4_mmq(qa_h[sel], ds_h[sel], qs_h, sm_h, K, group=G32)
    close(yh[sel], ref, what)


@pytest.mark.parametrize("M,N,K,outl", [(1, 1, 256, False), (130, 129, 768, True),
                                        (128, 128, 2560, False), (257, 385, 1024, True),
                                        (100, 200, 2048, True), (64, 1000, 4096, False)])
def test_mmq_g32_parity(q4, orc, M, N, K, outl):
    say("mmq g32 M=%d N=%d K=%d outliers=%s" % (M, N, K, outl))
    mmq_g32_check(q4, orc, M, N, K, M + N + 3, outl, "mmq g32 %dx%dx%d" % (M, N, K))


def test_mmq_g32_512(q4, orc):
    c = wl.MMQ_512
    say("mmq g32 M=512 K=2560 N=9216 (every output)")
    mmq_g32_check(q4, orc, c["M"], c["N"], c["K"], c["seed"], c["outliers"], "mmq g32 512")


@pytest.mark.parametrize("idx", [0, 1])
def test_mmq_g32_2048(q4, orc, idx):
    c = wl.MMQ_2048[idx]
    say("mmq g32 M=2048 %s (every output)" % c["name"])
    mmq_g32_check(q4, orc, c["M"], c["N"], c["K"], c["seed"], c["outliers"], "mmq g32 2048 " + c["name"])


def test_mmq_g32_equal_pairs_match_g256(q4, orc):
    say("mmq g32 with repeated pairs vs g256")
    W, x = wl.mmq_case(12, 300, 700, 2560, True)
    qs, sm = q4.q4_pack(dev(W))
    qa, ds = q4.q8_1_quantize(dev(x))
    sm32 = sm.repeat_interleave(8, dim=1).contiguous()
    close(q4.q4_mmq_gemm_g32(qa, ds, qs, sm32).cpu().numpy(), q4.q4_mmq_gemm(qa, ds, qs, sm).cpu().numpy(),
          "mmq g32 repeated vs g256")


# Shapes whose grid fills the GPU run on the fp16 matrix-core design, where
# each lane's (scale, minimum) pair changes every Q8_1 block.

def test_mmq_g32_f16_ragged(q4, orc):
    M, N, K = 300, 12700, 512
    say("mmq g32, fp16 design, M=%d N=%d K=%d" % (M, N, K))
    assert q4.q4_mmq_workspace_bytes(M, N, K) == f16_workspace(M, N, K)  # two tiles of 192 rows
    mmq_g32_check(q4, orc, M, N, K, 74, True, "mmq g32 fp16 ragged")


def test_mmq_g32_f16_equal_pairs_match_g256(q4, orc):
    # the same pair in all eight blocks of each group: the operands are the
    # group-256 design's, bit for bit, and so is the result
    M, N, K = 300, 12288, 1024
    say("mmq g32 with repeated pairs vs g256, fp16 design, M=%d N=%d K=%d" % (M, N, K))
    W, x = wl.mmq_case(75, M, N, K, True)
    qs, sm = q4.q4_pack(dev(W))
    qa, ds = q4.q8_1_quantize(dev(x))
    sm32 = sm.repeat_interleave(8, dim=1).contiguous()
    assert torch.equal(q4.q4_mmq_gemm_g32(qa, ds, qs, sm32), q4.q4_mmq_gemm(qa, ds, qs, sm))
