"""MMQ on operands beyond the 2 GiB reach of one buffer descriptor.

Every MMQ launcher addresses its operands through descriptors with 32-bit
offsets, so a call whose packed weights pass 2 GiB runs as several row
ranges of the weights, each with its own launch, and one whose activations
pass it as several row ranges of the activations.  1048576 x 4096 weights
hold exactly 2 GiB of codes: the fp16 design and the unpipelined integer
kernel cut them into 1048448 rows and a 128-row tail.  600000 x 4096 Q8_1
activations run in 32768-row chunks (the fp16 design's activation image) or
524160-row ranges (the integer kernel).  These tests check, against the CPU
oracle, the outputs on both sides of each cut and at the ends (a sample of
weight rows and activation rows; the oracle takes the sampled rows as a
smaller problem of its own, since packing and Q8_1 are per row), and that
the Q8_1-output route is the fp32 route quantized bit for bit across the
weight cut.
"""
import numpy as np
import pytest
import torch

from bit_quantized_matmul_q4_amd import workloads as wl
from test_gpu_parity import close, say

pytestmark = pytest.mark.gpu

N_BIG, K_BIG, M_BIG = 1048576, 4096, 256
CUT = 1048448  # rows of the first range: 2^31 - 1 bytes of codes, whole 128-row tiles


def sampled_weight_rows():
    edges = [0, 1, CUT - 2, CUT - 1, CUT, CUT + 1, N_BIG - 2, N_BIG - 1]
    rng = np.random.default_rng(2048)
    return np.unique(np.concatenate([edges, rng.choice(N_BIG, 400, replace=False)]))


def sampled_act_rows():
    rng = np.random.default_rng(2049)
    return np.unique(np.concatenate([[0, M_BIG - 1], rng.choice(M_BIG, 30, replace=False)]))


@pytest.fixture(scope="module")
def big_case(q4, orc):
    # W drawn on the device (16 GiB of fp32), packed there both ways; the
    # oracle packs its own copy of the sampled rows
    g = torch.Generator(device="cuda").manual_seed(2047)
    W = torch.randn((N_BIG, K_BIG), generator=g, device="cuda", dtype=torch.float32).mul_(0.02)
    qs, sm = q4.q4_pack(W)
    qs32, sm32 = q4.q4_pack_g32(W)
    nrows = sampled_weight_rows()
    Wr = W.index_select(0, torch.from_numpy(nrows).cuda()).cpu().numpy()
    del W
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    x = wl.draw_activations(wl.generator(2050), M_BIG, K_BIG, True)
    qa, ds = q4.q8_1_quantize(x.cuda())
    mrows = sampled_act_rows()
    qa_h = qa.cpu().numpy()[mrows]
    ds_h = ds.cpu().view(torch.int16).numpy().view(np.uint16)[mrows]
    yield dict(qs=qs, sm=sm, qs32=qs32, sm32=sm32, qa=qa, ds=ds, nrows=nrows, mrows=mrows, Wr=Wr,
               qa_h=qa_h, ds_h=ds_h)
    del qs, sm, qs32, sm32
    torch.cuda.empty_cache()


def sampled(y, c):
    m = torch.from_numpy(c["mrows"]).cuda()
    n = torch.from_numpy(c["nrows"]).cuda()
    return y.index_select(0, m).index_select(1, n).cpu().numpy()


def test_mmq_beyond_2gib_of_weights(q4, orc, big_case):
    c = big_case
    qs_o, sm_o = orc.q4_pack(c["Wr"])
    ridx = torch.from_numpy(c["nrows"]).cuda()
    assert np.array_equal(c["qs"].index_select(0, ridx).cpu().numpy(), qs_o)
    assert np.array_equal(c["sm"].index_select(0, ridx).cpu().view(torch.int16).numpy().view(np.uint16), sm_o)
    ref = orc.q4_mmq(c["qa_h"], c["ds_h"], qs_o, sm_o, K_BIG)
    say("mmq beyond 2 GiB of weights, routed: M=%d N=%d K=%d (sampled rows)" % (M_BIG, N_BIG, K_BIG))
    y = q4.q4_mmq_gemm(c["qa"], c["ds"], c["qs"], c["sm"])
    close(sampled(y, c), ref, "mmq routed beyond 2 GiB")
    say("  Q8_1 output across the cut")
    qo, dso = q4.q4_mmq_gemm_q8_1(c["qa"], c["ds"], c["qs"], c["sm"])
    qe, dse = q4.q8_1_quantize(y)
    assert torch.equal(qo, qe)
    assert torch.equal(dso.view(torch.int16), dse.view(torch.int16))
    del y, qo, dso, qe, dse
    say("  integer design")
    yi = q4.q4_mmq_gemm_int8(c["qa"], c["ds"], c["qs"], c["sm"])
    close(sampled(yi, c), ref, "mmq int8 design beyond 2 GiB")
    del yi
    torch.cuda.empty_cache()


def test_mmq_g32_beyond_2gib_of_weights(q4, orc, big_case):
    c = big_case
    qs_o, sm_o = orc.q4_pack(c["Wr"], group=32)
    ridx = torch.from_numpy(c["nrows"]).cuda()
    assert np.array_equal(c["qs32"].index_select(0, ridx).cpu().numpy(), qs_o)
    assert np.array_equal(c["sm32"].index_select(0, ridx).cpu().view(torch.int16).numpy().view(np.uint16), sm_o)
    say("mmq g32 beyond 2 GiB of weights: M=%d N=%d K=%d (sampled rows)" % (M_BIG, N_BIG, K_BIG))
    y = q4.q4_mmq_gemm_g32(c["qa"], c["ds"], c["qs32"], c["sm32"])
    close(sampled(y, c), orc.q4_mmq(c["qa_h"], c["ds_h"], qs_o, sm_o, K_BIG, group=32),
          "mmq g32 beyond 2 GiB")
    del y
    torch.cuda.empty_cache()


def test_mmq_beyond_2gib_of_activations(q4, orc):
    # 600000 x 4096 Q8_1 activations (2.46 GB of codes): the fp16 design runs
    # them in chunks of 32768 rows (its 256 MiB activation image), the
    # unpipelined integer kernel in ranges of 524160 rows (2 GiB of codes)
    M, N, K = 600000, 128, 4096
    say("mmq beyond 2 GiB of activations: M=%d N=%d K=%d (sampled rows)" % (M, N, K))
    g = wl.generator(2051, "cuda")
    W = wl.draw_weights(g, N, K, "cuda")
    qs, sm = q4.q4_pack(W)
    x = wl.draw_activations(g, M, K, True, "cuda")
    qa, ds = q4.q8_1_quantize(x)
    del x
    torch.cuda.empty_cache()
    cuts = [32767, 32768, 524159, 524160]
    rows = np.unique(np.concatenate([[0, 1, M - 2, M - 1], cuts,
                                     np.random.default_rng(2052).choice(M, 60, replace=False)]))
    ridx = torch.from_numpy(rows).cuda()
    qa_h = qa.index_select(0, ridx).cpu().numpy()
    ds_h = ds.index_select(0, ridx).cpu().view(torch.int16).numpy().view(np.uint16)
    qs_o, sm_o = orc.q4_pack(W.cpu().numpy())
    assert np.array_equal(qs.cpu().numpy(), qs_o)
    assert np.array_equal(sm.cpu().view(torch.int16).numpy().view(np.uint16), sm_o)
    ref = orc.q4_mmq(qa_h, ds_h, qs_o, sm_o, K)
    y = q4.q4_mmq_gemm(qa, ds, qs, sm)
    close(y.index_select(0, ridx).cpu().numpy(), ref, "mmq routed beyond 2 GiB of activations")
    del y
    say("  integer design")
    yi = q4.q4_mmq_gemm_int8(qa, ds, qs, sm)
    close(yi.index_select(0, ridx).cpu().numpy(), ref, "mmq int8 design beyond 2 GiB of activations")
    del yi, qa, ds
    torch.cuda.empty_cache()
