"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bit-exact: packing, Q8_1 quantization, per-block int32 dots.
fp32 outputs: max|y - ref| / max|ref| <= 2e-3 and NMSE = sum (y - ref)^2 /
sum ref^2 <= 1e-6 against the oracle's fp64 sums.

Small cases span several tiles and ragged tails; full-size cases use the
workload shapes with the launch configuration the benchmark times, checking
every output the oracle can afford and a seeded sample of rows otherwise.
"""
import sys

import numpy as np
import pytest
import torch

from bit_quantized_matmul_q4_amd import workloads as wl

pytestmark = pytest.mark.gpu

MAX_REL = 2e-3
MAX_NMSE = 1e-6




def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(t):
    return t.contiguous().cuda()


def close(y, ref, what):
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = y - ref
    den = np.abs(ref).max()
    rel = np.abs(err).max() / den if den > 0 else np.abs(err).max()
    nmse = (err ** 2).sum() / max((ref ** 2).sum(), 1e-300)
    say("  %s: max_rel=%.3e nmse=%.3e" % (what, rel, nmse))
    assert np.all(np.isfinite(y)), what + ": non-finite output"
    assert rel <= MAX_REL, "%s: max rel %.3e" % (what, rel)
    assert nmse <= MAX_NMSE, "%s: nmse %.3e" % (what, nmse)


def pack_both(q4, orc, W):
    qs_o, sm_o = orc.q4_pack(W.numpy())
    qs_g, sm_g = q4.q4_pack(dev(W))
    torch.cuda.synchronize()
    return (qs_o, sm_o), (qs_g, sm_g)


def assert_pack_equal(qs_o, sm_o, qs_g, sm_g, what):
    qg = qs_g.cpu().numpy()
    sg = sm_g.cpu().view(torch.int16).numpy().view(np.uint16)
    bad = np.flatnonzero(qg.reshape(-1) != qs_o.reshape(-1))
    assert bad.size == 0, "%s: %d qs bytes differ, first at %s" % (what, bad.size, bad[:5])
    bad = np.flatnonzero(sg.reshape(-1) != sm_o.reshape(-1))
    assert bad.size == 0, "%s: %d sm entries differ, first at %s" % (what, bad.size, bad[:5])


# ------------------------------------------------------------------ pack ---

PACK_SHAPES = [(1, 256), (3, 512), (129, 768), (1000, 2560), (257, 9216)]


@pytest.mark.parametrize("N,K", PACK_SHAPES)
def test_pack_bitexact(q4, orc, N, K):
    say("pack N=%d K=%d seed=%d" % (N, K, N))
    W, _ = wl.small_case(N, 1, N, K)
    (qs_o, sm_o), (qs_g, sm_g) = pack_both(q4, orc, W)
    assert_pack_equal(qs_o, sm_o, qs_g, sm_g, "pack %dx%d" % (N, K))


def test_pack_edge_values(q4, orc):
    say("pack edge values")
    rng = np.random.default_rng(21)
    W = (rng.standard_normal((12, 512)) * 0.02).astype(np.float32)
    W[0, :256] = 0.25                                     # constant group: scale 0
    W[1, :256] = 0.0
    W[1, ::2] = -0.0                                      # zeros of both signs
    W[2, :256] = rng.standard_normal(256) * 1e-7          # scale in fp16 subnormals
    W[3, :256] = rng.standard_normal(256) * 1e-39         # fp32 subnormal weights
    W[4, :256] = np.where(np.arange(256) % 2, 3.0, -2.0)  # two values: codes 0/15
    W[5, :256] = 1000.0 + rng.standard_normal(256)        # large offset, small range
    W[6] = np.linspace(-1, 1, 512)                        # many exact ties
    W[7, :256] = (np.arange(256) % 16) * 0.0625 + 0.5 * 0.0625  # half-way codes
    W[8, :256] = 60000.0 * np.sign(rng.standard_normal(256))     # near fp16 max
    t = torch.from_numpy(W)
    (qs_o, sm_o), (qs_g, sm_g) = pack_both(q4, orc, t)
    assert_pack_equal(qs_o, sm_o, qs_g, sm_g, "pack edges")


def test_pack_lm_head_full(q4, orc):
    K, N = 2560, 151936
    say("pack full lm_head N=%d K=%d seed=7" % (N, K))
    W, _ = wl.gemv_case(7, 1, N, K)
    (qs_o, sm_o), (qs_g, sm_g) = pack_both(q4, orc, W)
    assert_pack_equal(qs_o, sm_o, qs_g, sm_g, "pack lm_head")


# ------------------------------------------------------------------ Q8_1 ---

@pytest.mark.parametrize("M,K,outl", [(1, 32, False), (5, 256, False), (64, 2560, True),
                                      (2048, 12288, True)])
def test_q8_1_bitexact(q4, orc, M, K, outl):
    say("q8_1 M=%d K=%d outliers=%s" % (M, K, outl))
    g = wl.generator(M + K)
    x = wl.draw_activations(g, M, K, outl)
    qa_o, ds_o = orc.q8_1_quantize(x.numpy())
    qa_g, ds_g = q4.q8_1_quantize(dev(x))
    torch.cuda.synchronize()
    assert np.array_equal(qa_g.cpu().numpy(), qa_o)
    assert np.array_equal(ds_g.cpu().view(torch.int16).numpy().view(np.uint16), ds_o)


def test_q8_1_beyond_one_descriptor(q4, orc):
    # 8200 x 65536 activations (2.15 GB of fp32, past 2^31 bytes): the
    # quantizer indexes with 64 bits in one launch; rows on both sides of the
    # 2 GiB mark (inside row 8191) and the last row are checked bit for bit
    M, K = 8200, 65536
    say("q8_1 M=%d K=%d (past 2 GiB of input)" % (M, K))
    g = torch.Generator(device="cuda").manual_seed(31)
    x = torch.randn((M, K), generator=g, device="cuda", dtype=torch.float32)
    qa_g, ds_g = q4.q8_1_quantize(x)
    torch.cuda.synchronize()
    for r0, r1 in ((0, 1), (8190, 8193), (M - 1, M)):
        qa_o, ds_o = orc.q8_1_quantize(x[r0:r1].cpu().numpy())
        assert np.array_equal(qa_g[r0:r1].cpu().numpy(), qa_o), (r0, r1)
        assert np.array_equal(ds_g[r0:r1].cpu().view(torch.int16).numpy().view(np.uint16), ds_o), (r0, r1)
    del x, qa_g, ds_g


def test_q8_1_edge_values(q4, orc):
    say("q8_1 edge values")
    rng = np.random.default_rng(22)
    x = rng.standard_normal((6, 256)).astype(np.float32)
    x[0, :32] = 0.0                      # zero block
    x[0, 32:64] = -0.0
    x[1, :32] = 1e-30                    # d underflows to 0 in fp16
    x[2, :32] = rng.standard_normal(32) * 1e-6   # fp16-subnormal d
    x[3, :32] = np.arange(32) * 0.0625 - 1.03125  # ties
    x[4, :32] = 2000.0 * np.sign(rng.standard_normal(32))
    gold = [7.9375, -7.9375, 0.15625, 0.21875, -0.15625, 0.03125, -0.03125, 7.90625]
    x[5, :8] = gold
    qa_o, ds_o = orc.q8_1_quantize(x)
    qa_g, ds_g = q4.q8_1_quantize(dev(torch.from_numpy(x)))
    torch.cuda.synchronize()
    assert np.array_equal(qa_g.cpu().numpy(), qa_o)
    assert np.array_equal(ds_g.cpu().view(torch.int16).numpy().view(np.uint16), ds_o)


def test_q8_1_near_ties(q4, orc):
    # quotients x / d at, and a few fp32 ulps around, half-integers, with
    # power-of-two and general fp16 block scales from 2^-30 to 2^9 (the first
    # value of each block, 127 d, sets d): the device takes x times a
    # reciprocal of d and divides exactly only near half-integers
    say("q8_1 near ties")
    rng = np.random.default_rng(23)
    M, K = 96, 1024
    nb = K // 32
    k = rng.integers(-127, 127, (M, K)).astype(np.float64)
    e = rng.integers(-30, 10, (M, nb, 1))
    d = np.broadcast_to(np.ldexp(1.0, e), (M, nb, 32)).reshape(M, K).copy()
    d[M // 2:] *= 1.0 + rng.integers(1, 1024, (M - M // 2, 1)) / 1024.0
    off = rng.choice([0.5, 0.5 + 2.0 ** -18, 0.5 - 2.0 ** -18, 0.5 + 2.0 ** -12, 0.25], (M, K))
    x = (k + off) * d
    x.reshape(M, nb, 32)[:, :, 0] = 127.0 * d.reshape(M, nb, 32)[:, :, 0]
    x = x.astype(np.float32)
    qa_o, ds_o = orc.q8_1_quantize(x)
    qa_g, ds_g = q4.q8_1_quantize(dev(torch.from_numpy(x)))
    torch.cuda.synchronize()
    assert np.array_equal(qa_g.cpu().numpy(), qa_o)
    assert np.array_equal(ds_g.cpu().view(torch.int16).numpy().view(np.uint16), ds_o)


# ------------------------------------------------------------ block dots ---

@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (32, 32, 256), (130, 200, 512), (257, 129, 768),
                                   (64, 300, 2560)])
def test_block_dots_bitexact(q4, orc, M, N, K):
    say("block_dots M=%d N=%d K=%d" % (M, N, K))
    W, x = wl.small_case(M * 7 + N, M, N, K)
    qs_o, _ = orc.q4_pack(W.numpy())
    qa_o, _ = orc.q8_1_quantize(x.numpy())
    ref = orc.q4_block_dots(qa_o, qs_o, K)
    got = q4.q4_mmq_block_dots(dev(torch.from_numpy(qa_o)), dev(torch.from_numpy(qs_o)))
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    bad = np.argwhere(got != ref)
    assert bad.size == 0, "block dots differ at %s" % bad[:5]


def test_block_dots_extreme_codes(q4, orc):
    say("block_dots extreme codes")
    M, N, K = 40, 70, 512
    qa = np.full((M, K), 127, dtype=np.int8)
    qa[::2] = -127
    qa[5] = np.tile(np.arange(-16, 16, dtype=np.int8), K // 32)
    W = np.full((N, K), 1.0, dtype=np.float32)
    W[:, ::256] = 0.0                     # codes: mostly 15, a 0 per group
    W[3] = np.tile(np.arange(16, dtype=np.float32), K // 16)
    qs, _ = orc.q4_pack(W)
    ref = orc.q4_block_dots(qa, qs, K)
    got = q4.q4_mmq_block_dots(dev(torch.from_numpy(qa)), dev(torch.from_numpy(qs)))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), ref)
    assert np.abs(ref).max() >= 127 * 15 * 31


# ------------------------------------------------------------------ GEMV ---

def gemv_case_check(q4, orc, M, N, K, seed, what, rows=None):
    W, x = wl.gemv_case(seed, M, N, K)
    qs, sm = q4.q4_pack(dev(W))
    y = q4.q4_gemv(dev(x), qs, sm)
    torch.cuda.synchronize()
    qs_h = qs.cpu().numpy()
    sm_h = sm.cpu().view(torch.int16).numpy().view(np.uint16)
    yh = y.cpu().numpy()
    if rows is None:
        # the oracle packs W itself: the GPU's packing must agree before its
        # codes feed the oracle's product
        qs_o, sm_o = orc.q4_pack(W.numpy())
        assert_pack_equal(qs_o, sm_o, qs, sm, what)
        ref = orc.q4_gemv(x.numpy(), qs_o, sm_o, K)
        close(yh, ref, what)
    else:
        # the oracle packs its own copy of the sampled rows from W
        qs_o, sm_o = orc.q4_pack(W.numpy()[rows])
        assert np.array_equal(qs_o, qs_h[rows]) and np.array_equal(sm_o, sm_h[rows])
        ref = orc.q4_gemv(x.numpy(), qs_o, sm_o, K)
        close(yh[:, rows], ref, what)
    return y, qs, sm, x


@pytest.mark.parametrize("M,N,K", [(1, 1, 256), (1, 37, 512), (1, 300, 768), (2, 129, 2560),
                                   (3, 77, 4096), (4, 1000, 1280), (1, 1000, 9216),
                                   (2, 513, 12288), (5, 64, 2560), (16, 260, 1024),
                                   (1, 5, 256 * 17)])
def test_gemv_parity_small(q4, orc, M, N, K):
    say("gemv M=%d N=%d K=%d" % (M, N, K))
    gemv_case_check(q4, orc, M, N, K, N + K, "gemv %dx%dx%d" % (M, N, K))


# matrix-core arm with activation images of 4, 8 and 16 rows holding fewer
# rows than that (zero rows between M and the image, copies past it)
@pytest.mark.parametrize("M,N,K", [(3, 65536, 512), (6, 700, 2560), (7, 1000, 4096), (9, 300, 2560),
                                   (12, 513, 1280), (15, 700, 9216)])
def test_gemv_matrix_core_partial_images(q4, orc, M, N, K):
    say("gemv matrix-core arm M=%d N=%d K=%d" % (M, N, K))
    gemv_case_check(q4, orc, M, N, K, 7 * M + N, "gemv %dx%dx%d" % (M, N, K))


def test_gemv_single_4096(q4, orc):
    c = wl.SINGLE_GEMV
    say("gemv single 4096x4096 seed 0")
    gemv_case_check(q4, orc, c["M"], c["N"], c["K"], c["seed"], "gemv 4096^2")


@pytest.mark.parametrize("idx", range(len(wl.DECODE_PROJECTIONS)))
def test_gemv_decode_projection(q4, orc, idx):
    name, K, N = wl.DECODE_PROJECTIONS[idx]
    say("gemv decode %s K=%d N=%d seed=%d" % (name, K, N, idx))
    gemv_case_check(q4, orc, 1, N, K, idx, "decode " + name)


@pytest.mark.parametrize("M", wl.TINY_M["Ms"])
def test_gemv_tiny_m(q4, orc, M):
    c = wl.TINY_M
    say("gemv tiny-M M=%d N=%d K=%d (sampled rows)" % (M, c["N"], c["K"]))
    rows = np.sort(np.random.default_rng(M).choice(c["N"], size=4096, replace=False))
    rows = np.concatenate([[0, 1, c["N"] - 1], rows])
    gemv_case_check(q4, orc, M, c["N"], c["K"], c["seed"], "tiny-M %d" % M, rows=np.unique(rows))


def test_gemv_rows_match_single_row_calls(q4, orc):
    say("gemv batched rows vs one-row calls")
    W, x = wl.gemv_case(3, 4, 700, 2560)
    qs, sm = q4.q4_pack(dev(W))
    xd = dev(x)
    y = q4.q4_gemv(xd, qs, sm)
    for m in range(4):
        y1 = q4.q4_gemv(xd[m:m + 1].contiguous(), qs, sm)
        close(y1.cpu().numpy()[0], y[m].cpu().numpy(), "row %d" % m)


# (M, N, K, seed, VALU arm): up to 4 rows run the one-row arm when the image
# fits (K <= 31744 for 2 rows, 15360 for 4) and, for 3-4 rows, N < 65536; for
# 2 rows, N < 65536 or K > 4096
FEW_ROW_CASES = [(2, 700, 2560, 21, True), (2, 37984, 4096, 22, True), (2, 300, 31744, 23, True),
                 (2, 96, 32000, 24, False), (3, 700, 2560, 25, True), (4, 1000, 15360, 26, True),
                 (4, 300, 15616, 27, False), (4, 65535, 2560, 28, True), (4, 65536, 2560, 29, False),
                 (2, 65535, 4096, 30, True), (2, 65536, 4096, 31, False), (2, 65536, 4352, 32, True)]


@pytest.mark.parametrize("M,N,K,seed,valu", FEW_ROW_CASES)
def test_gemv_few_rows_match_single_row_calls(q4, orc, M, N, K, seed, valu):
    # On the VALU arm the rows share every widened weight pair and each row's
    # arithmetic is a one-row call's, so the results are identical; on the
    # matrix-core arm they agree to the fp32 tolerance.
    say("gemv M=%d vs one-row calls N=%d K=%d" % (M, N, K))
    W, x = wl.gemv_case(seed, M, N, K)
    qs, sm = q4.q4_pack(dev(W))
    xd = dev(x)
    y = q4.q4_gemv(xd, qs, sm)
    for m in range(M):
        y1 = q4.q4_gemv(xd[m:m + 1].contiguous(), qs, sm)
        if valu:
            assert torch.equal(y1[0], y[m]), "row %d" % m
        else:
            close(y1.cpu().numpy()[0], y[m].cpu().numpy(), "row %d" % m)
    if N <= 1000:
        ref = orc.q4_gemv(x.numpy(), qs.cpu().numpy(), sm.cpu().view(torch.int16).numpy().view(np.uint16), K)
        close(y.cpu().numpy(), ref, "gemv M=%d %dx%d" % (M, N, K))


def test_gemv_one_hot_and_deterministic(q4, orc):
    say("gemv one-hot x and rerun determinism")
    N, K = 333, 2560
    W, _ = wl.gemv_case(4, 1, N, K)
    qs, sm = q4.q4_pack(dev(W))
    ks = [0, 1, 16, 31, 255, 256, 1000, 2559]
    x = torch.zeros((len(ks), K), dtype=torch.float32)
    for i, k in enumerate(ks):
        x[i, k] = 1.0
    xs = dev(x)
    got = []
    for i in range(0, len(ks), 4):
        got.append(q4.q4_gemv(xs[i:i + 4].contiguous(), qs, sm).cpu().numpy())
    got = np.concatenate(got)
    Wd = orc.q4_dequant(qs.cpu().numpy(), sm.cpu().view(torch.int16).numpy().view(np.uint16), K)
    assert np.array_equal(got.astype(np.float64), Wd[:, ks].T), "one-hot x must return column k"
    a = q4.q4_gemv(xs[:4].contiguous(), qs, sm)
    b = q4.q4_gemv(xs[:4].contiguous(), qs, sm)
    assert torch.equal(a, b)


# ------------------------------------------------------------------- MMQ ---

def mmq_check(q4, orc, M, N, K, seed, outliers, what, mrows=None):
    W, x = wl.mmq_case(seed, M, N, K, outliers)
    qs, sm = q4.q4_pack(dev(W))
    qa, ds = q4.q8_1_quantize(dev(x))
    y = q4.q4_mmq_gemm(qa, ds, qs, sm)
    torch.cuda.synchronize()
    qs_h = qs.cpu().numpy()
    sm_h = sm.cpu().view(torch.int16).numpy().view(np.uint16)
    qa_h = qa.cpu().numpy()
    ds_h = ds.cpu().view(torch.int16).numpy().view(np.uint16)
    yh = y.cpu().numpy()
    if mrows is None:
        ref = orc.q4_mmq(qa_h, ds_h, qs_h, sm_h, K)
        close(yh, ref, what)
    else:
        ref = orc.q4_mmq(qa_h[mrows], ds_h[mrows], qs_h, sm_h, K)
        close(yh[mrows], ref, what)
    return y


@pytest.mark.parametrize("M,N,K,outl", [(1, 1, 256, False), (1, 300, 512, False),
                                        (130, 129, 768, True), (128, 128, 2560, False),
                                        (257, 385, 1024, True), (64, 1000, 4096, False)])
def test_mmq_parity_small(q4, orc, M, N, K, outl):
    say("mmq M=%d N=%d K=%d outliers=%s" % (M, N, K, outl))
    mmq_check(q4, orc, M, N, K, M + N, outl, "mmq %dx%dx%d" % (M, N, K))


def test_mmq_512_full(q4, orc):
    c = wl.MMQ_512
    say("mmq M=512 K=2560 N=9216 (every output)")
    mmq_check(q4, orc, c["M"], c["N"], c["K"], c["seed"], c["outliers"], "mmq 512")


@pytest.mark.parametrize("idx", [0, 1])
def test_mmq_2048_full(q4, orc, idx):
    # every output of the layer (the oracle needs a few seconds on 16 threads)
    c = wl.MMQ_2048[idx]
    say("mmq M=2048 %s K=%d N=%d (every output)" % (c["name"], c["K"], c["N"]))
    mmq_check(q4, orc, c["M"], c["N"], c["K"], c["seed"], c["outliers"], "mmq 2048 " + c["name"])


def test_mmq_pp1024_gate_up(q4, orc):
    # the prefill sweep's pp = 1024 point on the 4096 -> 12288 layer: the
    # routed call takes the int8 design here (the fp16 design's 384 tiles of
    # 256 x 128 would be one and a half rounds of the CUs): the pipelined
    # kernel, 768 tiles of 128 x 128 with its per-row records in the
    # workspace, 16 groups per tile
    c = wl.MMQ_2048[0]
    M = 1024
    assert q4.q4_mmq_workspace_bytes(M, c["N"], c["K"]) == q4.q4_mmq_int8_workspace_bytes(M, c["N"], c["K"]) > 0
    say("mmq pp1024 gate_up M=%d K=%d N=%d (every output)" % (M, c["K"], c["N"]))
    mmq_check(q4, orc, M, c["N"], c["K"], c["seed"], True, "mmq pp1024 gate_up")


@pytest.mark.parametrize("M,N,K", [(1024, 4096, 12288), (640, 6144, 4096)])
def test_mmq_one_round_int8_route(q4, orc, M, N, K):
    # grids whose 128 x 128 tiles fill the CUs in one round (256 and 240
    # tiles) while the fp16 design's 256 x 128 tiles would leave about half
    # of them idle: the fp32 route takes the pipelined integer kernel (its
    # per-row records in the workspace); the prefill sweep's pp = 1024 point
    # on the 12288 -> 4096 layer is the first shape (256 sampled rows)
    assert q4.q4_mmq_workspace_bytes(M, N, K) >= q4.q4_mmq_int8_workspace_bytes(M, N, K) > 0
    rows = np.sort(np.random.default_rng(M + N).choice(M, size=256, replace=False))
    say("mmq one-round int8 route M=%d N=%d K=%d (256 sampled rows)" % (M, N, K))
    W, x = wl.mmq_case(M + K, M, N, K, True)
    qs, sm = q4.q4_pack(dev(W))
    qa, ds = q4.q8_1_quantize(dev(x))
    y = q4.q4_mmq_gemm(qa, ds, qs, sm)
    assert torch.equal(y, q4.q4_mmq_gemm_int8(qa, ds, qs, sm))
    qa_h = qa.cpu().numpy()
    ds_h = ds.cpu().view(torch.int16).numpy().view(np.uint16)
    ref = orc.q4_mmq(qa_h[rows], ds_h[rows], qs.cpu().numpy(), sm.cpu().view(torch.int16).numpy().view(np.uint16), K)
    close(y.cpu().numpy()[rows], ref, "mmq one-round int8 %dx%dx%d" % (M, N, K))


INT8_FULL = [dict(wl.MMQ_512, name="m512")] + wl.MMQ_2048


@pytest.mark.parametrize("idx", range(len(INT8_FULL)))
def test_mmq_int8_design_full(q4, orc, idx):
    # q4_mmq_gemm_int8 at the prefill configs, where q4_mmq_gemm takes the
    # fp16 design: exact int32 block dots on int8 matrix cores, every output
    c = INT8_FULL[idx]
    say("mmq int8 design M=%d K=%d N=%d (every output)" % (c["M"], c["K"], c["N"]))
    W, x = wl.mmq_case(c["seed"], c["M"], c["N"], c["K"], c["outliers"])
    qs, sm = q4.q4_pack(dev(W))
    qa, ds = q4.q8_1_quantize(dev(x))
    y = q4.q4_mmq_gemm_int8(qa, ds, qs, sm)
    torch.cuda.synchronize()
    qs_o, sm_o = orc.q4_pack(W.numpy())
    assert_pack_equal(qs_o, sm_o, qs, sm, "int8 design pack")
    qa_o, ds_o = orc.q8_1_quantize(x.numpy())
    assert np.array_equal(qa.cpu().numpy(), qa_o)
    assert np.array_equal(ds.cpu().view(torch.int16).numpy().view(np.uint16), ds_o)
    close(y.cpu().numpy(), orc.q4_mmq(qa_o, ds_o, qs_o, sm_o, c["K"]), "mmq int8 design " + c["name"])


@pytest.mark.parametrize("M,N,K", [(100, 224, 2048), (1024, 12288, 4096), (257, 385, 1024)])
def test_mmq_int8_entry_matches_routed_int8(q4, orc, M, N, K):
    # where q4_mmq_gemm routes to the int8 design (K split, unsplit, ragged),
    # q4_mmq_gemm_int8 runs the same kernels: identical bits
    say("mmq int8 entry vs routed int8 M=%d N=%d K=%d" % (M, N, K))
    assert q4.q4_mmq_workspace_bytes(M, N, K) == q4.q4_mmq_int8_workspace_bytes(M, N, K)
    W, x = wl.mmq_case(M + N + K, M, N, K, True)
    qs, sm = q4.q4_pack(dev(W))
    qa, ds = q4.q8_1_quantize(dev(x))
    assert torch.equal(q4.q4_mmq_gemm_int8(qa, ds, qs, sm), q4.q4_mmq_gemm(qa, ds, qs, sm))


def test_mmq_split_k_small(q4, orc):
    # 2 output tiles and 8 groups of K: the launch splits K four ways and sums
    # the partials in a second pass
    say("mmq K split: M=100 N=200 K=2048 (4 splits)")
    assert q4.q4_mmq_workspace_bytes(100, 200, 2048) == 4 * 100 * 200 * 4
    mmq_check(q4, orc, 100, 200, 2048, 41, True, "mmq split 100x200x2048")


def test_mmq_split_k_pp256_down(q4, orc):
    # the 12288 -> 4096 prefill layer at 256 tokens: 64 tiles, K split 8 ways
    c = wl.MMQ_2048[1]
    say("mmq K split: M=256 K=%d N=%d (sampled activation rows)" % (c["K"], c["N"]))
    assert q4.q4_mmq_workspace_bytes(256, c["N"], c["K"]) == 8 * 256 * c["N"] * 4
    rows = np.unique(np.concatenate([[0, 255], np.random.default_rng(7).choice(256, 30, replace=False)]))
    mmq_check(q4, orc, 256, c["N"], c["K"], c["seed"], True, "mmq pp256 down", mrows=rows)


def test_gemv_k_beyond_one_workgroup(q4, orc):
    # K = 65792: the M = 1 and M = 2 activation images no longer fit one
    # workgroup's LDS, so they run on the matrix-core arm (one- and two-row
    # images) with K split over workgroups
    K = 65792
    assert q4.q4_gemv_workspace_bytes(1, 100, K) > 0
    for M in (1, 2, 3):
        say("gemv M=%d N=100 K=%d" % (M, K))
        W, x = wl.gemv_case(50 + M, M, 100, K)
        qs, sm = q4.q4_pack(dev(W))
        y = q4.q4_gemv(dev(x), qs, sm).cpu().numpy()
        ref = orc.q4_gemv(x.numpy(), qs.cpu().numpy(), sm.cpu().view(torch.int16).numpy().view(np.uint16), K)
        close(y, ref, "gemv K=%d M=%d" % (K, M))


def test_mmq_long_k(q4, orc):
    say("mmq M=130 N=100 K=65792")
    mmq_check(q4, orc, 130, 100, 65792, 77, True, "mmq long K")


@pytest.mark.parametrize("M,N,K,seed", [(100, 224, 512, 61), (100, 224, 2048, 62), (512, 9216, 2560, 0),
                                        (600, 6144, 4096, 63), (1024, 4096, 12288, 64),
                                        (1024, 12288, 4096, 65)])
def test_mmq_q8_1_output_bit_exact(q4, orc, M, N, K, seed):
    # the Q8_1-producing epilogue equals quantizing the fp32 GEMM result, bit
    # for bit (K = 2048 at 2 tiles takes the K-split path, whose sum pass
    # quantizes; the last three shapes, 240, 256 and 768 tiles of 128 x 128,
    # the pipelined integer kernel's epilogue, the first with ragged rows);
    # and the oracle's quantizer on that fp32 result agrees too
    say("mmq -> Q8_1 M=%d N=%d K=%d" % (M, N, K))
    W, x = wl.mmq_case(seed, M, N, K, True)
    qs, sm = q4.q4_pack(dev(W))
    qa, ds = q4.q8_1_quantize(dev(x))
    qo, dso = q4.q4_mmq_gemm_q8_1(qa, ds, qs, sm)
    y = q4.q4_mmq_gemm(qa, ds, qs, sm)
    qr, dsr = q4.q8_1_quantize(y)
    assert torch.equal(qo, qr)
    assert torch.equal(dso.view(torch.int16), dsr.view(torch.int16))
    rows = slice(None) if M <= 100 else slice(0, 64)
    oq, ods = orc.q8_1_quantize(y[rows].cpu().numpy())
    assert np.array_equal(qo[rows].cpu().numpy(), oq)
    assert np.array_equal(dso[rows].cpu().view(torch.int16).numpy().view(np.uint16), ods)


def test_mmq_m1_matches_gemv_on_dequantized_row(q4, orc):
    say("mmq M=1 vs gemv on the dequantized Q8_1 row")
    W, x = wl.mmq_case(5, 1, 777, 2560)
    qs, sm = q4.q4_pack(dev(W))
    qa, ds = q4.q8_1_quantize(dev(x))
    y1 = q4.q4_mmq_gemm(qa, ds, qs, sm)
    xd = orc.q8_1_dequant(qa.cpu().numpy(), ds.cpu().view(torch.int16).numpy().view(np.uint16))
    y2 = q4.q4_gemv(dev(torch.from_numpy(xd.astype(np.float32))), qs, sm)
    close(y1.cpu().numpy(), y2.cpu().numpy(), "mmq(M=1) vs gemv")


def test_mmq_deterministic(q4, orc):
    say("mmq rerun determinism")
    W, x = wl.mmq_case(6, 300, 500, 1024)
    qs, sm = q4.q4_pack(dev(W))
    qa, ds = q4.q8_1_quantize(dev(x))
    a = q4.q4_mmq_gemm(qa, ds, qs, sm)
    b = q4.q4_mmq_gemm(qa, ds, qs, sm)
    assert torch.equal(a, b)


def _mmq_vs_oracle(q4, orc, W, x, what):
    qs, sm = q4.q4_pack(dev(W))
    qa, ds = q4.q8_1_quantize(dev(x))
    y = q4.q4_mmq_gemm(qa, ds, qs, sm).cpu().numpy()
    ref = orc.q4_mmq(qa.cpu().numpy(), ds.cpu().view(torch.int16).numpy().view(np.uint16), qs.cpu().numpy(),
                     sm.cpu().view(torch.int16).numpy().view(np.uint16), W.shape[1])
    close(y, ref, what)


def test_mmq_extreme_block_sums(q4, orc):
    # The fp32-output MMQ sums each group's eight block dots in int32 with
    # 13-bit block scales.  Near its bound: every activation at +-127 with all
    # block scales equal (D = 8191) against groups whose 255 lowest weights
    # give code 0 (centred -8), i.e. |block dot| close to 32 * 127 * 8.
    say("mmq near the int32 bound of the group sums")
    M, N, K = 130, 100, 2048
    rng = np.random.default_rng(11)
    W = torch.full((N, K), -0.01, dtype=torch.float32)
    W[:, 255::256] = 0.03  # one maximum per group: scale != 0, all other codes 0
    W[N // 2:] = torch.from_numpy((0.02 * rng.standard_normal((N - N // 2, K))).astype(np.float32))
    x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32))
    x[0:40] = 1.5
    x[40:80] = -2.5
    _mmq_vs_oracle(q4, orc, W, x, "mmq extreme block sums")


def test_mmq_massive_activations(q4, orc):
    # block scales within one group far apart: one channel 1000x, 1 % of the
    # rest 100x
    say("mmq with a 1000x channel and 100x outliers")
    M, N, K = 257, 385, 1024
    rng = np.random.default_rng(12)
    W = torch.from_numpy((0.02 * rng.standard_normal((N, K))).astype(np.float32))
    x = rng.standard_normal((M, K)).astype(np.float32)
    x = np.where(rng.random((M, K)) < 0.01, x * 100, x).astype(np.float32)
    x[:, 7] *= 1000
    _mmq_vs_oracle(q4, orc, W, torch.from_numpy(x), "mmq massive activations")


def test_mmq_degenerate_groups(q4, orc):
    # the integer group combination at its edges: rows of zeros (every block
    # scale 0, step 0), one non-zero block per group, a group whose block
    # scales span fp16-subnormal to large values, constant weight groups
    # (scale 0, only the minimum term) and a zero weight row
    say("mmq degenerate activation and weight groups")
    M, N, K = 10, 70, 1024
    rng = np.random.default_rng(13)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[0] = 0.0
    x[1] = 0.0
    x[1, 40:72] = rng.standard_normal(32)           # one block of group 0 only
    x[1, 300] = 5.0                                  # one value in group 1
    x[2, :32] = 3e4                                  # huge block next to
    x[2, 32:64] = rng.standard_normal(32) * 1e-6     # an fp16-subnormal d
    x[3, ::256] = -7e3                               # a spike per group
    W = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    W[0, :256] = 0.125                               # constant group: scale 0
    W[1] = -0.5                                      # constant row
    W[2] = 0.0                                       # zero row
    _mmq_vs_oracle(q4, orc, torch.from_numpy(W), torch.from_numpy(x), "mmq degenerate groups")


# ------------------------------------------------- MMQ, fp16 matrix cores ---
# Shapes whose grid of 256 x 128 tiles fills the GPU run on the fp16 design;
# its workspace (the fp16 activation image, 2 K bytes per row padded to whole
# tiles of 256 or 192 rows, plus 4 bytes per row) tells which design a shape
# takes.

def f16_tile_rows(M, N):
    # 192-row tiles where the grid of 256-row tiles fills at most two rounds
    # of 256 CUs and 192-row tiles take fewer rows x rounds, else 256
    nt = (N + 127) // 128
    t256, t192 = (M + 255) // 256 * nt, (M + 191) // 192 * nt
    if t256 > 512:
        return 256
    return 192 if (t192 + 255) // 256 * 192 < (t256 + 255) // 256 * 256 else 256


def f16_workspace(M, N, K):
    # activation image (2 K bytes per row, rows padded to whole tiles), a row
    # factor per row, and (E, 2^-E) per weight row (rows padded to 128)
    fm = f16_tile_rows(M, N)
    rows = (M + fm - 1) // fm * fm
    return rows * K * 2 + rows * 4 + (N + 127) // 128 * 128 * 8


@pytest.mark.parametrize("design,M,N,K", [("f16", 1024, 8192, 512), ("int8", 300, 200, 768),
                                          ("int8", 2048, 256, 4096)])
def test_mmq_layout_probe(q4, orc, design, M, N, K):
    # one nonzero activation per row, at k = m mod K: y[m][n] is that value
    # (as Q8_1 holds it) times the dequantized W[n][m mod K], so every
    # (m, n, k) place of the operand layouts meets its own weight; the
    # expectation uses the oracle's dequantizers only, not its product
    say("mmq layout probe (%s design) M=%d N=%d K=%d" % (design, M, N, K))
    if design == "f16":
        assert q4.q4_mmq_workspace_bytes(M, N, K) == f16_workspace(M, N, K)
    W, _ = wl.gemv_case(M + N, 1, N, K)
    rows, ks = np.arange(M), np.arange(M) % K
    x = np.zeros((M, K), dtype=np.float32)
    x[rows, ks] = 1.0 + (rows % 7) / 8.0
    qs, sm = q4.q4_pack(dev(W))
    qa, ds = q4.q8_1_quantize(dev(torch.from_numpy(x)))
    gemm = q4.q4_mmq_gemm if design == "f16" else q4.q4_mmq_gemm_int8
    y = gemm(qa, ds, qs, sm).cpu().numpy()
    wdq = orc.q4_dequant(qs.cpu().numpy(), sm.cpu().view(torch.int16).numpy().view(np.uint16), K)
    xdq = orc.q8_1_dequant(qa.cpu().numpy(), ds.cpu().view(torch.int16).numpy().view(np.uint16))
    ref = xdq[rows, ks][:, None] * wdq[:, ks].T
    assert np.count_nonzero(xdq) == M
    close(y, ref, "mmq layout probe " + design)


def test_mmq_f16_ragged(q4, orc):
    # 2 x 100 tiles, both edges ragged (300 = 256 + 44 rows, 12700 = 99 * 128 + 28)
    M, N, K = 300, 12700, 512
    say("mmq fp16 design M=%d N=%d K=%d" % (M, N, K))
    assert q4.q4_mmq_workspace_bytes(M, N, K) == f16_workspace(M, N, K)
    mmq_check(q4, orc, M, N, K, 71, True, "mmq fp16 ragged")


def test_mmq_f16_persistent_uneven(q4, orc):
    # 5 x 100 = 500 tiles over one workgroup per CU: most workgroups take two
    # tiles (the second one's stages stream in behind the first one's
    # epilogue), the rest one, and both edges are ragged (1100 = 4 * 256 +
    # 76 rows, 12700 = 99 * 128 + 28); the Q8_1 output takes the same tiles
    M, N, K = 1100, 12700, 512
    say("mmq fp16 design, uneven persistent tiles M=%d N=%d K=%d" % (M, N, K))
    assert q4.q4_mmq_workspace_bytes(M, N, K) == f16_workspace(M, N, K)
    y = mmq_check(q4, orc, M, N, K, 75, True, "mmq fp16 persistent uneven")
    N8 = 12672  # a multiple of 32 for the Q8_1 output, still ragged at 99 * 128
    W, x = wl.mmq_case(76, M, N8, K, True)
    qs, sm = q4.q4_pack(dev(W))
    qa, ds = q4.q8_1_quantize(dev(x))
    qo, dso = q4.q4_mmq_gemm_q8_1(qa, ds, qs, sm)
    qr, dsr = q4.q8_1_quantize(q4.q4_mmq_gemm(qa, ds, qs, sm))
    torch.cuda.synchronize()
    assert torch.equal(qo, qr) and torch.equal(dso.view(torch.int16), dsr.view(torch.int16))


def test_mmq_f16_extremes(q4, orc):
    # the per-row and per-weight-row powers of two at their edges: the
    # degenerate activation rows and weight groups of the int8 test, plus
    # activation rows scaled by 1e-4 and 6e4 and weight rows by 1e-5 and 1e4
    M, N, K = 260, 12300, 1024
    say("mmq fp16 design with extreme and degenerate rows M=%d N=%d K=%d" % (M, N, K))
    assert q4.q4_mmq_workspace_bytes(M, N, K) == f16_workspace(M, N, K)
    rng = np.random.default_rng(14)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[0] = 0.0
    x[1] = 0.0
    x[1, 40:72] = rng.standard_normal(32)
    x[2, :32] = 3e4
    x[2, 32:64] = rng.standard_normal(32) * 1e-6
    x[3, ::256] = -7e3
    x[4] *= 1e-4
    x[5] *= 6e4 / np.abs(x[5]).max()
    x[257] = 1.0                                     # a row of the ragged tile
    W = (0.02 * rng.standard_normal((N, K))).astype(np.float32)
    W[0, :256] = 0.125
    W[1] = -0.5
    W[2] = 0.0
    W[3] *= 1e-5 / 0.02
    W[4] *= 1e4 / 0.02
    W[5, 256:512] = 3.0                              # a constant group amid N(0, 0.02)
    W[N - 1] = 0.25                                  # last (ragged) weight row
    qs, sm = q4.q4_pack(dev(torch.from_numpy(W)))
    qa, ds = q4.q8_1_quantize(dev(torch.from_numpy(x)))
    y = q4.q4_mmq_gemm(qa, ds, qs, sm).cpu().numpy()
    ref = orc.q4_mmq(qa.cpu().numpy(), ds.cpu().view(torch.int16).numpy().view(np.uint16), qs.cpu().numpy(),
                     sm.cpu().view(torch.int16).numpy().view(np.uint16), K)
    assert np.isfinite(y).all()
    close(y, ref, "mmq fp16 extremes")
    # the huge rows dominate the global measure: check the ordinary block and
    # each extreme row and weight row on its own scale as well
    close(y[6:257, 6:N - 1], ref[6:257, 6:N - 1], "mmq fp16 extremes, ordinary block")
    for r in (1, 2, 3, 4, 5, 257):
        close(y[r:r + 1, 6:N - 1], ref[r:r + 1, 6:N - 1], "mmq fp16 extremes, activation row %d" % r)
    for c in (0, 1, 3, 4, 5, N - 1):
        close(y[6:257, c:c + 1], ref[6:257, c:c + 1], "mmq fp16 extremes, weight row %d" % c)


def test_mmq_f16_q8_1_output_bit_exact(q4, orc):
    M, N, K = 300, 12288, 512
    say("mmq fp16 design -> Q8_1 M=%d N=%d K=%d" % (M, N, K))
    assert q4.q4_mmq_workspace_bytes(M, N, K) == f16_workspace(M, N, K)
    W, x = wl.mmq_case(72, M, N, K, True)
    qs, sm = q4.q4_pack(dev(W))
    qa, ds = q4.q8_1_quantize(dev(x))
    qo, dso = q4.q4_mmq_gemm_q8_1(qa, ds, qs, sm)
    y = q4.q4_mmq_gemm(qa, ds, qs, sm)
    qr, dsr = q4.q8_1_quantize(y)
    assert torch.equal(qo, qr)
    assert torch.equal(dso.view(torch.int16), dsr.view(torch.int16))
    rows = slice(256, 300)
    oq, ods = orc.q8_1_quantize(y[rows].cpu().numpy())
    assert np.array_equal(qo[rows].cpu().numpy(), oq)
    assert np.array_equal(dso[rows].cpu().view(torch.int16).numpy().view(np.uint16), ods)


def test_mmq_f16_deterministic(q4, orc):
    M, N, K = 512, 9216, 2560
    say("mmq fp16 design rerun determinism M=%d N=%d K=%d" % (M, N, K))
    assert q4.q4_mmq_workspace_bytes(M, N, K) == f16_workspace(M, N, K)
    W, x = wl.mmq_case(73, M, N, K, True)
    qs, sm = q4.q4_pack(dev(W))
    qa, ds = q4.q8_1_quantize(dev(x))
    a = q4.q4_mmq_gemm(qa, ds, qs, sm)
    b = q4.q4_mmq_gemm(qa, ds, qs, sm)
    assert torch.equal(a, b)
