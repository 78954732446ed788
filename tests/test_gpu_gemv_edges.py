"""GEMV edge cases against the CPU oracle: activation magnitudes at both ends
of fp32's range on every arm, and weight matrices beyond the 2 GiB reach of
one buffer descriptor (several row ranges in one call).

The GEMV scales each chunk of 32 (VALU arm) or group of 256 (matrix-core arm)
of x by a power of two before rounding it to fp16, and carries its partial
sums at 2^-10 of their value; these tests hold both to the oracle where that
bookkeeping is at its limits: fp32 subnormal and all-zero chunks next to
ordinary ones, rows that are tiny or huge throughout, and chunks beyond 2^118.
"""
import numpy as np
import pytest
import torch

from bit_quantized_matmul_q4_amd import workloads as wl
from test_gpu_parity import close, dev, say

pytestmark = pytest.mark.gpu

K_EDGE, N_EDGE = 2560, 300   # 80 chunks, 10 groups; N small enough for the K-split paths


def magnitude_rows(seed):
    """Eight activation rows of K_EDGE values spanning fp32's range."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((8, K_EDGE)).astype(np.float32)
    c = lambda i: slice(32 * i, 32 * i + 32)  # noqa: E731  chunk i
    x[0, c(3)] *= np.float32(1e-36)           # ordinary row with tiny chunks,
    x[0, c(5)] *= np.float32(1e-40)           # an fp32-subnormal chunk,
    x[0, c(7)] = 0.0                          # a zero chunk
    x[0, 256 * 2:256 * 3] *= np.float32(1e-38)  # and a tiny group of 256
    x[1] *= np.float32(1e-36)                 # tiny throughout (y still normal)
    x[2] *= np.float32(1e-40)                 # subnormal throughout (y subnormal)
    x[3, c(9)] *= np.float32(1e30)            # huge chunks next to ordinary ones,
    x[3, c(40)] *= np.float32(1e37)           # one beyond 2^118
    x[4] *= np.float32(1e37)                  # huge throughout
    x[5] = 0.0                                # zero row
    x[6] *= np.float32(3e-39)
    x[6, c(0)] = np.float32(1.4e-45) * np.sign(x[6, c(0)])  # the smallest subnormal
    x[6, c(0)][x[6, c(0)] == 0] = np.float32(1.4e-45)
    return x                                  # row 7: ordinary


def check_rows(y, ref, what):
    """Rows whose reference reaches 1e-37 are held to the usual tolerance on
    their own scale; rows whose outputs are fp32 subnormals must be finite
    and within 2^-126 of the reference."""
    y = np.asarray(y, np.float64)
    assert np.isfinite(y).all(), what + ": non-finite output"
    for r in range(ref.shape[0]):
        top = np.abs(ref[r]).max()
        if top >= 1e-37:
            close(y[r], ref[r], "%s row %d" % (what, r))
        else:
            err = np.abs(y[r] - ref[r]).max()
            say("  %s row %d: max|ref|=%.3e max|err|=%.3e" % (what, r, top, err))
            assert err <= 2.0 ** -126, "%s row %d: error %.3e" % (what, r, err)


def gemv_fn(q4, group):
    return q4.q4_gemv if group == 256 else q4.q4_gemv_g32


def pack_fn(q4, group):
    return q4.q4_pack if group == 256 else q4.q4_pack_g32


@pytest.mark.parametrize("group", [256, 32])
def test_gemv_activation_magnitudes_every_arm(q4, orc, group):
    say("gemv activation magnitudes, group %d, K=%d N=%d" % (group, K_EDGE, N_EDGE))
    W, _ = wl.gemv_case(60, 1, N_EDGE, K_EDGE)
    x = magnitude_rows(61)
    qs, sm = pack_fn(q4, group)(dev(W))
    qs_o, sm_o = orc.q4_pack(W.numpy(), group=group)
    assert np.array_equal(qs.cpu().numpy(), qs_o)
    assert np.array_equal(sm.cpu().view(torch.int16).numpy().view(np.uint16), sm_o)
    ref = orc.q4_gemv(x, qs_o, sm_o, K_EDGE, group=group)
    xd = dev(torch.from_numpy(x))
    f = gemv_fn(q4, group)
    # one row per call (VALU arm, one row), pairs (two rows), quads (four
    # rows below 65536 weight rows) and all eight (matrix-core arm, K split)
    for rows in [[r] for r in range(8)] + [[0, 1], [2, 3], [4, 5], [6, 7]] + [[0, 1, 2, 3], [4, 5, 6, 7]] + \
            [list(range(8))]:
        got = f(xd[rows].contiguous(), qs, sm).cpu().numpy()
        check_rows(got, ref[rows], "g%d M=%d rows %s" % (group, len(rows), rows))


def test_gemv_activation_magnitudes_long_k(q4, orc):
    # M = 1 beyond arm A's LDS: the matrix-core arm's K split on the same
    # kinds of rows (chunks repeat every 2560 of K)
    K = 65792
    say("gemv activation magnitudes, matrix-core arm at K=%d" % K)
    W, _ = wl.gemv_case(62, 1, 100, K)
    base = magnitude_rows(63)
    x = np.concatenate([base] * (K // K_EDGE + 1), axis=1)[:, :K].copy()
    qs, sm = q4.q4_pack(dev(W))
    ref = orc.q4_gemv(x, qs.cpu().numpy(), sm.cpu().view(torch.int16).numpy().view(np.uint16), K)
    xd = dev(torch.from_numpy(x))
    for rows in ([0], [1], [3], [4], [2], [0, 1, 2, 3, 4, 5, 6, 7]):
        got = q4.q4_gemv(xd[rows].contiguous(), qs, sm).cpu().numpy()
        check_rows(got, ref[rows], "long K rows %s" % rows)


def test_gemv_beyond_2gib_of_weights(q4, orc):
    # 1048576 x 4096 weights: 2 GiB of codes, so the call runs two row ranges
    # (1048512 rows, then 64).  Every range must use the plan of the whole
    # shape: M = 8 needs no workspace for N = 1048576, and the 64-row tail
    # must not switch to a K split of its own.
    N, K = 1048576, 4096
    assert q4.q4_gemv_workspace_bytes(8, N, K) == 0
    say("gemv beyond 2 GiB of weights: N=%d K=%d" % (N, K))
    g = torch.Generator(device="cuda").manual_seed(64)
    W = torch.randn((N, K), generator=g, device="cuda", dtype=torch.float32).mul_(0.02)
    qs, sm = q4.q4_pack(W)
    boundary = 1048512
    rows = np.unique(np.concatenate([[0, 1, boundary - 2, boundary - 1, boundary, boundary + 1, N - 2, N - 1],
                                     np.random.default_rng(65).choice(N, 500, replace=False)]))
    ridx = torch.from_numpy(rows).cuda()
    Wr = W.index_select(0, ridx).cpu().numpy()
    del W
    torch.cuda.synchronize()
    qs_o, sm_o = orc.q4_pack(Wr)
    assert np.array_equal(qs.index_select(0, ridx).cpu().numpy(), qs_o)
    assert np.array_equal(sm.index_select(0, ridx).cpu().view(torch.int16).numpy().view(np.uint16), sm_o)
    for M in (1, 2, 8, 16):
        say("  M=%d" % M)
        x = wl.draw_activations(wl.generator(66 + M), M, K)
        y = q4.q4_gemv(dev(x), qs, sm)
        got = y.index_select(1, ridx).cpu().numpy()
        close(got, orc.q4_gemv(x.numpy(), qs_o, sm_o, K), "gemv %d x %d x %d (sampled rows)" % (M, N, K))
    del qs, sm
    torch.cuda.empty_cache()


def test_gemv_g32_beyond_2gib_of_weights(q4, orc):
    # the group-32 GEMV on 1048576 x 4096 weights: two row ranges (1048512
    # rows and 64) as above, and at M >= 2 a K split in two whose partials
    # for every range fit the workspace sized for the whole shape
    N, K = 1048576, 4096
    say("gemv g32 beyond 2 GiB of weights: N=%d K=%d" % (N, K))
    g = torch.Generator(device="cuda").manual_seed(67)
    W = torch.randn((N, K), generator=g, device="cuda", dtype=torch.float32).mul_(0.02)
    qs, sm = q4.q4_pack_g32(W)
    boundary = 1048512
    rows = np.unique(np.concatenate([[0, 1, boundary - 2, boundary - 1, boundary, boundary + 1, N - 2, N - 1],
                                     np.random.default_rng(68).choice(N, 500, replace=False)]))
    ridx = torch.from_numpy(rows).cuda()
    Wr = W.index_select(0, ridx).cpu().numpy()
    del W
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    qs_o, sm_o = orc.q4_pack(Wr, group=32)
    assert np.array_equal(qs.index_select(0, ridx).cpu().numpy(), qs_o)
    assert np.array_equal(sm.index_select(0, ridx).cpu().view(torch.int16).numpy().view(np.uint16), sm_o)
    for M in (1, 2, 8, 16):
        say("  M=%d (workspace %d bytes)" % (M, q4.q4_gemv_g32_workspace_bytes(M, N, K)))
        x = wl.draw_activations(wl.generator(69 + M), M, K)
        y = q4.q4_gemv_g32(dev(x), qs, sm)
        got = y.index_select(1, ridx).cpu().numpy()
        close(got, orc.q4_gemv(x.numpy(), qs_o, sm_o, K, group=32),
              "gemv g32 %d x %d x %d (sampled rows)" % (M, N, K))
    del qs, sm
    torch.cuda.empty_cache()
