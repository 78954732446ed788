"""The C oracle against a second, independently written implementation.

A small vectorised numpy version of every oracle function is written here
from the definitions alone: the HFQ4-G256 format of the hipfire MMQ-prefill
note as this project reads it, 4-bit codes in groups of 256 (or 32) with an
fp16 scale and minimum; Q8_1 blocks of 32 with an fp16 d and s, as the same
note's "list of changes" names them; and the block dot products and fp64
sums built on them.  It runs on tiny shapes.  Integer results and fp16 bit
patterns must agree exactly, and fp64 sums to 1e-12 relative.

This does not replace the pins in test_oracle_pins.py: both implementations
follow the same readings, so they can share a misreading.  What it catches
is an implementation slip in either one, such as a wrong byte or nibble
position, a swapped operand, an off-by-one group, or a rounding taken in
the wrong precision.  The decisions are taken as the readings state: IEEE
fp32 with round-to-nearest-even, and numpy's float16 conversion for fp16.
"""
import numpy as np
import pytest

F32 = np.float32


def np_code_layout(K):
    """byte index and nibble (0 low, 1 high) of each element k of a row"""
    k = np.arange(K)
    j, i = k // 32, k % 32
    return 16 * j + (i & 15), (i >= 16).astype(np.int64)


def np_pack(W, group):
    W = np.asarray(W, dtype=F32)
    N, K = W.shape
    Wg = W.reshape(N, K // group, group)
    mn = Wg.min(axis=2) + F32(0.0)          # -0 counts as +0
    mx = Wg.max(axis=2) + F32(0.0)
    s16 = ((mx - mn) / F32(15.0)).astype(np.float16)
    m16 = mn.astype(np.float16)
    sf, mf = s16.astype(F32), m16.astype(F32)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = (Wg - mf[:, :, None]) / sf[:, :, None]
    q = np.clip(np.rint(t), 0, 15)
    q = np.where(sf[:, :, None] == 0, 0, q).astype(np.uint8).reshape(N, K)
    byte, hi = np_code_layout(K)
    qs = np.zeros((N, K // 2), dtype=np.uint8)
    for h in (0, 1):
        cols = np.flatnonzero(hi == h)
        qs[:, byte[cols]] |= (q[:, cols] << (4 * h)).astype(np.uint8)
    sm = np.stack([s16.view(np.uint16), m16.view(np.uint16)], axis=2)
    return qs, sm


def np_codes(qs, K):
    byte, hi = np_code_layout(K)
    return (qs[:, byte] >> (4 * hi)) & 15


def np_dequant(qs, sm, K, group):
    q = np_codes(qs, K).astype(np.float64)
    s = sm[:, :, 0].view(np.float16).astype(np.float64)
    m = sm[:, :, 1].view(np.float16).astype(np.float64)
    return np.repeat(s, group, axis=1) * q + np.repeat(m, group, axis=1)


def np_q8_1(x):
    x = np.asarray(x, dtype=F32)
    M, K = x.shape
    xb = x.reshape(M, K // 32, 32)
    d16 = (np.abs(xb).max(axis=2) / F32(127.0)).astype(np.float16)
    df = d16.astype(F32)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = xb / df[:, :, None]
    a = np.clip(np.rint(t), -127, 127)
    a = np.where(df[:, :, None] == 0, 0, a).astype(np.int32)
    s16 = (df * a.sum(axis=2).astype(F32)).astype(np.float16)
    ds = np.stack([d16.view(np.uint16), s16.view(np.uint16)], axis=2)
    return a.reshape(M, K).astype(np.int8), ds


def np_block_dots(qa, qs, K):
    q = np_codes(qs, K).astype(np.int64)
    a = qa.astype(np.int64)
    M, N = a.shape[0], q.shape[0]
    return np.einsum("mbi,nbi->mnb", a.reshape(M, K // 32, 32), q.reshape(N, K // 32, 32))


def np_mmq(qa, ds, qs, sm, K, group):
    d = ds[:, :, 0].view(np.float16).astype(np.float64)
    xq = qa.astype(np.float64) * np.repeat(d, 32, axis=1)
    return xq @ np_dequant(qs, sm, K, group).T


def rel(a, b):
    den = max(np.abs(b).max(), 1e-300)
    return np.abs(np.asarray(a) - np.asarray(b)).max() / den


def weights(rng, N, K):
    W = (rng.standard_normal((N, K)) * 0.02).astype(F32)
    W[0, :32] = 0.0                      # a constant run
    W[1 % N, 40:72] = -0.0
    W[2 % N, :256] = np.float32(0.25)    # a constant group
    return W


def activations(rng, M, K):
    x = rng.standard_normal((M, K)).astype(F32)
    x[rng.random((M, K)) < 0.02] *= 20.0
    x[0, :32] = 0.0                      # an all-zero block
    # the last block of the last row: d = 2^-3 exactly and x / d = j + 1/2,
    # exact ties for the int8 rounding (to even, not away from zero)
    h = np.float32(0.125)
    tie = (np.arange(-16, 16, dtype=F32) + F32(0.5)) * h
    tie[0] = F32(127.0) * h
    x[M - 1, K - 32:] = tie
    return x


@pytest.mark.parametrize("group", [256, 32])
@pytest.mark.parametrize("N,K,seed", [(1, 256, 1), (5, 512, 2), (7, 768, 3)])
def test_pack_and_dequant_agree(orc, group, N, K, seed):
    W = weights(np.random.default_rng(seed), N, K)
    qs_c, sm_c = orc.q4_pack(W, group=group)
    qs_n, sm_n = np_pack(W, group)
    assert np.array_equal(qs_c, qs_n)
    assert np.array_equal(sm_c, sm_n)
    assert np.array_equal(orc.q4_codes(qs_c, K), np_codes(qs_n, K))
    assert rel(orc.q4_dequant(qs_c, sm_c, K, group=group), np_dequant(qs_n, sm_n, K, group)) == 0.0


@pytest.mark.parametrize("M,K,seed", [(1, 32, 4), (3, 256, 5), (4, 1024, 6)])
def test_q8_1_agrees(orc, M, K, seed):
    x = activations(np.random.default_rng(seed), M, K)
    qa_c, ds_c = orc.q8_1_quantize(x)
    qa_n, ds_n = np_q8_1(x)
    assert np.array_equal(qa_c, qa_n)
    assert np.array_equal(ds_c, ds_n)
    d = ds_n[:, :, 0].view(np.float16).astype(np.float64)
    assert rel(orc.q8_1_dequant(qa_c, ds_c), qa_n.astype(np.float64) * np.repeat(d, 32, axis=1)) == 0.0


@pytest.mark.parametrize("group", [256, 32])
@pytest.mark.parametrize("M,N,K,seed", [(1, 3, 256, 7), (3, 5, 512, 8), (2, 9, 1024, 9)])
def test_products_agree(orc, group, M, N, K, seed):
    rng = np.random.default_rng(seed)
    W = weights(rng, N, K)
    x = activations(rng, M, K)
    qs, sm = np_pack(W, group)
    qa, ds = np_q8_1(x)
    assert np.array_equal(orc.q4_block_dots(qa, qs, K), np_block_dots(qa, qs, K))
    y_gemv = x.astype(np.float64) @ np_dequant(qs, sm, K, group).T
    assert rel(orc.q4_gemv(x, qs, sm, K, group=group), y_gemv) < 1e-12
    assert rel(orc.q4_mmq(qa, ds, qs, sm, K, group=group), np_mmq(qa, ds, qs, sm, K, group)) < 1e-12


CROSS_CASES = [(test_pack_and_dequant_agree, (256, 5, 512, 2)), (test_pack_and_dequant_agree, (32, 7, 768, 3)),
               (test_q8_1_agrees, (3, 256, 5)), (test_products_agree, (256, 3, 5, 512, 8)),
               (test_products_agree, (32, 2, 9, 1024, 9))]


@pytest.mark.parametrize("mut", range(1, 11))
def test_cross_check_catches_planted_mistakes(orc, mut):
    # each of the oracle's test-only planted mistakes makes at least one of
    # the comparisons above fail
    orc.set_mutation(mut)
    try:
        assert orc.get_mutation() == mut
        failed = 0
        for fn, args in CROSS_CASES:
            try:
                fn(orc, *args)
            except AssertionError:
                failed += 1
        assert failed > 0, "planted mistake %d not caught" % mut
    finally:
        orc.set_mutation(0)
