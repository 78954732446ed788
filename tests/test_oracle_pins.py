"""Pins of the CPU oracle to facts outside itself.

Each ``pin_*`` function checks the oracle against something the pages, the
project's stated readings or plain mathematics fix: hand-derived byte layouts
and rounding ties (tests/golden/), closed forms built so that the exact answer
is known by construction, brute-force nearest-level searches on small inputs,
library routines on the special cases they cover (numpy's IEEE binary16
conversion, numpy fp64 matmul of an input that is exactly representable), and
invariants (idempotence, power-of-two equivariance, linearity, row
independence, error bounds).

``test_mutations_are_caught`` plants each of the oracle's test-only mistakes
in turn and requires at least one pin to fail for every one of them.
"""
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = vals
    return out


def _hexbytes(tokens):
    return np.frombuffer(bytes.fromhex("".join(tokens)), dtype=np.uint8)


def _f16(v):
    return np.float32(np.float16(v))


def grid_weights(rng, N, K, with_ends=True, group=256):
    """W exactly on the 4-bit grid: W[n, k] = mf + sf * c with fp16-exact
    (mf, sf) per group of ``group`` weights.  Returns (W fp32, codes, sf per
    group, mf per group).  With ``with_ends`` every group contains codes 0 and
    15, so the group min and max are mf and mf + 15 sf and packing must return
    exactly c."""
    G = K // group
    codes = rng.integers(0, 16, size=(N, K)).astype(np.int64)
    if with_ends:
        for n in range(N):
            for g in range(G):
                i0, i1 = rng.choice(group, size=2, replace=False)
                codes[n, g * group + i0] = 0
                codes[n, g * group + i1] = 15
    # scales: small integers times powers of two, all exact in fp16 and fp32
    sf = (rng.integers(1, 32, size=(N, G)) * 2.0 ** rng.integers(-12, -4, size=(N, G)))
    mf = (rng.integers(-64, 64, size=(N, G)) * 2.0 ** rng.integers(-10, -5, size=(N, G)))
    sfk = np.repeat(sf, group, axis=1)
    mfk = np.repeat(mf, group, axis=1)
    W = mfk + sfk * codes
    assert np.all(W.astype(np.float32).astype(np.float64) == W)
    return W.astype(np.float32), codes, sf, mf


def grid_activations(rng, M, K):
    """x exactly on the Q8_1 grid: x = 2^j * c with integer c, |c| <= 127 and
    |c| = 127 present in every block; returns (x fp32, codes, d per block)."""
    B = K // 32
    c = rng.integers(-127, 128, size=(M, K)).astype(np.int64)
    for m in range(M):
        for b in range(B):
            i = rng.integers(0, 32)
            c[m, b * 32 + i] = 127 if rng.random() < 0.5 else -127
    j = rng.integers(-9, 3, size=(M, B)).astype(np.float64)
    d = 2.0 ** j
    x = c * np.repeat(d, 32, axis=1)
    assert np.all(x.astype(np.float32).astype(np.float64) == x)
    return x.astype(np.float32), c, d


# ---------------------------------------------------------------- fp16 ----

def pin_f16_matches_ieee(o):
    rng = np.random.default_rng(11)
    v = rng.standard_normal(3000) * 10.0 ** rng.integers(-10, 6, 3000)
    edge = [0.0, -0.0, 65504, 65519.99, 65520, 65536, 1e-8, 2 ** -24, 2 ** -25,
            3 * 2 ** -26, 2 ** -14, -1.5 * 2 ** -14, 1 + 2 ** -11, 1 + 3 * 2 ** -11,
            2049, 2051, np.inf, -np.inf]
    v = np.concatenate([v, edge]).astype(np.float32)
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    ours = o.f32_to_f16(v)
    assert np.array_equal(ours, ref), "fp32->fp16 differs from IEEE RNE"
    h = np.arange(0, 65536, 97, dtype=np.uint16)
    h = h[(h & 0x7C00) != 0x7C00]
    assert np.array_equal(o.f16_to_f32(h), h.view(np.float16).astype(np.float32))


# ---------------------------------------------------------------- pack ----

def pin_pack_layout_golden(o):
    g = _golden("nibble_layout.txt")
    k = np.arange(256)
    for name, codes in (("pattern_a", k % 16), ("pattern_b", (k // 16) % 16)):
        W = (-0.5 + 0.0625 * codes).astype(np.float32)[None, :]
        qs, sm = o.q4_pack(W)
        assert np.array_equal(qs[0], _hexbytes(g[name])), name
        assert o.f16_to_f32(sm[0, 0, 0]) == 0.0625 and o.f16_to_f32(sm[0, 0, 1]) == -0.5
    row = np.concatenate([-0.5 + 0.0625 * (k % 16), -0.5 + 0.0625 * ((k // 16) % 16)])
    qs, _ = o.q4_pack(row.astype(np.float32)[None, :])
    assert np.array_equal(qs[0], _hexbytes(g["row_two_groups"]))


def pin_pack_closed_form(o):
    rng = np.random.default_rng(1)
    W, codes, sf, mf = grid_weights(rng, 5, 1024)
    qs, sm = o.q4_pack(W)
    assert np.array_equal(o.q4_codes(qs, 1024), codes), "codes of an exact grid"
    assert np.array_equal(o.f16_to_f32(sm[..., 0]), sf.astype(np.float32))
    assert np.array_equal(o.f16_to_f32(sm[..., 1]), mf.astype(np.float32))
    assert np.array_equal(o.q4_dequant(qs, sm, 1024), W.astype(np.float64))


def pin_pack_constant_and_two_valued(o):
    W = np.full((1, 512), 0.3, dtype=np.float32)
    W[0, 256:] = np.where(np.arange(256) % 3 == 0, -0.125, 0.75)
    qs, sm = o.q4_pack(W)
    c = o.q4_codes(qs, 512)[0]
    assert sm[0, 0, 0] == 0 and np.all(c[:256] == 0), "constant group"
    assert o.f16_to_f32(sm[0, 0, 1]) == _f16(0.3)
    assert np.all(o.q4_dequant(qs, sm, 512)[0, :256] == np.float64(_f16(0.3)))
    want = np.where(np.arange(256) % 3 == 0, 0, 15)
    assert np.array_equal(c[256:], want), "two-valued group"


def pin_pack_ties_golden(o):
    g = _golden("pack_ties.txt")
    tie = [(q + 0.5) * 0.0625 for q in range(14)]
    rest = [(j % 16) * 0.0625 for j in range(256 - 2 - 14)]
    W = np.array([0.0, 0.9375] + tie + rest, dtype=np.float32)[None, :]
    qs, sm = o.q4_pack(W)
    c = o.q4_codes(qs, 256)[0]
    assert o.f16_to_f32(sm[0, 0, 0]) == float(g["scale"][0])
    assert np.array_equal(c[2:16], np.array(g["tie_codes"], dtype=int)), "RNE ties"
    assert np.array_equal(c[16:], np.arange(256 - 16) % 16)


def pin_pack_nearest_level(o):
    rng = np.random.default_rng(2)
    W = (rng.standard_normal((16, 512)) * 0.02).astype(np.float32)
    qs, sm = o.q4_pack(W)
    c = o.q4_codes(qs, 512)
    for n in range(16):
        for g in range(2):
            s = float(o.f16_to_f32(sm[n, g, 0]))
            m = float(o.f16_to_f32(sm[n, g, 1]))
            levels = m + s * np.arange(16)
            w = W[n, g * 256:(g + 1) * 256].astype(np.float64)
            dist = np.abs(w[:, None] - levels[None, :])
            got = dist[np.arange(256), c[n, g * 256:(g + 1) * 256]]
            assert np.all(got <= dist.min(axis=1) + 1e-6 * s), "not the nearest level"


def pin_pack_error_bound(o):
    rng = np.random.default_rng(3)
    W = (rng.standard_normal((32, 768)) * 0.02).astype(np.float32)
    W[3] *= 1e-3
    W[4, :256] = 5.0 + rng.standard_normal(256).astype(np.float32)
    qs, sm = o.q4_pack(W)
    Wd = o.q4_dequant(qs, sm, 768)
    for n in range(32):
        for g in range(3):
            w = W[n, g * 256:(g + 1) * 256].astype(np.float64)
            s = float(o.f16_to_f32(sm[n, g, 0]))
            m = float(o.f16_to_f32(sm[n, g, 1]))
            s_true = (w.max() - w.min()) / 15.0
            bound = 0.5 * s * (1 + 1e-5) + abs(m - w.min()) + 15 * abs(s - s_true)
            err = np.abs(Wd[n, g * 256:(g + 1) * 256] - w)
            assert err.max() <= bound, (n, g, err.max(), bound)


def pin_pack_idempotent_and_pow2(o):
    rng = np.random.default_rng(4)
    W = (rng.standard_normal((24, 512)) * 0.02).astype(np.float32)
    qs, sm = o.q4_pack(W)
    c = o.q4_codes(qs, 512).reshape(24, 2, 256)
    full = (c.min(axis=2) == 0) & (c.max(axis=2) == 15)
    Wd = o.q4_dequant(qs, sm, 512)
    assert np.all(Wd.astype(np.float32).astype(np.float64) == Wd)
    qs2, sm2 = o.q4_pack(Wd.astype(np.float32))
    for n in range(24):
        for g in range(2):
            if full[n, g]:
                sl = slice(g * 128, (g + 1) * 128)
                assert np.array_equal(qs2[n, sl], qs[n, sl]) and np.array_equal(sm2[n, g], sm[n, g])
    assert full.mean() > 0.9
    for k in (-3, 5):
        qs3, sm3 = o.q4_pack((W * np.float32(2.0 ** k)).astype(np.float32))
        assert np.array_equal(qs3, qs), "codes are invariant under 2^k scaling"
        assert np.array_equal(o.f16_to_f32(sm3), o.f16_to_f32(sm) * np.float32(2.0 ** k))


# ---------------------------------------------------------------- Q8_1 ----

def pin_q8_ties_golden(o):
    g = _golden("q8_1_ties.txt")
    x = np.array(g["x"], dtype=np.float32)[None, :]
    qa, ds = o.q8_1_quantize(x)
    assert np.array_equal(qa[0], np.array(g["a"], dtype=np.int8)), "RNE ties"
    assert o.f16_to_f32(ds[0, 0, 0]) == float(g["d"][0])
    assert o.f16_to_f32(ds[0, 0, 1]) == float(g["s"][0])


def pin_q8_closed_form(o):
    rng = np.random.default_rng(5)
    x, c, d = grid_activations(rng, 6, 256)
    qa, ds = o.q8_1_quantize(x)
    assert np.array_equal(qa.astype(np.int64), c)
    assert np.array_equal(o.f16_to_f32(ds[..., 0]).astype(np.float64), d)
    sums = c.reshape(6, 8, 32).sum(axis=2)
    want = (d * sums).astype(np.float16).astype(np.float32)
    assert np.array_equal(o.f16_to_f32(ds[..., 1]), want)
    z = np.zeros((1, 64), dtype=np.float32)
    z[0, 32:] = -0.0
    qa, ds = o.q8_1_quantize(z)
    assert np.all(qa == 0) and np.all(ds == 0), "zero block: a = 0, d = +0, s = +0"


def pin_q8_nearest_and_bound(o):
    rng = np.random.default_rng(6)
    x = rng.standard_normal((8, 128)).astype(np.float32)
    x[2] *= np.float32(1e-4)
    x[3, :32] *= 300.0
    qa, ds = o.q8_1_quantize(x)
    for m in range(8):
        for b in range(4):
            xb = x[m, b * 32:(b + 1) * 32].astype(np.float64)
            df = float(o.f16_to_f32(ds[m, b, 0]))
            a = qa[m, b * 32:(b + 1) * 32].astype(np.float64)
            cand = np.arange(-127, 128)
            dist = np.abs(xb[:, None] - df * cand[None, :])
            got = np.abs(xb - df * a)
            assert np.all(got <= dist.min(axis=1) + 1e-6 * df), "not the nearest code"
            amax = np.abs(xb).max()
            assert got.max() <= 0.5 * df * (1 + 1e-6) + max(0.0, amax - 127 * df)
            assert df == float(np.float16(np.float32(amax) / np.float32(127.0)))


def pin_q8_pow2(o):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((4, 256)).astype(np.float32)
    qa, ds = o.q8_1_quantize(x)
    for k in (-4, 3):
        qa2, ds2 = o.q8_1_quantize(x * np.float32(2.0 ** k))
        assert np.array_equal(qa2, qa)
        assert np.array_equal(o.f16_to_f32(ds2), o.f16_to_f32(ds) * np.float32(2.0 ** k))


# ---------------------------------------------------------- block dots ----

def pin_dots_closed_form(o):
    rng = np.random.default_rng(8)
    W, cw, _, _ = grid_weights(rng, 7, 512)
    x, ca, _ = grid_activations(rng, 3, 512)
    qs, _ = o.q4_pack(W)
    qa, _ = o.q8_1_quantize(x)
    got = o.q4_block_dots(qa, qs, 512)
    want = np.einsum("mbk,nbk->mnb", ca.reshape(3, 16, 32), cw.reshape(7, 16, 32))
    assert np.array_equal(got.astype(np.int64), want)


def pin_dots_all_code_pairs(o):
    # every int8 code -127..127 against every 4-bit code 0..15 on one block
    a = np.repeat(np.arange(-127, 128, dtype=np.int8)[:, None], 256, axis=1)
    codes = np.repeat(np.arange(16)[:, None], 256, axis=1)
    codes[:, 0] = 0
    codes[:, 1] = 15
    W = (-1.0 + 0.125 * codes).astype(np.float32)
    qs, _ = o.q4_pack(W)
    got = o.q4_block_dots(a, qs, 256)[:, :, 0].astype(np.int64)
    av = np.arange(-127, 128)[:, None]
    want = av * (0 + 15 + 30 * np.arange(16)[None, :])
    assert np.array_equal(got, want)
    assert got.min() == -127 * 15 * 31 + 0 and np.abs(got).max() <= 60960


# ---------------------------------------------------------------- GEMV ----

def pin_gemv_one_hot_and_group_sum(o):
    rng = np.random.default_rng(9)
    W, _, _, _ = grid_weights(rng, 6, 768)
    qs, sm = o.q4_pack(W)
    ks = [0, 1, 15, 16, 17, 31, 32, 255, 256, 300, 767]
    x = np.zeros((len(ks), 768), dtype=np.float32)
    x[np.arange(len(ks)), ks] = 1.0
    y = o.q4_gemv(x, qs, sm, 768)
    assert np.array_equal(y, W[:, ks].T.astype(np.float64)), "one-hot x picks column k"
    x = np.zeros((3, 768), dtype=np.float32)
    for g in range(3):
        x[g, g * 256:(g + 1) * 256] = 1.0
    y = o.q4_gemv(x, qs, sm, 768)
    want = W.astype(np.float64).reshape(6, 3, 256).sum(axis=2).T
    assert np.allclose(y, want, rtol=0, atol=1e-12)


def pin_gemv_exact_grid_vs_matmul(o):
    rng = np.random.default_rng(10)
    W, _, _, _ = grid_weights(rng, 40, 1280)
    x = rng.standard_normal((3, 1280)).astype(np.float32)
    qs, sm = o.q4_pack(W)
    y = o.q4_gemv(x, qs, sm, 1280)
    want = x.astype(np.float64) @ W.astype(np.float64).T
    assert np.allclose(y, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def pin_gemv_rows_and_linearity(o):
    rng = np.random.default_rng(12)
    W = (rng.standard_normal((20, 512)) * 0.02).astype(np.float32)
    qs, sm = o.q4_pack(W)
    x = rng.standard_normal((5, 512)).astype(np.float32)
    y = o.q4_gemv(x, qs, sm, 512)
    for m in range(5):
        assert np.array_equal(o.q4_gemv(x[m:m + 1], qs, sm, 512)[0], y[m])
    # disjoint supports and power-of-two weights keep x2 exact in fp32
    even = (np.arange(512) % 2 == 0)
    xa = np.where(even, x[0], 0).astype(np.float32)
    xb = np.where(even, 0, x[1]).astype(np.float32)
    x2 = (2 * xa - 0.5 * xb).astype(np.float32)
    ya, yb, y2 = o.q4_gemv(np.stack([xa, xb, x2]), qs, sm, 512)
    assert np.allclose(y2, 2.0 * ya - 0.5 * yb, rtol=0, atol=1e-12)
    assert np.allclose(ya + yb, o.q4_gemv(xa[None] + xb[None], qs, sm, 512)[0], rtol=0, atol=1e-12)


# ----------------------------------------------------------------- MMQ ----

def pin_mmq_exact_grid_vs_matmul(o):
    rng = np.random.default_rng(13)
    W, _, _, _ = grid_weights(rng, 9, 768)
    x, _, _ = grid_activations(rng, 4, 768)
    qs, sm = o.q4_pack(W)
    qa, ds = o.q8_1_quantize(x)
    y = o.q4_mmq(qa, ds, qs, sm, 768)
    want = x.astype(np.float64) @ W.astype(np.float64).T
    assert np.allclose(y, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def pin_mmq_matches_gemv_on_dequantized_x(o):
    rng = np.random.default_rng(14)
    W = (rng.standard_normal((11, 512)) * 0.02).astype(np.float32)
    x = rng.standard_normal((3, 512)).astype(np.float32)
    qs, sm = o.q4_pack(W)
    qa, ds = o.q8_1_quantize(x)
    xd = o.q8_1_dequant(qa, ds)
    assert np.all(xd.astype(np.float32).astype(np.float64) == xd)
    y1 = o.q4_mmq(qa, ds, qs, sm, 512)
    y2 = o.q4_gemv(xd.astype(np.float32), qs, sm, 512)
    assert np.array_equal(y1, y2)


def pin_mmq_unit_scales_sum_block_dots(o):
    # scale 1, minimum 0, d = 1: y is the sum over blocks of the integer dots
    rng = np.random.default_rng(15)
    codes = rng.integers(0, 16, size=(5, 512))
    codes[:, ::256] = 0
    codes[:, 1::256] = 15
    W = codes.astype(np.float32)
    c = rng.integers(-127, 128, size=(4, 512))
    c[:, ::32] = 127
    x = c.astype(np.float32)
    qs, sm = o.q4_pack(W)
    qa, ds = o.q8_1_quantize(x)
    assert np.all(o.f16_to_f32(sm[..., 0]) == 1) and np.all(sm[..., 1] == 0)
    assert np.all(o.f16_to_f32(ds[..., 0]) == 1)
    y = o.q4_mmq(qa, ds, qs, sm, 512)
    dots = o.q4_block_dots(qa, qs, 512).sum(axis=2)
    assert np.array_equal(y, dots.astype(np.float64))


# ------------------------------------------------------------ group 32 ----
# The group-32 variant keeps the code bytes and carries a (scale, minimum)
# pair per 32 weights.

def pin_g32_closed_form(o):
    rng = np.random.default_rng(21)
    W, codes, sf, mf = grid_weights(rng, 5, 512, group=32)
    qs, sm = o.q4_pack(W, group=32)
    assert sm.shape == (5, 16, 2)
    assert np.array_equal(o.q4_codes(qs, 512), codes), "codes of an exact grid"
    assert np.array_equal(o.f16_to_f32(sm[..., 0]), sf.astype(np.float32))
    assert np.array_equal(o.f16_to_f32(sm[..., 1]), mf.astype(np.float32))
    assert np.array_equal(o.q4_dequant(qs, sm, 512, group=32), W.astype(np.float64))


def pin_g32_same_bytes_as_g256(o):
    # a group-256 grid whose every run of 32 holds codes 0 and 15: both group
    # sizes find the same codes, so the code bytes agree and every run of 32
    # carries its group's pair
    rng = np.random.default_rng(22)
    W, codes, sf, mf = grid_weights(rng, 4, 512)
    for n in range(4):
        for r in range(16):
            i0, i1 = rng.choice(32, size=2, replace=False)
            codes[n, 32 * r + i0], codes[n, 32 * r + i1] = 0, 15
    W = (np.repeat(mf, 256, axis=1) + np.repeat(sf, 256, axis=1) * codes).astype(np.float32)
    qs256, sm256 = o.q4_pack(W)
    qs32, sm32 = o.q4_pack(W, group=32)
    assert np.array_equal(qs32, qs256)
    assert np.array_equal(sm32, np.repeat(sm256, 8, axis=1))


def pin_g32_nearest_level_and_constant_run(o):
    rng = np.random.default_rng(23)
    W = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    W[2, 64:96] = np.float32(0.01)  # one constant run of 32
    qs, sm = o.q4_pack(W, group=32)
    c = o.q4_codes(qs, 256)
    for n in range(8):
        for g in range(8):
            s = float(o.f16_to_f32(sm[n, g, 0]))
            m = float(o.f16_to_f32(sm[n, g, 1]))
            levels = m + s * np.arange(16)
            w = W[n, g * 32:(g + 1) * 32].astype(np.float64)
            dist = np.abs(w[:, None] - levels[None, :])
            got = dist[np.arange(32), c[n, g * 32:(g + 1) * 32]]
            assert np.all(got <= dist.min(axis=1) + 1e-6 * max(s, 1e-30)), "not the nearest level"
    assert sm[2, 2, 0] == 0 and np.all(c[2, 64:96] == 0)
    assert np.all(o.q4_dequant(qs, sm, 256, group=32)[2, 64:96] == np.float64(_f16(0.01)))


def pin_g32_gemv_and_mmq_exact_grid(o):
    rng = np.random.default_rng(24)
    W, _, _, _ = grid_weights(rng, 7, 768, group=32)
    qs, sm = o.q4_pack(W, group=32)
    x = rng.standard_normal((3, 768)).astype(np.float32)
    y = o.q4_gemv(x, qs, sm, 768, group=32)
    want = x.astype(np.float64) @ W.astype(np.float64).T
    assert np.allclose(y, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())
    ks = [0, 31, 32, 33, 100, 767]
    e = np.zeros((len(ks), 768), dtype=np.float32)
    e[np.arange(len(ks)), ks] = 1.0
    assert np.array_equal(o.q4_gemv(e, qs, sm, 768, group=32), W[:, ks].T.astype(np.float64))
    xg, _, _ = grid_activations(rng, 4, 768)
    qa, ds = o.q8_1_quantize(xg)
    y = o.q4_mmq(qa, ds, qs, sm, 768, group=32)
    want = xg.astype(np.float64) @ W.astype(np.float64).T
    assert np.allclose(y, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())


def pin_g32_equal_runs_reduce_to_g256(o):
    # pairs repeated over the eight runs of each group give the group-256 results
    rng = np.random.default_rng(25)
    W = (rng.standard_normal((9, 512)) * 0.02).astype(np.float32)
    qs, sm = o.q4_pack(W)
    sm32 = np.repeat(sm, 8, axis=1)
    x = rng.standard_normal((2, 512)).astype(np.float32)
    assert np.array_equal(o.q4_gemv(x, qs, sm32, 512, group=32), o.q4_gemv(x, qs, sm, 512))
    qa, ds = o.q8_1_quantize(x)
    assert np.array_equal(o.q4_mmq(qa, ds, qs, sm32, 512, group=32), o.q4_mmq(qa, ds, qs, sm, 512))


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_threads_do_not_change_results(orc):
    rng = np.random.default_rng(16)
    W = (rng.standard_normal((37, 512)) * 0.02).astype(np.float32)
    x = rng.standard_normal((3, 512)).astype(np.float32)
    old = orc.get_threads()
    try:
        orc.set_threads(1)
        qs1, sm1 = orc.q4_pack(W)
        y1 = orc.q4_gemv(x, qs1, sm1, 512)
        orc.set_threads(7)
        qs7, sm7 = orc.q4_pack(W)
        y7 = orc.q4_gemv(x, qs7, sm7, 512)
    finally:
        orc.set_threads(old)
    assert np.array_equal(qs1, qs7) and np.array_equal(sm1, sm7) and np.array_equal(y1, y7)


MUTATIONS = list(range(1, 11))


@pytest.mark.parametrize("mut", MUTATIONS)
def test_mutations_are_caught(orc, mut):
    failed = []
    orc.set_mutation(mut)
    try:
        assert orc.get_mutation() == mut
        for pin in ALL_PINS:
            try:
                pin(orc)
            except AssertionError:
                failed.append(pin.__name__)
    finally:
        orc.set_mutation(0)
    assert failed, "planted mistake %d passed every pin" % mut
