"""Error budget of the fp16 matrix-core design of the MMQ GEMM.

For shapes whose grid fills the GPU the MMQ runs on fp16 matrix cores: each
activation becomes x' = fp16(d * a * 2^f[m]) with one power of two per row
(f = 8 - e, e the binary exponent of the row's largest Q8_1 scale d), each
weight w' = fp16(q * s' + mn') with s' = scale * 2^E[n], mn' = minimum *
2^E[n] (E[n] = -6 - e', e' the binary exponent of the row's largest
|minimum| + 15 |scale|), the products are summed and y = sum / 2^(f + E).
This CPU model of that arithmetic (numpy fp16 conversions, round to nearest
even, subnormals kept; sums in fp64, where the GPU sums in fp32) is checked
against the oracle's exact fp64 sums on the prefill activation distributions
and at the edges of the exponent choices; the GPU parity tests then hold the
kernel to the oracle directly.  The model shares no code with the kernel or
the oracle; it reads the oracle's packed weights and Q8_1 codes as inputs.
"""
import numpy as np
import pytest

MAX_REL = 2e-3
MAX_NMSE = 1e-6


def _f16(h):
    return np.asarray(h, dtype=np.uint16).view(np.float16).astype(np.float64)


def _exponent(v):
    """e with v = f * 2^e, f in [0.5, 1); 0 where v == 0."""
    return np.where(v > 0, np.frexp(np.where(v > 0, v, 1.0))[1], 0)


def f16_design_model(qa, ds, codes, sm):
    """(y [M][N], x' [M][K], w' [N][K]) of the fp16 design from Q8_1 (qa int8
    [M][K], ds uint16 [M][K/32][2]), codes uint8 [N][K], sm uint16 [N][K/256][2]."""
    M, K = qa.shape
    d = np.repeat(_f16(ds[:, :, 0]), 32, axis=1)                  # [M][K]
    dmax = _f16(ds[:, :, 0]).max(axis=1)
    f = np.where(dmax > 0, 8 - _exponent(dmax), 0)
    xp = (d * qa.astype(np.float64) * np.ldexp(1.0, f)[:, None]).astype(np.float16)
    scale, minimum = _f16(sm[:, :, 0]), _f16(sm[:, :, 1])
    wmax = (np.abs(minimum) + 15 * np.abs(scale)).max(axis=1)
    E = np.where(wmax > 0, -6 - _exponent(wmax), 0)
    # the kernel's fp16 FMA operands: s' * 2^24 (the code enters as the fp16
    # subnormal q * 2^-24) and mn'; the sum q * s' + mn' is rounded once
    S = (scale * np.ldexp(1.0, E + 24)[:, None]).astype(np.float16).astype(np.float64)
    MN = (minimum * np.ldexp(1.0, E)[:, None]).astype(np.float16).astype(np.float64)
    q = codes.astype(np.float64)
    wp = (q * np.repeat(S, 256, axis=1) * 2.0 ** -24 + np.repeat(MN, 256, axis=1)).astype(np.float16)
    acc = xp.astype(np.float64) @ wp.astype(np.float64).T
    y = acc * np.ldexp(1.0, -f)[:, None] * np.ldexp(1.0, -E)[None, :]
    return y, xp, wp


def _run(orc, W, x):
    K = W.shape[1]
    qs, sm = orc.q4_pack(W.astype(np.float32))
    qa, ds = orc.q8_1_quantize(x.astype(np.float32))
    ref = orc.q4_mmq(qa, ds, qs, sm, K)
    y, xp, wp = f16_design_model(qa, ds, orc.q4_codes(qs, K), sm)
    return y, ref, xp, wp


def _measures(y, ref):
    err = y - ref
    den = np.abs(ref).max()
    return (err ** 2).sum() / (ref ** 2).sum(), np.abs(err).max() / den


@pytest.mark.parametrize("seed,kind", [(30, "normal"), (31, "outliers20"), (32, "outliers1000")])
def test_f16_design_error_budget(orc, seed, kind):
    rng = np.random.default_rng(seed)
    M, N, K = 48, 80, 1024
    x = rng.standard_normal((M, K))
    if kind != "normal":
        amp = 20.0 if kind == "outliers20" else 1000.0
        x = np.where(rng.random((M, K)) < 0.01, x * amp, x)
    W = 0.02 * rng.standard_normal((N, K))
    y, ref, xp, wp = _run(orc, W, x)
    nmse, rel = _measures(y, ref)
    # fp16 operands: about 2^-12 rms relative error each
    assert nmse < 3e-7, nmse
    assert rel < 1e-3, rel
    assert nmse > 1e-9  # the model does round: a plain fp64 sum would not


def test_f16_design_operand_ranges(orc):
    # the exponent choices keep every operand finite: |x'| < 2^15 with the
    # largest of each row at least 2^13, |w'| <= 2^-6 with each row's bound
    # in [2^-7, 2^-6)
    rng = np.random.default_rng(33)
    M, N, K = 16, 24, 512
    x = rng.standard_normal((M, K)) * np.logspace(-6, 4.5, M)[:, None]
    W = 0.02 * rng.standard_normal((N, K)) * np.logspace(-4, 5, N)[:, None]
    y, ref, xp, wp = _run(orc, W, x)
    ax = np.abs(xp.astype(np.float64))
    assert np.isfinite(ax).all() and ax.max() < 2 ** 15
    live = ax.max(axis=1) > 0  # the 1e-6 row quantizes to zero in Q8_1 (d below fp16's range)
    assert live.sum() >= M - 1 and (ax.max(axis=1)[live] >= 2 ** 13).all()
    aw = np.abs(wp.astype(np.float64))
    assert np.isfinite(aw).all() and aw.max() <= 2 ** -6
    # every (row, weight row) pair on a common scale: divide out each row's
    # and each weight row's magnitude, then measure all entries together
    rs = np.abs(x).max(axis=1)[live][:, None]
    cs = np.abs(W).max(axis=1)[None, :]
    nmse, rel = _measures(y[live] / rs / cs, ref[live] / rs / cs)
    assert nmse <= MAX_NMSE and rel <= MAX_REL, (nmse, rel)


def test_f16_design_degenerate_groups(orc):
    # zero activation rows, one live block, a huge block beside an
    # fp16-subnormal one, spikes; constant, zero and offset weight groups
    rng = np.random.default_rng(34)
    M, N, K = 8, 40, 1024
    x = rng.standard_normal((M, K))
    x[0] = 0.0
    x[1] = 0.0
    x[1, 40:72] = rng.standard_normal(32)
    x[2, :32] = 3e4
    x[2, 32:64] = rng.standard_normal(32) * 1e-6
    x[3, ::256] = -7e3
    W = 0.02 * rng.standard_normal((N, K))
    W[0, :256] = 0.125
    W[1] = -0.5
    W[2] = 0.0
    W[3, 256:512] = 3.0
    y, ref, xp, wp = _run(orc, W, x)
    assert (y[0] == 0).all() and (y[:, 2] == 0).all()
    nmse, rel = _measures(y, ref)
    assert nmse <= MAX_NMSE and rel <= MAX_REL, (nmse, rel)
    for r in (1, 2, 3):
        nmse, rel = _measures(y[r], ref[r])
        assert nmse <= MAX_NMSE and rel <= MAX_REL, (r, nmse, rel)


def test_f16_rounding_is_the_error(orc):
    # with the fp16 roundings taken out (the same scaling in fp64) the model
    # reproduces the oracle to fp64 precision: the exponent bookkeeping is
    # exact and only the two fp16 roundings move the result
    rng = np.random.default_rng(35)
    M, N, K = 12, 20, 512
    x = rng.standard_normal((M, K))
    W = 0.02 * rng.standard_normal((N, K))
    qs, sm = orc.q4_pack(W.astype(np.float32))
    qa, ds = orc.q8_1_quantize(x.astype(np.float32))
    ref = orc.q4_mmq(qa, ds, qs, sm, K)
    codes = orc.q4_codes(qs, K)
    d = np.repeat(_f16(ds[:, :, 0]), 32, axis=1)
    dmax = _f16(ds[:, :, 0]).max(axis=1)
    f = np.where(dmax > 0, 8 - _exponent(dmax), 0)
    scale, minimum = _f16(sm[:, :, 0]), _f16(sm[:, :, 1])
    wmax = (np.abs(minimum) + 15 * np.abs(scale)).max(axis=1)
    E = np.where(wmax > 0, -6 - _exponent(wmax), 0)
    xe = d * qa * np.ldexp(1.0, f)[:, None]
    we = (codes * np.repeat(scale, 256, axis=1) + np.repeat(minimum, 256, axis=1)) * np.ldexp(1.0, E)[:, None]
    y = (xe @ we.T) * np.ldexp(1.0, -f)[:, None] * np.ldexp(1.0, -E)[None, :]
    assert np.abs(y - ref).max() <= 1e-12 * np.abs(ref).max()
