"""The reciprocal rule behind the device Q8_1 codes.

Q8_1 quantization fixes each code as clamp(rint(x / d), -127, 127), with the
quotient rounded once as IEEE fp32 division rounds it and d an fp16 block
scale (hipfire MMQ note, list of changes: activations pre-quantized to Q8_1
blocks of 32 with an fp16 scale).  The kernels multiply by the hardware
reciprocal of d (within one ulp of 1/d) and divide exactly only when the
product lies within 2^-11 of a half-integer.  This CPU model of that decision
(numpy fp32, round to nearest even; every reciprocal within one ulp of the
correctly rounded 1/d is tried) must give the correctly rounded code on
random quotients, on exact and near ties, on clamped quotients and across the
fp16 range of d.  The GPU parity tests then hold the kernels' codes to the
oracle's bit for bit.  The model shares no code with the kernels or the
oracle.
"""
import numpy as np

MARGIN = np.float32(2.0 ** -11)


def exact_codes(x, d):
    q = np.float32(x) / np.float32(d)
    return np.clip(np.rint(q), -127, 127)


def rule_codes(x, d, rdf, margin=MARGIN):
    q = (x * rdf).astype(np.float32)
    n = np.rint(q)
    near = ~(np.abs(np.abs(q - n) - np.float32(0.5)) > margin)
    r = np.where(near, np.rint(x / d), n)
    return np.clip(r, -127, 127), near


def reciprocals(d):
    r0 = (np.float32(1.0) / d).astype(np.float32)
    return [np.nextafter(r0, np.float32(0.0)), r0, np.nextafter(r0, np.float32(np.inf))]


def fp16_scales(rng, n):
    """fp16 block scales over the normal and subnormal range, as fp32."""
    bits = rng.integers(1, 0x7BFF, size=n, dtype=np.uint16)
    return bits.view(np.float16).astype(np.float32)


def cases(rng):
    n = 200_000
    d = fp16_scales(rng, n)
    # random quotients inside the code range and beyond it
    u = rng.uniform(-1.0, 1.0, n)
    yield "random", (u * 127.0 * d).astype(np.float32), d
    yield "wide", (u * 1e6 * d).astype(np.float32), d
    # quotients at and around every half-integer, down to one fp32 ulp away
    k = rng.integers(-128, 128, n).astype(np.float64)
    delta = np.where(rng.integers(0, 2, n) == 0, -1.0, 1.0) * np.ldexp(1.0, -rng.integers(8, 26, n))
    delta[rng.integers(0, 4, n) == 0] = 0.0
    yield "near-ties", ((k + 0.5 + delta) * d.astype(np.float64)).astype(np.float32), d
    # exact ties with power-of-two scales (x / d exact in fp32)
    d2 = np.ldexp(np.float32(1.0), rng.integers(-24, 15, n)).astype(np.float32)
    yield "ties", ((k + 0.5) * d2).astype(np.float32), d2
    # a block whose largest value sets d: the quotients of the largest value
    # sit next to 127
    amax = np.abs(rng.normal(size=n)).astype(np.float32) * np.float32(2.0) ** rng.integers(-20, 20, n)
    d3 = (amax / np.float32(127.0)).astype(np.float16).astype(np.float32)
    ok = d3 > 0
    yield "amax", amax[ok], d3[ok]


def test_rule_matches_correctly_rounded_division():
    rng = np.random.default_rng(11)
    for name, x, d in cases(rng):
        want = exact_codes(x, d)
        for rdf in reciprocals(d):
            got, _ = rule_codes(x, d, rdf)
            bad = np.flatnonzero(got != want)
            assert bad.size == 0, (name, x[bad[:4]], d[bad[:4]])


def test_rule_divides_rarely_on_random_quotients():
    rng = np.random.default_rng(12)
    d = fp16_scales(rng, 100_000)
    x = (rng.uniform(-1.0, 1.0, d.size) * 127.0 * d).astype(np.float32)
    _, near = rule_codes(x, d, reciprocals(d)[1])
    assert near.mean() < 0.01


def test_rule_without_its_exact_fallback_fails():
    """Planted mistake: no exact division near half-integers.  The tie cases
    must catch it (a reciprocal one ulp off moves exact ties)."""
    rng = np.random.default_rng(13)
    caught = False
    for name, x, d in cases(rng):
        want = exact_codes(x, d)
        for rdf in reciprocals(d):
            got, _ = rule_codes(x, d, rdf, margin=np.float32(-1.0))
            caught |= bool(np.any(got != want))
    assert caught
