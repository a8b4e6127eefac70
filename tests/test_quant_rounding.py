"""The quantizing kernels round x / s to an integer from x * rcp(s) and fall
back to the correctly rounded division only within 2^-13 of a half-integer.
This checks that rule on the CPU, in float32, with the reciprocal off by up
to one unit in the last place either way (the hardware reciprocal's bound):
the fast rule must give rint(fl32(x / s)) (ties to even) everywhere the
kernels use it (|x / s| < 300, s an fp16 value)."""

import numpy as np

F32 = np.float32


def fast_rint_div(x, s, rcp):
    q = (x * rcp).astype(F32)
    c = np.rint(q)
    slow = np.abs(q - c) > F32(0.5 - 2.0 ** -13)
    return np.where(slow, np.rint((x / s).astype(F32)), c)


def exact_rint_div(x, s):
    return np.rint((x / s).astype(F32))


def fp16_scales(rng, n):
    """Positive fp16 values over the whole range, subnormals included."""
    bits = rng.integers(1, 0x7C00, size=n, dtype=np.uint16)
    return bits.view(np.float16).astype(F32)


def check(x, s):
    r0 = (F32(1.0) / s).astype(F32)
    for rcp in (np.nextafter(r0, F32(0)), r0, np.nextafter(r0, F32(np.inf))):
        got = fast_rint_div(x, s, rcp)
        want = exact_rint_div(x, s)
        bad = got != want
        assert not bad.any(), (x[bad][:5], s[bad][:5])


def test_random_quotients():
    rng = np.random.default_rng(11)
    s = fp16_scales(rng, 400_000)
    x = (rng.uniform(-300, 300, size=s.size) * s).astype(F32)
    keep = np.abs(x / s) < 300
    check(x[keep], s[keep])


def test_quotients_at_and_next_to_half_integers():
    """Exact ties (x = (k + 1/2) s when representable) and the float32
    neighbours of them on both sides, where the fast rule must hand over."""
    rng = np.random.default_rng(12)
    s = fp16_scales(rng, 200_000)
    k = rng.integers(-255, 255, size=s.size)
    x0 = ((k + 0.5) * s.astype(np.float64)).astype(F32)
    xs = [x0]
    for _ in range(3):
        xs.append(np.nextafter(xs[-1], F32(np.inf)))
    lo = [x0]
    for _ in range(3):
        lo.append(np.nextafter(lo[-1], F32(-np.inf)))
    x = np.concatenate(xs + lo[1:])
    ss = np.tile(s, 7)
    keep = (np.abs(x / ss) < 300) & np.isfinite(x)
    check(x[keep], ss[keep])


def test_quantizer_shapes_of_quotient():
    """The quotients the quantizers form: k / fp16(amax / 127) and
    (v - z) / fp16((max - min) / 15) over random rows."""
    rng = np.random.default_rng(13)
    for scale in (1e-3, 1.0, 30.0):
        k = (rng.standard_normal((20_000, 128)) * scale).astype(F32)
        amax = np.abs(k).max(axis=1)
        s = (amax / F32(127)).astype(F32).astype(np.float16).astype(F32)
        ok = s > 0
        kk, ss = k[ok], np.broadcast_to(s[ok, None], k[ok].shape)
        check(kk.reshape(-1), np.ascontiguousarray(ss).reshape(-1))
        v = (rng.standard_normal((20_000, 32)) * scale).astype(F32)
        mn, mx = v.min(axis=1), v.max(axis=1)
        s = ((mx - mn) / F32(15)).astype(F32).astype(np.float16).astype(F32)
        z = mn.astype(np.float16).astype(F32)
        d = (v - z[:, None]).astype(F32)
        ok = s > 0
        check(d[ok].reshape(-1), np.ascontiguousarray(np.broadcast_to(s[ok, None], d[ok].shape)).reshape(-1))
