"""Pins of the oracle's hand-written fp16 <-> fp32 conversions.

Both directions are checked against numpy's own binary16 conversion (an
independent implementation of IEEE-754 round-to-nearest-even): exhaustively
for fp16 -> fp32, and on special values plus a large random sample for
fp32 -> fp16.
"""
import numpy as np


def test_h2f_exhaustive(orc):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.h2f(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _check_f2h(orc, f):
    f = np.ascontiguousarray(f, np.float32)
    got = orc.f2h(f)
    with np.errstate(over="ignore", invalid="ignore"):
        ref = f.astype(np.float16).view(np.uint16)
    nan = np.isnan(f)
    assert np.all((got[nan] & 0x7C00) == 0x7C00) and np.all((got[nan] & 0x3FF) != 0)
    bad = np.nonzero(got[~nan] != ref[~nan])[0]
    assert bad.size == 0, (f[~nan][bad[:5]], got[~nan][bad[:5]], ref[~nan][bad[:5]])


def test_f2h_special_values(orc):
    vals = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.996, 65520.0, 65536.0, 1e30, -1e30,
            np.inf, -np.inf, np.nan, 2.0 ** -14, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26,
            2.0 ** -25 * 1.0000001, 2.0 ** -26, 1e-45, 6.1e-5, 6.0975552e-05,
            1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 2049.0, 2051.0, 0.1, 1 / 3.0]
    _check_f2h(orc, np.array(vals + [-v for v in vals], np.float32))


def test_f2h_every_halfway_point(orc):
    # every fp16 value and every midpoint between neighbours (ties-to-even cases)
    h = np.arange(0, 0x7C00, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)
    _check_f2h(orc, np.concatenate([lo.astype(np.float32), mid, -mid,
                                    np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(np.inf))]))


def test_f2h_random_bit_patterns(orc):
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    _check_f2h(orc, bits.view(np.float32))
    _check_f2h(orc, rng.standard_normal(2_000_000).astype(np.float32) * 100)
