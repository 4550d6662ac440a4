"""Pins of the oracle's packed KIVI storage (oracle.kivi_pack / kivi_unpack).

["veloxquant_mlx.cache.kivi_cache", module docstring: per-token storage at
bit-width b and group size g is b-bit codes plus an fp16 (scale, zero) pair
per group; _quantized_bytes] The group math is the page's
_quant_dequant_along with the pair rounded to fp16 before use. Pinned here
by:
  - reduction to the pinned binary32 round trip (oracle.kivi_round_trip)
    wherever every group's binary32 scale is itself an fp16 value;
  - a closed-form error bound on random data;
  - exact cases: the group minimum reconstructs exactly, a constant group
    gives codes 0 and the smallest positive fp16 scale;
  - the stored scale is (max - min)/levels rounded down to fp16 (within one
    step below it), so no reconstruction leaves its group's [min, max];
  - flush chunking independence and the page's byte formula.
"""
import math

import numpy as np
import pytest

import oracle

EPS = 1e-8


def f16(a):
    return np.asarray(a, np.float16).view(np.uint16)


def val(u):
    return np.asarray(u, np.uint16).view(np.float16).astype(np.float64)


def ulp16(x):
    """Spacing of fp16 at |x| (subnormal spacing below 2^-14)."""
    a = np.maximum(np.abs(x), 2.0 ** -14)
    return 2.0 ** (np.floor(np.log2(a)) - 10)


def _grid_keys(rng, B, H, S, D, bits, gs):
    """Keys whose every (channel, group) has min m and max m + levels*2^-4
    (both fp16), the rest fp16 values in between: the binary32 scale is 2^-4."""
    lev = (1 << bits) - 1
    x = np.zeros((B, H, S, D), np.float64)
    for g0 in range(0, S, gs):
        m = rng.integers(-40, 40, size=(B, H, 1, D)) * 2.0 ** -4
        span = lev * 2.0 ** -4
        blk = m + rng.integers(0, lev * 4 + 1, size=(B, H, min(gs, S - g0), D)) * 2.0 ** -6
        blk[:, :, 0] = m[:, :, 0]
        if blk.shape[2] > 1:
            blk[:, :, 1] = m[:, :, 0] + span
        x[:, :, g0:g0 + gs] = blk
    return f16(x)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_keys_reduce_to_binary32_round_trip_on_fp16_scales(bits):
    rng = np.random.default_rng(bits)
    B, H, S, D, gs = 2, 2, 96, 16, 32
    x = _grid_keys(rng, B, H, S, D, bits, gs)
    codes, sc, zr = oracle.kivi_pack(x, 0, S, 1, bits, gs)
    rec, c32, s32, m32 = oracle.kivi_round_trip(x, 0, S, 1, bits, gs, want_params=True)
    assert np.array_equal(codes, c32)
    assert np.array_equal(sc, f16(s32))
    assert np.array_equal(zr, f16(m32))
    assert np.array_equal(oracle.kivi_unpack(codes, sc, zr, 0, S, 1, bits, gs, D), rec)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_values_reduce_to_binary32_round_trip_on_fp16_scales(bits):
    rng = np.random.default_rng(10 + bits)
    lev = (1 << bits) - 1
    B, H, S, D, gs = 1, 3, 40, 64, 32
    x = np.zeros((B, H, S, D))
    for g0 in range(0, D, gs):
        m = rng.integers(-40, 40, size=(B, H, S, 1)) * 2.0 ** -3
        blk = m + rng.integers(0, lev * 2 + 1, size=(B, H, S, gs)) * 2.0 ** -4
        blk[..., 0] = m[..., 0]
        blk[..., 1] = m[..., 0] + lev * 2.0 ** -3
        x[..., g0:g0 + gs] = blk
    x = f16(x)
    codes, sc, zr = oracle.kivi_pack(x, 5, 37, 0, bits, gs)
    rec, c32, s32, m32 = oracle.kivi_round_trip(x, 5, 37, 0, bits, gs, want_params=True)
    assert np.array_equal(codes[:, :, 5:37], c32)
    assert np.array_equal(sc[:, :, 5:37], f16(s32))
    assert np.array_equal(zr[:, :, 5:37], f16(m32))
    out = oracle.kivi_unpack(codes, sc, zr, 5, 37, 0, bits, gs, D)
    assert np.array_equal(out[:, :, 5:37], rec[:, :, 5:37])
    assert not out[:, :, :5].any() and not out[:, :, 37:].any()


def _groups(x, per_channel, gs, lo, hi):
    """(values float64 [..., gs], group index arrays) of the region, by axis."""
    B, H, S, D = x.shape
    out = []
    if per_channel:
        for t0 in range(lo, hi, gs):
            t1 = min(t0 + gs, hi)
            out.append((np.s_[:, :, t0:t1, :], t0 // gs, 2))
    else:
        for g0 in range(0, D, gs):
            out.append((np.s_[:, :, lo:hi, g0:min(g0 + gs, D)], g0 // gs, 3))
    return out


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("per_channel", [1, 0])
def test_error_bound_and_exact_minimum(bits, per_channel):
    """|x - recon| <= s/2 + levels*s*2^-10 + |x - min|*2^-22 + ulp16(recon)/2
    (nearest level up to the quotient's two roundings; the fp16 scale may sit
    below the binary32 one by 2^-11 relative, clamping the top; one fp16
    rounding of the reconstruction); the group minimum reconstructs exactly."""
    rng = np.random.default_rng(100 * bits + per_channel)
    B, H, S, D, gs = 2, 2, 128, 64, 32
    xf = rng.standard_normal((B, H, S, D)) * np.where(rng.random(D) < 0.06, 8.0, 1.0)
    x = f16(xf)
    lo, hi = 32, 128
    codes, sc, zr = oracle.kivi_pack(x, lo, hi, per_channel, bits, gs)
    out = oracle.kivi_unpack(codes, sc, zr, lo, hi, per_channel, bits, gs, D)
    lev = (1 << bits) - 1
    xv, rv = val(x), val(out)
    for sl, g, axis in _groups(x, per_channel, gs, lo, hi):
        xs, rs = xv[sl], rv[sl]
        if per_channel:
            s = val(sc[:, :, g])[:, :, None, :]
            z = val(zr[:, :, g])[:, :, None, :]
            mn = xs.min(axis=2, keepdims=True)
        else:
            s = val(sc[:, :, lo:hi, g])[..., None]
            z = val(zr[:, :, lo:hi, g])[..., None]
            mn = xs.min(axis=3, keepdims=True)
        assert np.array_equal(z + 0.0, mn + 0.0)  # zero = group minimum (fp16, exact)
        bound = s / 2 + lev * s * 2.0 ** -10 + np.abs(xs - mn) * 2.0 ** -22 + ulp16(rs) / 2
        assert np.all(np.abs(xs - rs) <= bound)
        at_min = xs == mn
        assert np.array_equal(rs[at_min], xs[at_min])


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_stored_scale_is_range_over_levels_rounded_down(bits):
    rng = np.random.default_rng(7 + bits)
    x = f16(rng.standard_normal((1, 2, 64, 64)) * 3)
    lev = (1 << bits) - 1
    _, sc, zr = oracle.kivi_pack(x, 0, 64, 0, bits, 32)
    xv = val(x)
    for g in range(2):
        grp = xv[..., 32 * g:32 * (g + 1)]
        exact = (grp.max(-1) - grp.min(-1)) / lev
        s = val(sc[..., g])
        assert np.all(s <= exact * (1 + 2.0 ** -23))  # never above (binary32 quotient aside)
        assert np.all(exact - s < ulp16(exact) + exact * 2.0 ** -23)  # within one fp16 step
        assert np.array_equal(val(zr[..., g]), grp.min(-1) + 0.0)


def test_constant_group_and_negative_zero():
    x = np.full((1, 1, 32, 16), 1.5)
    x[..., 8:] = -0.0
    x = f16(x)
    for per_channel in (1, 0):
        codes, sc, zr = oracle.kivi_pack(x, 0, 32, per_channel, 4, 8 if not per_channel else 32)
        assert not codes.any()
        assert np.all(sc[sc != 0] == 1)  # 2^-24: the eps floor rounded up to fp16's smallest step
        out = oracle.kivi_unpack(codes, sc, zr, 0, 32, per_channel, 4, 8 if not per_channel else 32, 16)
        assert np.array_equal(val(out), np.where(val(x) == 0, 0.0, val(x)))
        assert not (zr == 0x8000).any()  # -0 is stored as +0


@pytest.mark.parametrize("per_channel", [1, 0])
def test_reconstructions_stay_in_group_range(per_channel):
    rng = np.random.default_rng(21)
    x = f16(rng.standard_normal((2, 2, 64, 64)) * rng.choice([1e-3, 1, 300], size=(2, 2, 64, 64)))
    for bits in (2, 4, 8):
        codes, sc, zr = oracle.kivi_pack(x, 0, 64, per_channel, bits, 32)
        out = val(oracle.kivi_unpack(codes, sc, zr, 0, 64, per_channel, bits, 32, 64))
        for sl, g, axis in _groups(x, per_channel, 32, 0, 64):
            xs, rs = val(x)[sl], out[sl]
            assert np.all(rs >= xs.min(axis=axis, keepdims=True))
            assert np.all(rs <= xs.max(axis=axis, keepdims=True))


@pytest.mark.parametrize("per_channel", [1, 0])
def test_flush_chunking_independence(per_channel):
    """Packing [0, 96) at once equals packing [0, 32), [32, 64), [64, 96) into
    the same storage (group-aligned flushes, as the cache issues them)."""
    rng = np.random.default_rng(3)
    x = f16(rng.standard_normal((2, 2, 128, 32)))
    whole = oracle.kivi_pack(x, 0, 96, per_channel, 2, 32)
    parts = oracle.kivi_pack(x, 0, 32, per_channel, 2, 32)
    oracle.kivi_pack(x, 32, 64, per_channel, 2, 32, into=parts)
    oracle.kivi_pack(x, 64, 96, per_channel, 2, 32, into=parts)
    for a, b in zip(whole, parts):
        assert np.array_equal(a, b)


def test_b8_full_fp16_range():
    x = np.zeros((1, 1, 32, 32))
    x[..., 0] = -65504.0
    x[..., 1] = 65504.0
    x[..., 2:] = np.linspace(-60000, 60000, 30)
    x = f16(x)
    codes, sc, zr = oracle.kivi_pack(x, 0, 32, 0, 8, 32)
    out = val(oracle.kivi_unpack(codes, sc, zr, 0, 32, 0, 8, 32, 32))
    assert np.all(np.isfinite(out)) and out.max() <= 65504 and out.min() == -65504
    s = val(sc[..., 0])[..., None]
    assert np.all(np.abs(out - val(x)) <= s / 2 + 255 * s * 2.0 ** -10 + ulp16(out) / 2 + 131008 * 2.0 ** -22)


@pytest.mark.parametrize("bits,gs", [(2, 32), (4, 32), (8, 16)])
def test_storage_sizes_are_the_pages_byte_formula(bits, gs):
    """[kivi_cache, _quantized_bytes] keys: ceil(n*D*b/8) code bytes + ceil(n/g)*D
    (scale, zero) fp16 pairs per (b, h); values: the same codes + n*ceil(D/g)
    pairs. The packed arrays hold exactly that much for a flush of n tokens."""
    B, H, S, D, n = 2, 3, 96, 64, 64
    x = f16(np.random.default_rng(1).standard_normal((B, H, S, D)))
    kc, ks, kz = oracle.kivi_pack(x, 0, n, 1, bits, gs)
    vc, vs, vz = oracle.kivi_pack(x, 0, n, 0, bits, gs)
    code = kc[:, :, :n].nbytes
    kpar = ks[:, :, :math.ceil(n / gs)].nbytes + kz[:, :, :math.ceil(n / gs)].nbytes
    vpar = vs[:, :, :n].nbytes + vz[:, :, :n].nbytes
    k_page = math.ceil(n * D * bits / 8) * H * B + math.ceil(n / gs) * D * 2 * 2 * H * B
    v_page = math.ceil(n * D * bits / 8) * H * B + n * math.ceil(D / gs) * 2 * 2 * H * B
    assert code + kpar == k_page
    assert vc[:, :, :n].nbytes + vpar == v_page
