"""Pins of the oracle's KIVI asymmetric group round trip.

Source: "veloxquant_mlx.cache.kivi_cache" module source -- the module
docstring (keys per channel, values per token, fp16 residual window,
determinism, the residual bound) and KIVIKVCache._quant_dequant_along /
_quantization_boundary. The pins use properties the pages state or the
definition forces: grid-aligned data round-trips exactly (this fails if
groups are cut in the wrong place or along the wrong axis), a group's minimum
is reproduced exactly, codes stay in [0, 2^b-1], the eps floor on the scale,
the single-element-group degenerate case the page describes, determinism,
independence of how tokens were chunked, and the residual-window bound.
"""
import numpy as np
import pytest

EPS = np.float32(1e-8)


def _bases(rng, shape, axis, m):
    """Group base offsets on a (m+5)-spaced grid, neighbours along the group
    axis always different, all values exact in fp16 after the 2^-4 scaling."""
    K = 2047 // (m + 5) - 1
    idx = rng.integers(0, K, size=shape)
    idx = np.moveaxis(idx, axis, 0)
    for g in range(1, idx.shape[0]):
        same = idx[g] == idx[g - 1]
        idx[g][same] = (idx[g][same] + 1) % K
    return np.moveaxis(idx, 0, axis) * (m + 5)


def _grid(rng, B, H, S, D, lo, hi, gs, bits, per_channel):
    """Data whose every KIVI group is {base_g + 0..m} with both ends present."""
    m = (1 << bits) - 1
    x = np.zeros((B, H, S, D), np.float64)
    x[:] = rng.standard_normal(x.shape)  # outside [lo, hi): must stay untouched
    sl = x[:, :, lo:hi, :]
    n = hi - lo
    if per_channel:
        ng = (n + gs - 1) // gs
        base = _bases(rng, (B, H, ng, D), 2, m)
        gidx = np.arange(n) // gs
        b = base[:, :, gidx, :]  # [B,H,n,D]
        off = rng.integers(0, m + 1, size=sl.shape)
        for g in range(ng):
            t0, t1 = g * gs, min(g * gs + gs, n)
            off[:, :, t0, :] = 0
            off[:, :, t1 - 1, :] = m if t1 - t0 > 1 else 0
    else:
        ng = (D + gs - 1) // gs
        base = _bases(rng, (B, H, n, ng), 3, m)
        gidx = np.arange(D) // gs
        b = base[:, :, :, gidx]
        off = rng.integers(0, m + 1, size=sl.shape)
        for g in range(ng):
            d0, d1 = g * gs, min(g * gs + gs, D)
            off[:, :, :, d0] = 0
            off[:, :, :, d1 - 1] = m if d1 - d0 > 1 else 0
    sl[:] = (b + off) * 2.0 ** -4  # exact in fp16 while < 2048 * 2^-4
    assert np.abs(sl).max() < 128
    return x.astype(np.float16), off


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("per_channel", [1, 0])
def test_grid_data_roundtrips_exactly(orc, bits, per_channel):
    rng = np.random.default_rng(bits * 10 + per_channel)
    B, H, S, D, gs = 2, 3, 120, 40, 8       # n = 101 tokens: ragged last key group
    lo, hi = 5, 106
    if not per_channel:
        D = 44                               # ragged channel tail for values
    x, off = _grid(rng, B, H, S, D, lo, hi, gs, bits, per_channel)
    rec, codes, scale, mn = orc.kivi_round_trip(x.view(np.uint16), lo, hi, per_channel, bits, gs,
                                                want_params=True)
    assert np.array_equal(rec, x.view(np.uint16))  # exact, including untouched rows
    assert np.all(scale == np.float32(2.0 ** -4))
    # packed codes (LSB-first along D) unpack to the grid offsets
    cb = np.unpackbits(codes, axis=-1, bitorder="little")[..., : D * bits]
    c = (cb.reshape(*cb.shape[:-1], D, bits) * (1 << np.arange(bits))).sum(-1)
    assert np.array_equal(c, off)


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("per_channel", [1, 0])
def test_random_data_invariants(orc, bits, per_channel):
    rng = np.random.default_rng(bits + 100 * per_channel)
    B, H, S, D, gs = 2, 2, 77, 64, 32
    lo, hi = 3, 71
    x = rng.standard_normal((B, H, S, D))
    x[..., rng.integers(0, D, 4)] *= 8
    x = x.astype(np.float16)
    rec, codes, scale, mn = orc.kivi_round_trip(x.view(np.uint16), lo, hi, per_channel, bits, gs,
                                                want_params=True)
    rec2, *_ = orc.kivi_round_trip(x.view(np.uint16), lo, hi, per_channel, bits, gs)
    assert np.array_equal(rec, rec2)  # deterministic
    r = rec.view(np.float16).astype(np.float64)
    xf = x.astype(np.float64)
    # rows outside [lo, hi) untouched
    assert np.array_equal(rec[:, :, :lo], x.view(np.uint16)[:, :, :lo])
    assert np.array_equal(rec[:, :, hi:], x.view(np.uint16)[:, :, hi:])
    m = (1 << bits) - 1
    cb = np.unpackbits(codes, axis=-1, bitorder="little")[..., : D * bits]
    c = (cb.reshape(*cb.shape[:-1], D, bits) * (1 << np.arange(bits))).sum(-1)
    assert c.min() >= 0 and c.max() <= m
    sl = xf[:, :, lo:hi]
    n = hi - lo
    if per_channel:
        g_of = np.arange(n) // gs
        gmin = np.stack([sl[:, :, g * gs:(g + 1) * gs].min(2) for g in range(g_of[-1] + 1)], 2)
        gmax = np.stack([sl[:, :, g * gs:(g + 1) * gs].max(2) for g in range(g_of[-1] + 1)], 2)
        s_e, mn_e = scale[:, :, g_of, :], mn[:, :, g_of, :]
        gmin_e = gmin[:, :, g_of, :]
    else:
        ng = (D + gs - 1) // gs
        gmin = np.stack([sl[..., g * gs:(g + 1) * gs].min(-1) for g in range(ng)], -1)
        gmax = np.stack([sl[..., g * gs:(g + 1) * gs].max(-1) for g in range(ng)], -1)
        g_of = np.arange(D) // gs
        s_e, mn_e = scale[..., g_of], mn[..., g_of]
        gmin_e = gmin[..., g_of]
    assert np.array_equal(mn.astype(np.float64), gmin)  # stored min is the group min
    # scale is (max-min)/m up to binary32 rounding, floored at eps
    assert np.allclose(scale, np.maximum((gmax - gmin) / m, 1e-8), rtol=2 ** -22, atol=0)
    # the group minimum itself is reproduced exactly
    at_min = sl == gmin_e
    assert np.array_equal(r[:, :, lo:hi][at_min], sl[at_min])
    # error bound: half a step plus binary32 slack plus the fp16 store
    err = np.abs(r[:, :, lo:hi] - sl)
    ulp16 = np.spacing(np.abs(r[:, :, lo:hi]).astype(np.float16)).astype(np.float64)
    assert np.all(err <= s_e * 0.5 * (1 + 2 ** -20) + np.abs(sl) * 2 ** -22 + ulp16 / 2 + 1e-12)


def test_eps_floor(orc):
    x = np.zeros((1, 1, 4, 32), np.float16)
    x[0, 0, 1, 0] = np.float16(2.0 ** -24)  # group range far below 255*eps
    rec, _, scale, mn = orc.kivi_round_trip(x.view(np.uint16), 0, 4, 0, 8, 32, want_params=True)
    assert scale[0, 0, 1, 0] == EPS and scale[0, 0, 0, 0] == EPS


@pytest.mark.parametrize("per_channel", [1, 0])
def test_single_element_groups_are_exact(orc, per_channel):
    """The page's degenerate case: a one-element group has min == max, the
    scale collapses to eps and the round trip is bit-exact."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((2, 2, 9, 16)) * 5).astype(np.float16)
    if per_channel:
        rec, *_ = orc.kivi_round_trip(x.view(np.uint16), 4, 5, 1, 2, 32)  # one token
    else:
        rec, *_ = orc.kivi_round_trip(x.view(np.uint16), 0, 9, 0, 2, 1)   # gs = 1
    assert np.array_equal(rec, x.view(np.uint16))


def test_boundary_and_residual_bound(orc):
    """The boundary is a multiple of the group size and the fp16 tail never
    exceeds residual_length + group_size - 1 tokens (page: residual_fp16_bytes)."""
    R, gs = 128, 32
    prev = 0
    for off in range(0, 2000):
        b = orc.kivi_boundary(off, R, gs)
        assert b % gs == 0 and b >= prev and b <= off
        tail = off - b
        assert tail <= R + gs - 1
        if off >= R:
            assert tail >= R
        else:
            assert b == 0
        prev = b


@pytest.mark.parametrize("chunks", [[1] * 300, [300], [7, 100, 1, 1, 64, 127], [129, 171]])
def test_chunking_independence(orc, chunks):
    """One-shot prefill and token-by-token arrival quantize the same positions
    with the same groups (page: _quantization_boundary docstring)."""
    R, gs, bits = 128, 32, 2
    rng = np.random.default_rng(9)
    T = sum(chunks)
    k = (rng.standard_normal((1, 2, T, 16)) * 3).astype(np.float16).view(np.uint16)
    v = (rng.standard_normal((1, 2, T, 16)) * 0.5).astype(np.float16).view(np.uint16)

    def run(parts):
        K, V = k.copy(), v.copy()
        off = nq = 0
        for p in parts:
            off += p
            b = orc.kivi_boundary(off, R, gs)
            if b > nq:
                K, *_ = orc.kivi_round_trip(K, nq, b, 1, bits, gs)
                V, *_ = orc.kivi_round_trip(V, nq, b, 0, bits, gs)
                nq = b
        return K, V, nq

    K1, V1, n1 = run([T])
    K2, V2, n2 = run(chunks)
    assert n1 == n2 == (T - R) // gs * gs
    assert np.array_equal(K1, K2) and np.array_equal(V1, V2)


# ------------------------------------------------------------------ library cross-check
def _torch_round_trip(x_u16, lo, hi, per_channel, bits, gs, eps=1e-8):
    """The kivi_cache page's group round trip (_quant_dequant_along) restated
    with torch CPU eager operations, one IEEE operation per step: float32
    cast, edge-replicating pad to whole groups, group min / max, scale =
    (max - min) / levels then the maximum with eps, (x - min) / scale, round
    (half to even), clip to [0, levels], then the product and the sum as two
    separate operations, cast to fp16. Returns (fp16 bits, codes)."""
    import torch

    x = torch.from_numpy(np.ascontiguousarray(x_u16).view(np.int16).copy()).view(torch.float16)
    out = x.clone()
    sl = x[:, :, lo:hi].to(torch.float32)
    axis = 2 if per_channel else 3
    n = sl.shape[axis]
    pad = (-n) % gs
    if pad:
        last = sl.narrow(axis, n - 1, 1)
        reps = [1, 1, 1, 1]
        reps[axis] = pad
        sl = torch.cat([sl, last.repeat(*reps)], dim=axis)
    shp = list(sl.shape)
    g = sl.reshape(*shp[:axis], shp[axis] // gs, gs, *shp[axis + 1:])
    gmin = g.amin(dim=axis + 1, keepdim=True)
    gmax = g.amax(dim=axis + 1, keepdim=True)
    levels = torch.full_like(gmin, float((1 << bits) - 1))
    scale = torch.div(torch.sub(gmax, gmin), levels)
    scale = torch.maximum(scale, torch.full_like(scale, eps))
    q = torch.round(torch.div(torch.sub(g, gmin), scale))
    q = torch.clamp(q, torch.zeros_like(q), levels.expand_as(q))
    prod = torch.mul(q, scale)
    rec = torch.add(prod, gmin)
    rec = rec.reshape(shp).narrow(axis, 0, n).to(torch.float16)
    out[:, :, lo:hi] = rec
    codes = q.reshape(shp).narrow(axis, 0, n).to(torch.int64).numpy()
    return out.view(torch.int16).numpy().view(np.uint16), codes


def _unpack_codes(codes, D, bits):
    cb = np.unpackbits(codes, axis=-1, bitorder="little")[..., : D * bits]
    return (cb.reshape(*cb.shape[:-1], D, bits) * (1 << np.arange(bits))).sum(-1)


def _tie_data(rng, B, H, S, D, lo, hi, gs, bits, per_channel):
    """Groups whose scale is a power of two (max - min = levels * 2^e) and
    whose other members sit exactly half-way between two codes, so every
    quotient (x - min)/scale of a non-end member is an exact .5 tie."""
    m = (1 << bits) - 1
    x = rng.standard_normal((B, H, S, D))
    e = -3 if bits < 8 else -7
    sl = x[:, :, lo:hi]
    axis = 2 if per_channel else 3
    n = sl.shape[axis]
    ng = (n + gs - 1) // gs
    for gi in range(ng):
        a, b = gi * gs, min(gi * gs + gs, n)
        idx = [slice(None)] * 4
        idx[axis] = slice(a, b)
        blk = np.moveaxis(sl[tuple(idx)], axis, -1)
        base = rng.integers(-64, 64, size=blk.shape[:-1] + (1,)) * 2.0 ** (e - 1)
        half = rng.integers(0, m, size=blk.shape) + 0.5
        vals = base + half * 2.0 ** e
        vals[..., 0] = base[..., 0]
        if b - a > 1:
            vals[..., -1] = base[..., 0] + m * 2.0 ** e
        sl[tuple(idx)] = np.moveaxis(vals, -1, axis)
    xf = x.astype(np.float16)
    assert np.array_equal(xf[:, :, lo:hi].astype(np.float64), sl)  # every value exact in fp16
    return xf


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("per_channel", [1, 0])
def test_matches_torch_transliteration(orc, bits, per_channel):
    """Bit-for-bit against the torch restatement on random data (ragged last
    groups on both axes) and on exact-tie data."""
    rng = np.random.default_rng(40 + bits + 7 * per_channel)
    B, H, S, D, gs = 2, 3, 150, 72, 32
    lo, hi = 6, 141                                   # 135 tokens: ragged key group
    x = rng.standard_normal((B, H, S, D)) * rng.choice([0.01, 1, 30], size=(B, H, 1, D))
    for data in (x.astype(np.float16), _tie_data(rng, B, H, S, D, lo, hi, gs, bits, per_channel)):
        rec, codes, _, _ = orc.kivi_round_trip(data.view(np.uint16), lo, hi, per_channel, bits, gs,
                                               want_params=True)
        ref, qref = _torch_round_trip(data.view(np.uint16), lo, hi, per_channel, bits, gs)
        assert np.array_equal(rec, ref)
        assert np.array_equal(_unpack_codes(codes, D, bits), qref)


@pytest.mark.parametrize("bits", [2, 4, 8])
@pytest.mark.parametrize("per_channel", [1, 0])
def test_exact_ties_round_to_even(orc, bits, per_channel):
    """A member half-way between codes c and c + 1 gets the even one (the page
    rounds with mx.round, which rounds half to even)."""
    rng = np.random.default_rng(60 + bits + 7 * per_channel)
    B, H, S, D, gs = 2, 2, 100, 64, 16
    lo, hi = 3, 99
    x = _tie_data(rng, B, H, S, D, lo, hi, gs, bits, per_channel)
    _, codes, scale, mn = orc.kivi_round_trip(x.view(np.uint16), lo, hi, per_channel, bits, gs, want_params=True)
    c = _unpack_codes(codes, D, bits)
    e = -3 if bits < 8 else -7
    assert np.all(scale == np.float32(2.0 ** e))
    t = x[:, :, lo:hi].astype(np.float64)
    if per_channel:
        g = np.arange(hi - lo) // gs
        t = (t - mn[:, :, g, :]) / 2.0 ** e
    else:
        g = np.arange(D) // gs
        t = (t - mn[..., g]) / 2.0 ** e
    tie = (t - np.floor(t)) == 0.5
    assert tie.sum() > 0.8 * t.size
    assert np.all(c[tie] % 2 == 0)
    assert np.all(np.abs(c[tie] - t[tie]) == 0.5)


def test_reconstruction_rounds_the_product_before_the_sum(orc):
    """x' = fp16(RN32(RN32(code * scale) + min)): on data where the fused
    form RN32(code * scale + min) differs, the oracle gives the unfused one."""
    rng = np.random.default_rng(77)
    B, H, S, D, gs, bits = 4, 4, 256, 64, 32, 4
    x = (rng.standard_normal((B, H, S, D)) * 3).astype(np.float16)
    rec, codes, scale, mn = orc.kivi_round_trip(x.view(np.uint16), 0, S, 0, bits, gs, want_params=True)
    c = _unpack_codes(codes, D, bits).astype(np.float32)
    g = np.arange(D) // gs
    s32, m32 = scale[..., g], mn[..., g]
    unfused = (c * s32).astype(np.float32) + m32
    fused = (c.astype(np.float64) * s32.astype(np.float64) + m32.astype(np.float64)).astype(np.float32)
    differ = unfused.astype(np.float16) != fused.astype(np.float16)
    assert differ.sum() > 0                     # the data separates the two forms
    got = rec.view(np.float16)
    assert np.array_equal(got[differ], unfused.astype(np.float16)[differ])
