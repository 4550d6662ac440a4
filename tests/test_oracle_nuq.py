"""Pins of the oracle's KVQuant-style non-uniform quantizer (NUQ).

Source: "veloxquant_mlx.cache.kvquant_cache module" -- module docstring
(per-channel keys / per-token values, Lloyd-Max fit as the unweighted k-means
special case, dense-and-sparse outliers with a nominal fraction, frozen key
levels and thresholds after prefill, value levels fit on every call,
attention-sink tokens kept exact and excluded from fits and thresholds) and
the KVQuantKVCache property docs (outlier_count realized vs nominal).

Pins: numpy's linear quantile for the initialisation; brute-force optimal
1-D k-means on tiny inputs (contiguous partitions); Lloyd fixed-point and
monotone-distortion properties; exact cluster means on separated clusters;
the closed-form optimal 1-bit Gaussian quantizer +-sqrt(2/pi); order-statistic
properties of the threshold; and the sink / outlier / frozen-level
invariants the page states.
"""
import itertools
import math

import numpy as np
import pytest


def f16(a):
    return np.asarray(a, np.float64).astype(np.float16)


def _assign(u, lev):
    return np.abs(u[:, None] - lev[None, :].astype(np.float64)).argmin(1)  # ties -> lower index


def _distortion(u, lev):
    return float(((u - lev.astype(np.float64)[_assign(u, lev)]) ** 2).sum())


def _brute_force_opt(u, L):
    u = np.sort(u)
    m = len(u)
    best = math.inf
    for k in range(1, min(L, m) + 1):
        for cuts in itertools.combinations(range(1, m), k - 1):
            parts = np.split(u, cuts)
            best = min(best, sum(float(((p - p.mean()) ** 2).sum()) for p in parts))
    return best


@pytest.mark.parametrize("L", [2, 4, 8, 16])
def test_quantile_init_matches_numpy(orc, L):
    rng = np.random.default_rng(L)
    for m in (1, 2, 3, 7, 100, 4092):
        u = f16(rng.standard_t(4, size=m))
        got = orc.nuq_fit(u, L, 0)
        p = (np.arange(L) + 0.5) / L
        ref = np.quantile(u.astype(np.float64), p, method="linear").astype(np.float32)
        assert np.array_equal(got, ref), (m, got, ref)


def test_separated_clusters_give_exact_means(orc):
    rng = np.random.default_rng(1)
    centers = np.array([-40.0, -3.0, 5.0, 90.0])
    u = np.concatenate([c + f16(rng.uniform(-1, 1, 3)).astype(np.float64) for c in centers])
    u = f16(u)
    lev = orc.nuq_fit(u, 4, 3)
    uf = np.sort(u.astype(np.float64))
    means = np.array([uf[3 * i:3 * i + 3].sum() / 3 for i in range(4)], np.float32)
    assert np.array_equal(lev, means)
    assert math.isclose(_distortion(uf, lev), _brute_force_opt(uf, 4), rel_tol=1e-6, abs_tol=1e-9)


def test_lloyd_properties_on_tiny_inputs(orc):
    rng = np.random.default_rng(2)
    for trial in range(150):
        m = int(rng.integers(1, 10))
        L = int(rng.choice([2, 4]))
        u = f16(rng.integers(-6, 7, size=m) * 0.5 + rng.choice([0, 0.125], size=m))
        uf = u.astype(np.float64)
        opt = _brute_force_opt(uf, L)
        prev = math.inf
        for it in range(0, 12):
            lev = orc.nuq_fit(u, L, it)
            assert np.all(np.diff(lev) >= 0)          # levels stay ordered
            d = _distortion(uf, lev)
            assert d <= prev * (1 + 1e-6) + 1e-12     # Lloyd never increases distortion
            assert d >= opt - 1e-9                    # cannot beat the optimum
            prev = d
        # after convergence: a fixed point of the Lloyd map
        a = _assign(uf, lev)
        for j in range(L):
            if np.any(a == j):
                assert lev[j] == np.float32(uf[a == j].sum() / np.sum(a == j))


def test_tie_heavy_data_keeps_an_ordered_table(orc):
    """Quantile initialisation on heavily tied data yields duplicate levels;
    the empty duplicate must not end up out of order (ordered signpost table),
    and the result must still be a Lloyd fixed point of the same codebook."""
    rng = np.random.default_rng(21)
    seen_dup_init = 0
    for trial in range(400):
        u = f16(rng.choice([-2, -1, 0, 1, 2, 3], size=32, p=[.04, .1, .5, .26, .08, .02]))
        init = orc.nuq_fit(u, 4, 0)
        seen_dup_init += int(np.any(np.diff(init) == 0))
        for it in range(1, 9):
            lev = orc.nuq_fit(u, 4, it)
            assert np.all(np.diff(lev) >= 0), (trial, it, lev)
        uf = u.astype(np.float64)
        lev = orc.nuq_fit(u, 4, 60)
        a = _assign(uf, lev)
        for j in range(4):
            if np.any(a == j):
                assert lev[j] == np.float32(uf[a == j].sum() / np.sum(a == j))
    assert seen_dup_init > 50  # the case this pin is about does occur


def test_one_bit_gaussian_closed_form(orc):
    # symmetrised sample: the 2-level Lloyd fixed point is +-mean|x|, which for
    # N(0,1) tends to sqrt(2/pi) (sampling sd ~ 0.005 at this size)
    rng = np.random.default_rng(4)
    h = f16(np.abs(rng.standard_normal(16384)))
    u = np.concatenate([h, -h])
    lev = orc.nuq_fit(u, 2, 30)
    assert lev[1] == -lev[0] == np.float32(h.astype(np.float64).mean())
    assert abs(lev[1] - math.sqrt(2 / math.pi)) < 0.02


def test_L_distinct_values_reconstruct_exactly(orc):
    rng = np.random.default_rng(6)
    vals = f16([-7.5, -1.25, -0.5, 0.0, 0.75, 2.0, 3.5, 11.0])
    u = rng.permutation(np.repeat(vals, 13))
    lev = orc.nuq_fit(u, 8, 8)
    assert np.array_equal(np.sort(lev), vals.astype(np.float32))
    for x in vals:
        assert lev[orc.nuq_nearest(np.float16(x).view(np.uint16), lev)] == np.float32(x)


def test_nearest_ties_go_low(orc):
    lev = np.array([0.0, 1.0, 1.0, 3.0], np.float32)
    assert orc.nuq_nearest(np.float16(0.5).view(np.uint16), lev) == 0
    assert orc.nuq_nearest(np.float16(1.0).view(np.uint16), lev) == 1
    assert orc.nuq_nearest(np.float16(2.0).view(np.uint16), lev) == 1
    assert orc.nuq_nearest(np.float16(2.001953125).view(np.uint16), lev) == 3


@pytest.mark.parametrize("frac", [0.0, 0.01, 0.05, 0.5])
def test_threshold_is_the_k_plus_1_th_largest(orc, frac):
    rng = np.random.default_rng(8)
    for n in (1, 5, 128, 4092):
        x = f16(rng.standard_t(4, size=n))
        x[: n // 10] = x[0]  # ties
        tau = np.uint16(orc.nuq_threshold(x, frac)).view(np.float16)
        k = math.floor(frac * n)
        a = np.abs(x.astype(np.float64))
        assert np.sum(a > tau) <= k < np.sum(a >= tau)


# ------------------------------------------------------------------ whole call
def _t4(rng, shape):
    return f16(rng.standard_t(4, size=shape))


@pytest.fixture(scope="module")
def prefill(orc):
    rng = np.random.default_rng(12)
    BH, S, D = 3, 70, 16
    k, v = _t4(rng, (BH, S, D)), _t4(rng, (BH, S, D))
    r = orc.nuq_fit_quant(k, v, 0, 3, 0.05, 8, 4, 1)
    return k, v, r


def _codes(c, D, bits=3):
    b = np.unpackbits(c, axis=-1, bitorder="little")[..., : D * bits]
    return (b.reshape(*b.shape[:-1], D, bits) * (1 << np.arange(bits))).sum(-1)


def test_sinks_exact_and_excluded(orc, prefill):
    k, v, r = prefill
    assert np.array_equal(r["k_recon"][:, :4], k.view(np.uint16)[:, :4])
    assert np.array_equal(r["v_recon"][:, :4], v.view(np.uint16)[:, :4])
    assert np.all(r["value_levels"][:, :4] == 0)
    assert np.all(_codes(r["k_codes"], 16)[:, :4] == 0) and np.all(_codes(r["v_codes"], 16)[:, :4] == 0)
    k2, v2 = k.copy(), v.copy()
    k2[:, :4] = f16(1000.0)
    v2[:, :4] = f16(-777.0)
    r2 = orc.nuq_fit_quant(k2, v2, 0, 3, 0.05, 8, 4, 1)
    for name in ("key_levels", "key_thresh", "value_levels"):
        assert np.array_equal(r[name], r2[name])
    assert np.array_equal(r["k_recon"][:, 4:], r2["k_recon"][:, 4:])
    assert np.array_equal(r["v_recon"][:, 4:], r2["v_recon"][:, 4:])
    # a later call (start_pos > 0) has no sinks
    r3 = orc.nuq_fit_quant(k, v, 70, 3, 0.05, 8, 4, 0, r["key_levels"], r["key_thresh"])
    assert not np.array_equal(r3["v_recon"][:, :4], v.view(np.uint16)[:, :4])


def test_outliers_exact_bounded_and_sorted(orc, prefill):
    k, v, r = prefill
    BH, S, D = k.shape
    for x, (pos, val), rec, thr_axis in ((k, r["k_out"], r["k_recon"], "k"), (v, r["v_out"], r["v_recon"], "v")):
        assert np.all(np.diff(pos) > 0)
        assert np.array_equal(val, x.reshape(-1).view(np.uint16)[pos])
        assert np.array_equal(rec.reshape(-1)[pos], val)
        flag = np.zeros(BH * S * D, bool)
        flag[pos] = True
        flag = flag.reshape(BH, S, D)
        assert not flag[:, :4].any()
        if thr_axis == "k":  # per channel over S-4 tokens
            kmax = math.floor(0.05 * (S - 4))
            assert flag.sum(1).max() <= kmax
            tau = r["key_thresh"].view(np.float16).astype(np.float64)
            a = np.abs(x.astype(np.float64))[:, 4:]
            assert np.array_equal(flag[:, 4:], a > tau[:, None, :])
        else:                # per token over D channels
            assert flag.sum(2).max() <= math.floor(0.05 * D)
        assert np.all(_codes(r["k_codes" if thr_axis == "k" else "v_codes"], D)[flag] == 0)


def test_inliers_use_their_levels(orc, prefill):
    k, v, r = prefill
    BH, S, D = k.shape
    kc, vc = _codes(r["k_codes"], D), _codes(r["v_codes"], D)
    kl, vl = r["key_levels"], r["value_levels"]
    rec_k = r["k_recon"].view(np.float16)
    rec_v = r["v_recon"].view(np.float16)
    for bh in range(BH):
        for s in range(4, S):
            for d in range(D):
                if abs(float(k[bh, s, d])) <= float(r["key_thresh"][bh, d].view(np.float16)):
                    assert rec_k[bh, s, d] == np.float16(kl[bh, d, kc[bh, s, d]])
                    assert kc[bh, s, d] == _assign(np.array([float(k[bh, s, d])]), kl[bh, d])[0]
            row = v[bh, s].astype(np.float64)
            a = _assign(row, vl[bh, s])
            inl = rec_v[bh, s] != v[bh, s]  # not exact -> must be an inlier's level
            assert np.all(vc[bh, s][inl] == a[inl])


def test_decode_keys_use_frozen_levels(orc, prefill):
    k, v, r = prefill
    BH, S, D = k.shape
    rng = np.random.default_rng(13)
    # one decode token equal to prefill token 10 -> identical key codes
    kd = k[:, 10:11].copy()
    vd = _t4(rng, (BH, 1, D))
    rd = orc.nuq_fit_quant(kd, vd, S, 3, 0.05, 8, 4, 0, r["key_levels"], r["key_thresh"])
    assert np.array_equal(rd["key_levels"], r["key_levels"])
    assert np.array_equal(_codes(rd["k_codes"], D)[:, 0], _codes(r["k_codes"], D)[:, 10])
    assert np.array_equal(rd["k_recon"][:, 0], r["k_recon"][:, 10])


def test_all_sink_prefill_and_tiny_vectors(orc):
    rng = np.random.default_rng(14)
    k, v = _t4(rng, (2, 3, 8)), _t4(rng, (2, 3, 8))
    r = orc.nuq_fit_quant(k, v, 0, 2, 0.01, 8, 4, 1)   # S=3 < n_sink: everything exact
    assert np.array_equal(r["k_recon"], k.view(np.uint16))
    assert np.all(r["key_levels"] == 0) and np.all(r["key_thresh"] == 0)
    r = orc.nuq_fit_quant(k, v, 0, 2, 0.01, 8, 2, 1)   # one non-sink token per channel
    assert np.array_equal(r["k_recon"][:, 2], k.view(np.uint16)[:, 2])  # single sample is its own level


# ------------------------------------------------------------------ outlier count reading
def _distinct_magnitudes(rng, n):
    """n fp16 values with pairwise different |x| (distinct positive normal
    patterns) and random signs."""
    pats = rng.choice(np.arange(0x2c00, 0x5c00, dtype=np.uint16), size=n, replace=False)
    sign = rng.integers(0, 2, size=n).astype(np.uint16) << 15
    return (pats | sign).astype(np.uint16)


# The page's kvquant_outlier_fraction is a Python float (binary64, default
# 0.01); the count is floor(fraction * n) of that binary64 product, so whole
# percentages of round sample counts give the integer one expects.
@pytest.mark.parametrize("frac,n,k", [(0.01, 100, 1), (0.01, 200, 2), (0.01, 1000, 10), (0.01, 99, 0),
                                      (0.01, 128, 1), (0.01, 4092, 40), (0.03, 100, 3), (0.05, 100, 5),
                                      (0.1, 1000, 100), (0.0, 500, 0), (0.5, 7, 3)])
def test_outlier_count_at_whole_percentages(orc, frac, n, k):
    rng = np.random.default_rng(n + int(frac * 1000))
    x = _distinct_magnitudes(rng, n)
    tau = np.uint16(orc.nuq_threshold(x, frac)).view(np.float16)
    a = np.abs(x.view(np.float16).astype(np.float64))
    assert int(np.sum(a > float(tau))) == k


def test_prefill_of_104_tokens_with_4_sinks_isolates_one_key_per_channel(orc):
    """100 non-sink tokens at 1%: exactly one key outlier per channel, and
    with D = 200 exactly two value outliers per token."""
    rng = np.random.default_rng(104)
    BH, S, D = 2, 104, 200
    k = np.stack([np.stack([_distinct_magnitudes(rng, S) for _ in range(D)], 1) for _ in range(BH)])
    v = np.stack([np.stack([_distinct_magnitudes(rng, D) for _ in range(S)], 0) for _ in range(BH)])
    r = orc.nuq_fit_quant(k, v, 0, 3, 0.01, 8, 4, 1)
    pos = r["k_out"][0]
    assert len(pos) == BH * D
    per_ch = np.bincount((pos // (S * D)) * D + pos % D, minlength=BH * D)
    assert np.all(per_ch == 1)
    vpos = r["v_out"][0]
    assert len(vpos) == BH * (S - 4) * 2
    assert np.all(np.bincount(vpos // D, minlength=BH * S)[np.arange(BH * S) % S >= 4] == 2)


# ------------------------------------------------------------------ outliers are left out of the fit
def test_outliers_are_excluded_from_the_level_fit(orc):
    """Dense-and-sparse: the levels are fit on the dense part only. Moving the
    isolated samples further out (they stay the isolated ones, the threshold
    does not change) leaves every key and value level unchanged, while a fit
    that included them would move a level (checked on the same data)."""
    rng = np.random.default_rng(31)
    BH, S, D = 2, 204, 64
    k, v = _t4(rng, (BH, S, D)), _t4(rng, (BH, S, D))
    frac = 0.02
    r = orc.nuq_fit_quant(k, v, 0, 3, frac, 8, 4, 1)
    k2 = k.reshape(-1).copy()
    v2 = v.reshape(-1).copy()
    kp, vp = r["k_out"][0], r["v_out"][0]
    assert len(kp) > 0 and len(vp) > 0
    k2[kp] = f16(k2[kp].astype(np.float64) * 8)
    v2[vp] = f16(v2[vp].astype(np.float64) * 8)
    k2, v2 = k2.reshape(k.shape), v2.reshape(v.shape)
    r2 = orc.nuq_fit_quant(k2, v2, 0, 3, frac, 8, 4, 1)
    for name in ("key_levels", "key_thresh", "value_levels", "k_codes", "v_codes"):
        assert np.array_equal(r[name], r2[name]), name
    assert np.array_equal(r2["k_out"][0], kp) and np.array_equal(r2["v_out"][0], vp)
    # the pin has power: fitting all samples of a vector moves at least one level
    moved = 0
    for bh in range(BH):
        for d in range(D):
            col = k2[bh, 4:, d]
            moved += int(not np.array_equal(orc.nuq_fit(col, 8, 8), r2["key_levels"][bh, d]))
        for s in range(4, S):
            moved += int(not np.array_equal(orc.nuq_fit(v2[bh, s], 8, 8), r2["value_levels"][bh, s]))
    assert moved > 0.5 * BH * (D + S - 4)
