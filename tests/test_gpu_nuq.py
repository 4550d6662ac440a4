"""GPU parity of the KVQuant-style NUQ path against the CPU oracle.

Every output is compared bit-for-bit: key level tables and thresholds,
value level tables, packed codes, the outlier lists (flat index and fp16
value, ascending) with their counts, and the reconstructions. The stated
tolerance for NUQ (levels within 1e-3 relative, at most 0.01% of codes
different and only next to a level boundary) is the fallback contract; the
exact-sum formulation makes bit-exact the expected result, so the tests
require it. Inputs: Student-t(4) like the pages' workload, plus tie-heavy,
zero-heavy and extreme-value cases, ragged S, every width 1..4, every
supported head dim, prefill then decode against the frozen key levels.
"""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_quantization_row_amd import inputs, kvq
from tests.gpu_util import Guarded, dev, first_diff, say, u16

pytestmark = pytest.mark.gpu


def gpu_nuq(k, v, start_pos, bits, frac, iters, n_sink, fit_keys, key_levels=None, key_thresh=None,
            want_recon=True):
    d = dev()
    g = Guarded(d)  # sentinel bands around every output and the workspace
    BH, S, D = k.shape
    L = 1 << bits
    kl = g.empty((BH, D, L), torch.float32, 0.0)
    kt = g.empty((BH, D), torch.int16, 0)
    if key_levels is not None:
        kl.copy_(torch.from_numpy(np.ascontiguousarray(key_levels)))
        kt.copy_(torch.from_numpy(np.ascontiguousarray(key_thresh).view(np.int16)))
    vl = g.empty((BH, S, L), torch.float32, 7.0)
    kc = g.empty((BH, S, D * bits // 8), torch.uint8, 0xA5)
    vc = g.empty((BH, S, D * bits // 8), torch.uint8, 0x5A)
    cap = max(kvq.kvq_nuq_outlier_bound(BH, S, D, start_pos, n_sink, frac, fit_keys, 0),
              kvq.kvq_nuq_outlier_bound(BH, S, D, start_pos, n_sink, frac, fit_keys, 1), 1)
    kp = g.empty((cap,), torch.int32, -1)
    kvv = g.empty((cap,), torch.int16, 0)
    vp = g.empty((cap,), torch.int32, -1)
    vvv = g.empty((cap,), torch.int16, 0)
    cnt = g.empty((2,), torch.int64, -1)
    wsb = kvq.kvq_nuq_workspace_bytes(BH, S, D, bits, start_pos, n_sink, frac, fit_keys)
    ws = g.empty((wsb,), torch.uint8, 0xEE)  # contents on entry must not matter
    kr = g.empty((BH, S, D), torch.float16, 0.0) if want_recon else None
    vr = g.empty((BH, S, D), torch.float16, 0.0) if want_recon else None
    kg = torch.from_numpy(np.ascontiguousarray(k).view(np.int16)).to(d).view(torch.float16)
    vg = torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).to(d).view(torch.float16)
    kvq.kvq_nuq_fit_quant(kg, vg, start_pos, bits, frac, iters, n_sink, fit_keys, kl, kt, vl, kc, vc,
                          kp, kvv, vp, vvv, cnt, ws, kr, vr)
    g.check("nuq call")
    c = cnt.cpu().numpy()
    out = dict(key_levels=kl.cpu().numpy(), key_thresh=u16(kt), value_levels=vl.cpu().numpy(),
               k_codes=kc.cpu().numpy(), v_codes=vc.cpu().numpy(),
               k_out=(kp.cpu().numpy()[:c[0]], u16(kvv)[:c[0]]),
               v_out=(vp.cpu().numpy()[:c[1]], u16(vvv)[:c[1]]))
    if want_recon:
        out["k_recon"] = u16(kr)
        out["v_recon"] = u16(vr)
    return out


def compare(got, ref, keys=None, what=""):
    for name in keys or ["key_levels", "key_thresh", "value_levels", "k_codes", "v_codes", "k_recon",
                         "v_recon"]:
        if name not in got:
            continue
        a, b = got[name], ref[name]
        if a.dtype == np.float32:
            a, b = a.view(np.uint32), b.view(np.uint32)
        assert a.shape == b.shape, (what, name, a.shape, b.shape)
        assert first_diff(a, b) is None, (what, name, first_diff(a, b))
    for name in ("k_out", "v_out"):
        (gp, gv), (rp, rv) = got[name], ref[name]
        assert len(gp) == len(rp), (what, name, "count", len(gp), len(rp))
        assert np.array_equal(gp, rp), (what, name, "positions", first_diff(gp, rp))
        assert np.array_equal(gv, rv), (what, name, "values", first_diff(gv, rv))


def t4(shape, seed):
    return inputs.student_t(shape, 4, seed=seed).numpy().view(np.uint16)


@pytest.mark.parametrize("bits", [3, 1, 2, 4])
@pytest.mark.parametrize("D", [128, 32, 64, 256])
def test_prefill_then_decode(bits, D):
    say("nuq prefill/decode", bits, D)
    BH, S = 3, 150
    k, v = t4((BH, S, D), 10 + D + bits), t4((BH, S, D), 20 + D + bits)
    frac, iters, ns = 0.02, 8, 4
    g = gpu_nuq(k, v, 0, bits, frac, iters, ns, 1)
    r = oracle.nuq_fit_quant(k, v, 0, bits, frac, iters, ns, 1)
    compare(g, r, what="prefill")
    for step in range(3):
        kd, vd = t4((BH, 1, D), 100 + step), t4((BH, 1, D), 200 + step)
        if step == 1:
            kd[:] = k[:, 77:78]  # a decode key equal to a prefill key
        g = gpu_nuq(kd, vd, S + step, bits, frac, iters, ns, 0, g["key_levels"], g["key_thresh"])
        r = oracle.nuq_fit_quant(kd, vd, S + step, bits, frac, iters, ns, 0, r["key_levels"],
                                 r["key_thresh"])
        compare(g, r, what="decode %d" % step)


@pytest.mark.parametrize("bits", [3, 1, 2, 4])
@pytest.mark.parametrize("D", [128, 32, 64, 256])
def test_many_tokens_value_path(bits, D):
    """More than 4096 (batch, head, token) value vectors: the value fit runs one
    lane (or two at D=256) per token instead of one wave per token."""
    say("nuq many tokens", bits, D)
    BH, S = 33, 130
    k, v = t4((BH, S, D), 30 + D + bits), t4((BH, S, D), 40 + D + bits)
    g = gpu_nuq(k, v, 0, bits, 0.02, 8, 4, 1)
    r = oracle.nuq_fit_quant(k, v, 0, bits, 0.02, 8, 4, 1)
    compare(g, r, what="BH=%d S=%d" % (BH, S))


@pytest.mark.parametrize("S", [1, 3, 4, 5, 129, 260, 1000, 2049])
def test_ragged_lengths_and_sinks(S):
    say("nuq ragged", S)
    BH, D, bits = 2, 64, 3
    k, v = t4((BH, S, D), S), t4((BH, S, D), S + 1)
    for sp, ns in [(0, 4), (0, 0), (9, 4)]:
        g = gpu_nuq(k, v, sp, bits, 0.01, 8, ns, 1)
        r = oracle.nuq_fit_quant(k, v, sp, bits, 0.01, 8, ns, 1)
        compare(g, r, what="S=%d start=%d sinks=%d" % (S, sp, ns))


@pytest.mark.parametrize("S", [104, 204, 1004])
def test_outlier_count_at_whole_percentages(S):
    """S - 4 non-sink tokens at a 1% fraction: 1, 2 and 10 key outliers per
    channel (floor of the binary64 product), as in the oracle."""
    say("nuq whole-percentage counts", S)
    BH, D, bits = 3, 128, 3
    k, v = t4((BH, S, D), 70 + S), t4((BH, S, D), 71 + S)
    g = gpu_nuq(k, v, 0, bits, 0.01, 8, 4, 1)
    r = oracle.nuq_fit_quant(k, v, 0, bits, 0.01, 8, 4, 1)
    compare(g, r, what="S=%d" % S)
    pos = g["k_out"][0]
    per_ch = np.bincount((pos // (S * D)) * D + pos % D, minlength=BH * D)
    assert per_ch.max() <= (S - 4) // 100 and len(pos) > 0


@pytest.mark.parametrize("BH", [2, 48])  # 48 x 90 tokens: the lane-per-token value path
@pytest.mark.parametrize("case", ["ties", "zeros", "signed_zeros", "extremes", "subnormal", "const"])
def test_degenerate_data(case, BH):
    say("nuq degenerate", case, BH)
    S, D = 90, 32
    rng = np.random.default_rng(["ties", "zeros", "signed_zeros", "extremes", "subnormal", "const"].index(case))
    if case == "ties":
        x = rng.integers(-3, 4, size=(2, BH, S, D)).astype(np.float16)
    elif case == "zeros":
        x = np.zeros((2, BH, S, D), np.float16)
        x[..., ::7] = 1.5
    elif case == "signed_zeros":
        x = np.where(rng.random((2, BH, S, D)) < 0.5, np.float16(0.0), np.float16(-0.0)).astype(np.float16)
        x[:, :, :, 3] = rng.standard_normal((2, BH, S)).astype(np.float16)
    elif case == "extremes":
        x = (rng.standard_t(4, size=(2, BH, S, D)) * 3000).clip(-65504, 65504).astype(np.float16)
        x[:, :, 10, 5] = 65504
        x[:, :, 11, 6] = -65504
    elif case == "subnormal":
        x = (rng.integers(-40, 40, size=(2, BH, S, D)) * 2.0 ** -24).astype(np.float16)
    else:
        x = np.full((2, BH, S, D), 0.25, np.float16)
    k, v = x[0].view(np.uint16), x[1].view(np.uint16)
    for frac, iters in [(0.05, 8), (0.0, 3), (0.3, 0)]:
        g = gpu_nuq(k, v, 0, 2, frac, iters, 4, 1)
        r = oracle.nuq_fit_quant(k, v, 0, 2, frac, iters, 4, 1)
        compare(g, r, what="%s frac=%g iters=%d" % (case, frac, iters))


# many-token key fits (the bucketed counting sort per channel): every width
# at several lengths, n = 4096 and 8192 (the whole sample array in LDS),
# and the degenerate data of the test above at these sizes
@pytest.mark.parametrize("S,bits", [(400, 2), (600, 1), (600, 2), (1100, 3), (1100, 4), (2500, 4), (4100, 3),
                                    (4100, 2), (8196, 4)])
def test_long_key_fits(S, bits):
    say("nuq long key fit", S, bits)
    BH, D = 2, 32
    k, v = t4((BH, S, D), 80 + S + bits), t4((BH, S, D), 90 + S + bits)
    for frac in (0.01, 0.1):
        g = gpu_nuq(k, v, 0, bits, frac, 8, 4, 1, want_recon=S < 8000)
        r = oracle.nuq_fit_quant(k, v, 0, bits, frac, 8, 4, 1)
        keys = None if S < 8000 else ["key_levels", "key_thresh", "k_codes"]
        compare(g, r, keys=keys, what="S=%d bits=%d frac=%g" % (S, bits, frac))


@pytest.mark.parametrize("D,S,BH", [(64, 1500, 3), (128, 1500, 3), (256, 1500, 3), (64, 4100, 2), (256, 8196, 1)])
def test_long_key_fit_head_dims(D, S, BH):
    say("nuq long key fit D S", D, S)
    bits = 3
    k, v = t4((BH, S, D), 300 + D + S), t4((BH, S, D), 301 + D + S)
    g = gpu_nuq(k, v, 0, bits, 0.01, 8, 4, 1, want_recon=S < 8000)
    r = oracle.nuq_fit_quant(k, v, 0, bits, 0.01, 8, 4, 1)
    keys = None if S < 8000 else ["key_levels", "key_thresh", "k_codes"]
    compare(g, r, keys=keys, what="D=%d S=%d" % (D, S))


@pytest.mark.parametrize("S,bits", [(1028, 2), (2100, 3)])
@pytest.mark.parametrize("case", ["ties", "zeros", "signed_zeros", "extremes", "subnormal", "const"])
def test_long_key_fit_degenerate(case, S, bits):
    say("nuq long key fit degenerate", case, S, bits)
    BH, D = 2, 32
    rng = np.random.default_rng(100 + ["ties", "zeros", "signed_zeros", "extremes", "subnormal", "const"].index(case))
    if case == "ties":
        x = rng.integers(-3, 4, size=(2, BH, S, D)).astype(np.float16)
    elif case == "zeros":
        x = np.zeros((2, BH, S, D), np.float16)
        x[..., ::7, :] = 1.5
    elif case == "signed_zeros":
        x = np.where(rng.random((2, BH, S, D)) < 0.5, np.float16(0.0), np.float16(-0.0)).astype(np.float16)
        x[:, :, ::3, :] = rng.standard_normal((2, BH, (S + 2) // 3, D)).astype(np.float16)
    elif case == "extremes":
        x = (rng.standard_t(4, size=(2, BH, S, D)) * 3000).clip(-65504, 65504).astype(np.float16)
        x[:, :, 10, :] = 65504
        x[:, :, 11, :] = -65504
    elif case == "subnormal":
        x = (rng.integers(-40, 40, size=(2, BH, S, D)) * 2.0 ** -24).astype(np.float16)
    else:
        x = np.full((2, BH, S, D), 0.25, np.float16)
    k, v = x[0].view(np.uint16), x[1].view(np.uint16)
    for frac, iters in [(0.05, 8), (0.0, 3), (0.3, 0)]:
        g = gpu_nuq(k, v, 0, bits, frac, iters, 4, 1, want_recon=False)
        r = oracle.nuq_fit_quant(k, v, 0, bits, frac, iters, 4, 1)
        compare(g, r, keys=["key_levels", "key_thresh", "k_codes"],
                what="%s S=%d bits=%d frac=%g iters=%d" % (case, S, bits, frac, iters))


@pytest.mark.parametrize("iters", [1, 2, 4, 16])
def test_lloyd_iteration_counts(iters):
    """The Lloyd iteration count the pages name as the speed / quality lever."""
    say("nuq iters", iters)
    BH, S, D = 4, 300, 128
    k, v = t4((BH, S, D), 60 + iters), t4((BH, S, D), 61 + iters)
    g = gpu_nuq(k, v, 0, 3, 0.01, iters, 4, 1)
    r = oracle.nuq_fit_quant(k, v, 0, 3, 0.01, iters, 4, 1)
    compare(g, r, what="iters=%d" % iters)
    kd, vd = t4((BH, 1, D), 70), t4((BH, 1, D), 71)
    g2 = gpu_nuq(kd, vd, S, 3, 0.01, iters, 4, 0, g["key_levels"], g["key_thresh"])
    r2 = oracle.nuq_fit_quant(kd, vd, S, 3, 0.01, iters, 4, 0, r["key_levels"], r["key_thresh"])
    compare(g2, r2, what="decode iters=%d" % iters)


def test_long_key_fit_64_chunks():
    """8192 non-sink tokens per key channel: 64 lanes per vector."""
    say("nuq 8192-token key fit")
    BH, S, D = 1, 8196, 32
    k, v = t4((BH, S, D), 5), t4((BH, S, D), 6)
    g = gpu_nuq(k, v, 0, 3, 0.01, 8, 4, 1, want_recon=False)
    r = oracle.nuq_fit_quant(k, v, 0, 3, 0.01, 8, 4, 1)
    compare(g, r, keys=["key_levels", "key_thresh", "value_levels", "k_codes", "v_codes"],
            what="S=8196")


def test_full_size_sampled():
    """Batch 4 x 8 KV heads, 4096-token prefill, D=128, 3 bits, 1% outliers,
    8 iterations, 4 sinks; then 64 decode tokens. Compared on sampled heads."""
    say("nuq full size")
    d = dev()
    BH, S, D, bits = 32, 4096, 128, 3
    kt = inputs.student_t((BH, S, D), 4, seed=1004, device=d)
    vt = inputs.student_t((BH, S, D), 4, seed=1005, device=d)
    k, v = u16(kt), u16(vt)
    g = gpu_nuq(k, v, 0, bits, 0.01, 8, 4, 1, want_recon=True)
    for bh in (0, 17, 31):
        r = oracle.nuq_fit_quant(k[bh:bh + 1], v[bh:bh + 1], 0, bits, 0.01, 8, 4, 1)
        sub = {n: g[n][bh:bh + 1] for n in ("key_levels", "key_thresh", "value_levels", "k_codes",
                                             "v_codes", "k_recon", "v_recon")}
        lo, hi = bh * S * D, (bh + 1) * S * D
        for n in ("k_out", "v_out"):
            p, val = g[n]
            m = (p >= lo) & (p < hi)
            sub[n] = (p[m] - lo, val[m])
        compare(sub, r, what="bh=%d" % bh)
    kl, kth = g["key_levels"], g["key_thresh"]
    for step in range(64):
        kd = u16(inputs.student_t((BH, 1, D), 4, seed=5000 + step, device=d))
        vd = u16(inputs.student_t((BH, 1, D), 4, seed=6000 + step, device=d))
        gd = gpu_nuq(kd, vd, S + step, bits, 0.01, 8, 4, 0, kl, kth)
        if step % 16 == 0:
            rd = oracle.nuq_fit_quant(kd, vd, S + step, bits, 0.01, 8, 4, 0, kl, kth)
            compare(gd, rd, what="decode %d" % step)


@pytest.mark.parametrize("S,D,bits", [(16388, 32, 3), (32772, 32, 4), (16388, 128, 2)])
def test_key_fit_beyond_the_lds_limit(S, D, bits):
    """Key fits over 16,384 and 32,768 non-sink tokens (the bucketed samples
    live in the workspace): levels, thresholds and codes of sampled channels
    against the oracle's threshold and Lloyd fit on each channel's samples."""
    say("nuq long key fit", S, D, bits)
    BH, L, frac = 2, 1 << bits, 0.01
    k, v = t4((BH, S, D), 700 + S + D), t4((BH, S, D), 701 + S + D)
    g = gpu_nuq(k, v, 0, bits, frac, 8, 4, 1, want_recon=False)
    rng = np.random.default_rng(S + D)
    for bh in range(BH):
        for d in rng.choice(D, size=6, replace=False):
            col = np.ascontiguousarray(k[bh, 4:, d])
            tau = oracle.nuq_threshold(col, frac)
            a = np.abs(col.view(np.float16).astype(np.float64))
            inl = col[a <= float(np.uint16(tau).view(np.float16))]
            lev = oracle.nuq_fit(inl, L, 8)
            assert g["key_thresh"][bh, d] == tau, (bh, d)
            assert np.array_equal(g["key_levels"][bh, d].view(np.uint32), lev.view(np.uint32)), (bh, d)
            # codes of the channel's inliers: the nearest level (ties to the lower index)
            codes = np.unpackbits(g["k_codes"][bh], axis=-1, bitorder="little")[:, : D * bits]
            codes = (codes.reshape(S, D, bits) * (1 << np.arange(bits))).sum(-1)[:, d]
            for s in rng.choice(np.arange(4, S), size=40, replace=False):
                x = k[bh, s, d]
                if abs(float(np.uint16(x).view(np.float16))) <= float(np.uint16(tau).view(np.float16)):
                    assert codes[s] == oracle.nuq_nearest(x, lev), (bh, d, s)
                else:
                    assert codes[s] == 0, (bh, d, s)


def _adversarial_level_tables(L):
    """Ascending binary32 level tables whose neighbour midpoints sit on fp16
    values, just off them by less than a binary32 rounding of the sum (a tiny
    level next to a large one), on duplicates (empty cells), on signed zeros,
    in the fp16 subnormal range and near the top of the fp16 range."""
    t = 2.0 ** -40
    pats = [
        [-3.0, -1.0, -0.5, 0.25, 0.75, 1.25, 2.0, 4.0],
        [-100.0, -t, 1.5 * t, 1 - 2.0 ** -24, 3.0, 3 + 2.0 ** -20, 6.0, 6 + 2.0 ** -21],
        [-1.0, -1.0, 0.0, 0.0, 0.0, 2.0, 2.0, 3.0],
        [-(2.0 ** -20), -0.0, 0.0, 2.0 ** -24, 2.0 ** -23, 1e-3, 5e-3, 1.0],
        [-60000.0, -59999.99, -1000.5, -1000.25, -3.3, -3.2999, -0.1, -0.05],
        [1e-3, 1e-3 + 2.0 ** -30, 0.5, 0.5 + 2.0 ** -25, 65000.0, 65503.0, 65504.0, 65504.0],
    ]
    out = []
    for p in range(len(pats)):
        a = np.array(pats[p], np.float32)
        if L == 16:
            a = np.sort(np.concatenate([a, np.array(pats[(p + 1) % len(pats)], np.float32)]), kind="stable")
        elif L == 4:
            a = a[[0, 2, 4, 6]] if p % 2 == 0 else a[[1, 3, 5, 7]]
        elif L == 2:
            a = a[[1, 4]]
        assert np.all(a[1:] >= a[:-1])
        out.append(a)
    return out


def _fp16_sweep(x, n=2):
    """fp16 patterns of the n finite fp16 values on each side of fp16(x) and fp16(x) itself."""
    with np.errstate(over="ignore"):  # sweeps past the top of the range are dropped below
        g = np.float16(x)
        vals = [g]
        lo = hi = g
        for _ in range(n):
            lo = np.nextafter(lo, np.float16(-np.inf))
            hi = np.nextafter(hi, np.float16(np.inf))
            vals += [lo, hi]
        v = np.array(vals, np.float16)
    return v[np.isfinite(v)].view(np.uint16)


@pytest.mark.parametrize("bits", [3, 2, 4, 1])
def test_frozen_levels_at_adversarial_midpoints(bits):
    """Quantization against frozen key levels whose cut points are decided by
    the last bit: every input lies on or next to a midpoint of neighbouring
    levels, including midpoints that binary32 cannot hold. Codes, outliers and
    reconstructions must match the oracle's exact nearest-level rule."""
    say("nuq adversarial frozen levels", bits)
    L = 1 << bits
    BH, S, D = 2, 96, 128
    tables = _adversarial_level_tables(L)
    scales = [1.0, 8.0, 0.125]
    kl = np.zeros((BH, D, L), np.float32)
    kt = np.full((BH, D), 0x7bff, np.uint16)
    k = np.zeros((BH, S, D), np.uint16)
    rng = np.random.default_rng(77 + bits)
    for b in range(BH):
        for c in range(D):
            p = (c + b) % len(tables)
            sc = scales[(c // len(tables)) % 3]
            if p == 5 and sc > 1:
                sc = 1.0  # keep the top pattern inside the fp16 range
            lev = (tables[p].astype(np.float64) * sc).astype(np.float32)
            kl[b, c] = lev
            if c % 7 == 3:
                kt[b, c] = np.float16(2.0 * sc).view(np.uint16)  # some channels keep |x| > 2 sc exact
            cand = [_fp16_sweep((float(lev[j]) + float(lev[j + 1])) / 2) for j in range(L - 1)]
            cand += [_fp16_sweep(float(x), 1) for x in lev]
            cand = np.unique(np.concatenate(cand + [np.array([0x0000, 0x8000], np.uint16)]))
            col = np.resize(cand, S)
            rng.shuffle(col)
            k[b, :, c] = col
    v = t4((BH, S, D), 31 + bits)
    g = gpu_nuq(k, v, 300, bits, 0.01, 8, 4, 0, kl, kt)
    r = oracle.nuq_fit_quant(k, v, 300, bits, 0.01, 8, 4, 0, kl, kt)
    compare(g, r, what="adversarial frozen levels")


def _degenerate(case, shape, rng):
    """fp16 samples of the degenerate kinds above: few distinct values (empty
    cells and equal levels), zeros, signed zeros, the range's ends,
    subnormals, constants."""
    if case == "ties":
        x = rng.integers(-3, 4, size=shape).astype(np.float16)
    elif case == "zeros":
        x = np.zeros(shape, np.float16)
        x[..., ::7] = 1.5
    elif case == "signed_zeros":
        x = np.where(rng.random(shape) < 0.5, np.float16(0.0), np.float16(-0.0)).astype(np.float16)
        x[..., 3] = rng.standard_normal(shape[:-1]).astype(np.float16)
    elif case == "extremes":
        x = (rng.standard_t(4, size=shape) * 3000).clip(-65504, 65504).astype(np.float16)
        x[..., 5] = 65504
        x[..., 6] = -65504
    elif case == "subnormal":
        x = (rng.integers(-40, 40, size=shape) * 2.0 ** -24).astype(np.float16)
    else:
        x = np.full(shape, 0.25, np.float16)
    return x.view(np.uint16)


@pytest.mark.parametrize("case", ["ties", "zeros", "signed_zeros", "extremes", "subnormal", "const"])
@pytest.mark.parametrize("bits,D", [(3, 128), (2, 128), (4, 128), (1, 128), (3, 256), (2, 64)])
def test_many_tokens_degenerate_values(case, bits, D):
    """The many-token value fits (a quad of lanes per token at D = 128, lanes
    per token otherwise) on data with tied samples, so that cells go empty
    and neighbouring levels become equal: the level sort and the equal-level
    cut rule run, at several outlier fractions and iteration counts."""
    say("nuq many tokens degenerate", case, bits, D)
    BH, S = 33, 130
    rng = np.random.default_rng(500 + 10 * D + bits)
    v = _degenerate(case, (BH, S, D), rng)
    k = t4((BH, S, D), 60 + D + bits)
    for frac, iters in [(0.05, 8), (0.0, 3), (0.3, 1), (0.01, 0)]:
        g = gpu_nuq(k, v, 0, bits, frac, iters, 4, 1)
        r = oracle.nuq_fit_quant(k, v, 0, bits, frac, iters, 4, 1)
        compare(g, r, keys=["value_levels", "v_codes", "v_recon"],
                what="%s bits=%d D=%d frac=%g iters=%d" % (case, bits, D, frac, iters))


@pytest.mark.parametrize("D,bits", [(128, 3), (32, 2), (256, 4)])
def test_frozen_levels_dense_outliers(D, bits):
    """A prefill-sized call against given key levels and thresholds (not a
    small call): key outliers come from the per-row bitmap, so channels with a
    low threshold put many outliers in every row and in every key block
    (16384/D rows), the last block is ragged, and the first rows are sinks.
    Codes, reconstructions and both outlier lists match the oracle."""
    say("nuq frozen dense outliers", D, bits)
    L = 1 << bits
    rb = 16384 // D
    BH, S = 3, 2 * rb + 37
    k, v = t4((BH, S, D), 900 + D), t4((BH, S, D), 950 + D)
    fit = oracle.nuq_fit_quant(k[:, :64], v[:, :64], 0, bits, 0.05, 4, 0, 1)  # levels from a short fit
    kl = fit["key_levels"]
    kt = fit["key_thresh"].copy()
    kt[:, ::3] = np.float16(0.5).view(np.uint16)   # about half of these channels' samples are outliers
    kt[:, 1::5] = np.float16(0.0).view(np.uint16)  # every nonzero sample of these is one
    g = gpu_nuq(k, v, 0, bits, 0.03, 8, 4, 0, kl, kt)
    r = oracle.nuq_fit_quant(k, v, 0, bits, 0.03, 8, 4, 0, kl, kt)
    assert len(r["k_out"][0]) > BH * S * D // 8, "the case must be dense in key outliers"
    compare(g, r, what="frozen dense outliers")
