"""Pins of the oracle's symmetric q8/q6/q4 quantizer, packing and storage arithmetic.

Source: MTPLX pull request #267, "feat(kv-cache): add q6 paged KV quantization"
(PR description: per-(token, head) symmetric quantizer with one fp16 scale,
qmax table, q6 bias and byte equations, packed_dim, storage arithmetic).
Each pin checks the oracle against something other than itself: the page's
printed values (tests/golden), an independent formulation (the q6 fields as
one little-endian bit string), numpy's float16/float64 arithmetic for closed
forms, or error bounds the definition implies.
"""
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")
QMAX = {8: 127, 6: 31, 4: 7}


def _read(name):
    rows = []
    for line in open(os.path.join(GOLD, name)):
        if line.strip() and not line.startswith("#"):
            rows.append(line.split())
    return rows


def _rows_with_codes(q, absmax_code):
    """fp16 rows whose codes are exactly q: scale 1.0 needs a +-qmax element."""
    q = np.asarray(q)
    pad = np.zeros((q.shape[0], 4), np.int64)
    pad[:, 0] = absmax_code
    return np.concatenate([q, pad], axis=1).astype(np.float16)


# ------------------------------------------------------------------ page values
def test_q6_pack_matches_page_worked_examples(orc):
    rows = _read("q6_pack_worked_examples.txt")
    u = np.array([[int(v) for v in r[:4]] for r in rows])
    expect = np.array([[int(v, 16) for v in r[4:]] for r in rows], np.uint8)
    x = _rows_with_codes(u - 32, 31)
    codes, scales = orc.sym_quant_rows(x, 6)
    assert np.all(scales == np.float16(1.0).view(np.uint16))
    assert np.array_equal(codes[:, :3], expect)


def test_storage_arithmetic_matches_page(orc):
    for r in _read("storage_arithmetic.txt"):
        if r[0] == "packed_dim":
            assert orc.packed_dim(int(r[1]), int(r[2])) == int(r[3])
        elif r[0] == "per_token_head":
            assert orc.sym_cache_bytes(1, 1, 1, 256, int(r[1])) == int(r[2])
        elif r[0] == "cache_gib":
            t, l, h, d, b = map(int, r[1:6])
            gib = orc.sym_cache_bytes(t, l, h, d, b) / 2 ** 30
            assert "%.2f" % gib == r[6]


def test_packed_dim_table_and_rejections(orc):
    assert orc.packed_dim(256, 8) == 256 and orc.packed_dim(256, 4) == 128
    assert orc.packed_dim(128, 6) == 96
    for D in (254, 255, 257, 6, 2):
        assert orc.packed_dim(D, 6) == -1  # q6 needs D % 4 == 0
    assert orc.packed_dim(255, 4) == -1
    for bits in (0, 1, 2, 3, 5, 7, 9, 16):
        assert orc.packed_dim(256, bits) == -1
        assert orc.sym_qmax(bits) == -1  # unknown widths are rejected, not mapped
    assert [orc.sym_qmax(b) for b in (8, 6, 4)] == [127, 31, 7]


# ------------------------------------------------------------------ exhaustive q6 packing
def test_q6_pack_exhaustive_equals_bitstring(orc):
    """Every valid field quadruple u in [1,63]^4 (63^4 = 15.8M groups)."""
    f = np.arange(1, 64)
    for u0 in range(1, 64):
        g = np.stack(np.meshgrid(np.full(1, u0), f, f, f, indexing="ij"), -1).reshape(-1, 4)
        x = _rows_with_codes(g - 32, 31)
        codes, _ = orc.sym_quant_rows(x, 6)
        v = g[:, 0] | (g[:, 1] << 6) | (g[:, 2] << 12) | (g[:, 3] << 18)
        le = np.stack([v & 255, (v >> 8) & 255, (v >> 16) & 255], 1).astype(np.uint8)
        assert np.array_equal(codes[:, :3], le)


def test_q6_unpack_exhaustive(orc):
    """Every 3-byte pattern unpacks to the four 6-bit fields of its bit string."""
    v = np.arange(2 ** 24, dtype=np.int64)
    b = np.stack([v & 255, (v >> 8) & 255, (v >> 16) & 255], 1).astype(np.uint8)
    q = orc.sym_unpack_rows(b, 4, 6)
    u = np.stack([(v >> (6 * i)) & 63 for i in range(4)], 1)
    assert np.array_equal(q, u - 32)


@pytest.mark.parametrize("bits", [8, 4])
def test_q8_q4_pack_roundtrip_all_codes(orc, bits):
    # layout is a reading (pages give only "one per byte" / "two per byte");
    # pinned here only as unpack(pack(q)) == q over every code pair.
    qm = QMAX[bits]
    c = np.arange(-qm, qm + 1)
    pairs = np.stack(np.meshgrid(c, c, indexing="ij"), -1).reshape(-1, 2)
    x = _rows_with_codes(np.concatenate([pairs, pairs], 1), qm)
    codes, _ = orc.sym_quant_rows(x, bits)
    assert np.array_equal(orc.sym_unpack_rows(codes, x.shape[1], bits)[:, :4],
                          np.concatenate([pairs, pairs], 1))
    if bits == 8:
        assert np.array_equal(codes[:, :2].view(np.int8), pairs)  # two's complement


# ------------------------------------------------------------------ quantizer invariants
def _data(rng, n, D, scale=1.0):
    x = rng.standard_normal((n, D)) * scale
    ch = rng.integers(0, D, size=3)
    x[:, ch] *= 10
    lap = rng.random(n) < 0.05
    x[lap] = rng.laplace(size=(lap.sum(), D)) * scale
    return x.astype(np.float16)


@pytest.mark.parametrize("bits", [8, 6, 4])
def test_sym_invariants(orc, bits):
    rng = np.random.default_rng(100 + bits)
    qm = QMAX[bits]
    x = np.concatenate([_data(rng, 3000, 256), _data(rng, 500, 256, 1e-2),
                        _data(rng, 500, 256, 300.0)])
    codes, sc = orc.sym_quant_rows(x, bits)
    q = orc.sym_unpack_rows(codes, 256, bits).astype(np.int64)
    s = sc.view(np.float16).astype(np.float64)
    xf = x.astype(np.float64)
    amax = np.abs(xf).max(1)
    # stored scale == RN16(absmax / qmax), computed independently in double
    assert np.array_equal(sc, (amax / qm).astype(np.float16).view(np.uint16))
    assert np.all(np.abs(q) <= qm)
    if bits == 6:  # biased fields never leave [1, 63]
        v = (codes.reshape(-1, 3).astype(np.int64) @ np.array([1, 256, 65536]))
        for i in range(4):
            f = (v >> (6 * i)) & 63
            assert f.min() >= 1 and f.max() <= 63
    # the absmax element lands on +-qmax (scale is a normal fp16 here)
    idx = np.abs(xf).argmax(1)
    assert np.array_equal(q[np.arange(len(q)), idx], np.sign(xf[np.arange(len(q)), idx]) * qm)
    # codes are taken against the STORED fp16 scale: equal to rint(x/s) in
    # double except within the reciprocal's rounding of a half-integer
    ref = np.clip(np.rint(xf / s[:, None]), -qm, qm)
    diff = ref != q
    frac = np.abs(xf / s[:, None] - np.floor(xf / s[:, None]) - 0.5)
    assert np.all(frac[diff] < 2.0 ** -15), frac[diff].max()
    assert diff.mean() < 1e-4
    # error bound in double: |x - q s| <= s (1/2 + 2^-16)
    err = np.abs(xf - q * s[:, None])
    assert np.all(err <= s[:, None] * (0.5 + 2.0 ** -16))
    # dequant == RN16(q * s) with numpy's own float16 rounding
    deq = orc.sym_dequant_rows(codes, sc, 256, bits)
    assert np.array_equal(deq, (q * s[:, None]).astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("bits", [8, 6, 4])
def test_sym_odd_symmetry(orc, bits):
    rng = np.random.default_rng(5)
    x = _data(rng, 2000, 128)
    c1, s1 = orc.sym_quant_rows(x, bits)
    c2, s2 = orc.sym_quant_rows(-x, bits)
    assert np.array_equal(s1, s2)
    assert np.array_equal(orc.sym_unpack_rows(c1, 128, bits), -orc.sym_unpack_rows(c2, 128, bits))


@pytest.mark.parametrize("bits", [8, 6, 4])
def test_sym_degenerate_rows(orc, bits):
    qm = QMAX[bits]
    x = np.zeros((4, 64), np.float16)
    x[1, 7] = 3.5           # single nonzero -> that element at +qmax, rest 0
    x[2, :] = -2.0          # constant row -> all -qmax
    x[3, 5] = np.float16(2.0 ** -24)  # scale underflows to 0 -> all-zero codes
    codes, sc = orc.sym_quant_rows(x, bits)
    q = orc.sym_unpack_rows(codes, 64, bits)
    assert sc[0] == 0 and np.all(q[0] == 0)
    assert q[1, 7] == qm and np.count_nonzero(q[1]) == 1
    assert np.all(q[2] == -qm)
    assert sc[3] == 0 and np.all(q[3] == 0)
    deq = orc.sym_dequant_rows(codes, sc, 64, bits)
    assert np.all(deq[0] == 0) and np.all(deq[3] == 0)  # +0, not -0
    assert np.all(deq[2].view(np.float16) == np.float16(-2.0))


def test_paged_write_read_roundtrip(orc):
    """Paged geometry is a reading (parity unpinned by the pages); pinned here
    only as: a paged write then a paged read equals the row-wise round trip."""
    rng = np.random.default_rng(11)
    T, H, D, P = 100, 4, 64, 8
    x = _data(rng, T * H, D).reshape(T, H, D)
    num_pages = 20
    perm = rng.permutation(num_pages)
    bt = np.full((2, 10), -1, np.int32)
    bt[0, :7] = perm[:7]
    bt[1, :7] = perm[7:14]
    lens = np.array([52, 48], np.int32)
    slot = np.concatenate([bt[0, np.arange(52) // P] * P + np.arange(52) % P,
                           bt[1, np.arange(48) // P] * P + np.arange(48) % P]).astype(np.int32)
    for bits in (8, 6, 4):
        pd = orc.packed_dim(D, bits)
        codes = np.zeros((num_pages * P, H, pd), np.uint8)
        scales = np.zeros((num_pages * P, H), np.uint16)
        orc.sym_quant_paged(x, bits, slot, codes, scales)
        out = orc.sym_dequant_paged(codes, scales, P, D, bits, bt, lens, 60)
        rt = orc.sym_dequant_rows(*orc.sym_quant_rows(x, bits), D, bits)
        assert np.array_equal(out[0, :52], rt[:52])
        assert np.array_equal(out[1, :48], rt[52:])
        assert np.all(out[0, 52:] == 0) and np.all(out[1, 48:] == 0)
