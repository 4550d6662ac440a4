"""Pins of the CPU cache-lifecycle models against what the pages state.

["veloxquant_mlx.cache.kivi_cache", KIVIKVCache]: one-shot prefill and
token-by-token decode quantize the same positions with the same groups
(_quantization_boundary); the fp16 residual holds at most
residual_length + group_size - 1 tokens (residual_fp16_bytes); rows
quantized again after a trim differ from their input by at most one
quantization step (_rollback_frontier); the byte accounting equals the size
of the packed codes plus one fp16 (scale, zero) pair per group
(_quantized_bytes), checked here against the arrays the oracle's round trip
actually emits.
["veloxquant_mlx.cache.kvquant_cache module", KVQuantKVCache.trim]: trimming
to empty starts a new sequence (sinks and a fresh key fit); a partial trim
keeps the frozen key state.
"""
import numpy as np
import pytest

import oracle
from oracle.caches import KiviCacheModel, NuqCacheModel


def _kv(B, H, S, D, seed):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((B, H, S, D)).astype(np.float16)
    k[:, :, :, 3] *= 8  # a high-variance key channel
    v = (rng.standard_normal((B, H, S, D)) * 0.5).astype(np.float16)
    return k.view(np.uint16), v.view(np.uint16)


def _feed(model, k, v, sizes):
    t = 0
    for n in sizes:
        model.update(k[:, :, t:t + n], v[:, :, t:t + n])
        t += n
    assert t == k.shape[2]
    return model


@pytest.mark.parametrize("bits", [2, 4])
def test_kivi_chunking_independence(bits):
    B, H, S, D = 1, 2, 700, 64
    k, v = _kv(B, H, S, D, 1)
    rng = np.random.default_rng(2)
    chunks = []
    while sum(chunks) < S:
        chunks.append(int(min(rng.integers(1, 98), S - sum(chunks))))
    runs = [_feed(KiviCacheModel(bits), k, v, s) for s in ([S], [1] * S, chunks, [129, 1, 1, 569])]
    ref = runs[0]
    assert ref.nq == ((S - 128) // 32) * 32
    for m in runs[1:]:
        assert m.nq == ref.nq
        assert np.array_equal(m.k, ref.k) and np.array_equal(m.v, ref.v)
        assert (m.key_bytes, m.value_bytes, m.residual_bytes) == (ref.key_bytes, ref.value_bytes, ref.residual_bytes)


def test_kivi_residual_window_bound():
    B, H, D, R, gs = 1, 1, 32, 128, 32
    k, v = _kv(B, H, 600, D, 3)
    m = KiviCacheModel(2, gs, R)
    for t in range(600):
        m.update(k[:, :, t:t + 1], v[:, :, t:t + 1])
        res = m.offset - m.nq
        assert min(m.offset, R) <= res <= R + gs - 1
        assert m.nq % gs == 0
        assert m.residual_bytes == res * D * 2 * 2 * H * B


def test_kivi_packed_bytes_match_emitted_arrays():
    """Every flush is charged exactly the bytes of the packed codes the round
    trip emits plus 4 bytes (fp16 scale + fp16 zero) per emitted group."""
    B, H, D, bits = 2, 3, 64, 2
    k, v = _kv(B, H, 1000, D, 4)
    m = KiviCacheModel(bits)
    t, kb, vb = 0, 0, 0
    for n in (300, 7, 64, 129, 500):
        before = m.nq
        m.update(k[:, :, t:t + n], v[:, :, t:t + n])
        t += n
        if m.nq > before:
            _, kc, ks, _ = oracle.kivi_round_trip(m.k, before, m.nq, 1, bits, 32, want_params=True)
            _, vc, vs, _ = oracle.kivi_round_trip(m.v, before, m.nq, 0, bits, 32, want_params=True)
            kb += kc.nbytes + ks.size * 4
            vb += vc.nbytes + vs.size * 4
        assert (m.key_bytes, m.value_bytes) == (kb, vb)
    assert m.key_fp16 == m.value_fp16 == B * H * t * D * 2


@pytest.mark.parametrize("bits", [2, 4])
def test_kivi_trim_rollback_within_one_step(bits):
    """Prefill 400 (frontier 256), trim 170 (length 230, frontier back to 224),
    append 300 (frontier 384): rows 224..229 are quantized twice, with
    different key groups; each stays within one quantization step of its
    input, and every count returns to that of an untrimmed history."""
    B, H, D, gs = 1, 2, 64, 32
    k, v = _kv(B, H, 700, D, 5)
    m = KiviCacheModel(bits)
    m.update(k[:, :, :400], v[:, :, :400])
    assert m.nq == 256
    _, _, s1k, _ = oracle.kivi_round_trip(k[:, :, :400], 0, 256, 1, bits, gs, want_params=True)
    _, _, s1v, _ = oracle.kivi_round_trip(v[:, :, :400], 0, 256, 0, bits, gs, want_params=True)
    assert m.trim(170) == 170 and m.offset == 230 and m.nq == 224
    once_k = m.k[:, :, 224:230].copy()
    once_v = m.v[:, :, 224:230].copy()
    newk = np.concatenate([once_k, k[:, :, 230:530]], axis=2)
    m.update(k[:, :, 230:530], v[:, :, 230:530])
    assert m.nq == 384
    _, _, s2k, _ = oracle.kivi_round_trip(np.concatenate([m.k[:, :, :224] * 0, newk], axis=2), 224, 384, 1, bits, gs,
                                          want_params=True)
    f16 = lambda a: a.view(np.float16).astype(np.float64)
    x_k, y_k = f16(k[:, :, 224:230]), f16(m.k[:, :, 224:230])
    x_v, y_v = f16(v[:, :, 224:230]), f16(m.v[:, :, 224:230])
    step_k = np.maximum(s1k[:, :, 7:8, :], s2k[:, :, 0:1, :]).astype(np.float64)   # group 7 of flush 1, group 0 of flush 2
    assert np.all(np.abs(y_k - x_k) <= step_k * (1 + 2 ** -10) + 2 ** -10 * np.abs(x_k))
    _, _, s2v, _ = oracle.kivi_round_trip(once_v, 0, 6, 0, bits, gs, want_params=True)
    step_v = np.maximum(s1v[:, :, 224:230, :].repeat(gs, axis=3), s2v.repeat(gs, axis=3)).astype(np.float64)
    assert np.all(np.abs(y_v - x_v) <= step_v * (1 + 2 ** -10) + 2 ** -10 * np.abs(x_v))
    straight = KiviCacheModel(bits)
    straight.update(k[:, :, :530], v[:, :, :530])
    assert (m.nq, m.offset) == (straight.nq, straight.offset)
    assert (m.key_bytes, m.value_bytes, m.residual_bytes) == \
        (straight.key_bytes, straight.value_bytes, straight.residual_bytes)


def test_nuq_trim_to_empty_starts_a_new_sequence():
    B, H, D = 1, 2, 32
    k1, v1 = _kv(B, H, 60, D, 6)
    k2, v2 = _kv(B, H, 50, D, 7)
    a = NuqCacheModel(3, 0.05, 8, 4)
    a.update(k1[:, :, :40], v1[:, :, :40])
    a.update(k1[:, :, 40:41], v1[:, :, 40:41])
    assert a.trim(41) == 41 and a.offset == 0
    a.update(k2[:, :, :45], v2[:, :, :45])
    a.update(k2[:, :, 45:46], v2[:, :, 45:46])
    b = NuqCacheModel(3, 0.05, 8, 4)
    b.update(k2[:, :, :45], v2[:, :, :45])
    b.update(k2[:, :, 45:46], v2[:, :, 45:46])
    assert np.array_equal(a.k, b.k) and np.array_equal(a.v, b.v)
    assert np.array_equal(a.key_levels.view(np.uint32), b.key_levels.view(np.uint32))
    assert (a.sink_kept, a.outlier_count) == (b.sink_kept, b.outlier_count) == (4, b.outlier_count)
    # the restarted sequence kept its sinks exact
    assert np.array_equal(a.k[:, :, :4], k2[:, :, :4])


def test_nuq_partial_trim_keeps_frozen_keys():
    B, H, D = 1, 2, 32
    k, v = _kv(B, H, 80, D, 8)
    m = NuqCacheModel(3, 0.05, 8, 4)
    m.update(k[:, :, :70], v[:, :, :70])
    lev, thr = m.key_levels.copy(), m.key_thresh.copy()
    assert m.trim(20) == 20 and m.offset == 50
    m.update(k[:, :, 70:71], v[:, :, 70:71])
    assert np.array_equal(m.key_levels.view(np.uint32), lev.view(np.uint32))
    r = oracle.nuq_fit_quant(k[:, :, 70:71].reshape(2, 1, D), v[:, :, 70:71].reshape(2, 1, D), 50, 3, 0.05, 8, 4, 0,
                             lev, thr)
    assert np.array_equal(m.k[:, :, 50:51].reshape(2, 1, D), r["k_recon"])
    assert m.sink_kept == 4


def test_nuq_refit_interval_refits_from_the_latest_call():
    """["kvquant_cache module", level lifecycle] with a positive refit
    interval N the key levels are fit again every N decode steps from the
    most recent token(s): the tables change exactly at decode calls N, 2N,
    and equal a fit of that call's tokens alone; in between they are reused;
    interval 0 never refits."""
    B, H, D, N = 1, 2, 32, 3
    k, v = _kv(B, H, 90, D, 9)
    frozen = NuqCacheModel(3, 0.05, 8, 4, refit_interval=0)
    m = NuqCacheModel(3, 0.05, 8, 4, refit_interval=N)
    for c in (frozen, m):
        c.update(k[:, :, :80], v[:, :, :80])
    lev0 = m.key_levels.copy()
    for step in range(1, 8):
        t = 79 + step
        prev = m.key_levels.copy()
        for c in (frozen, m):
            c.update(k[:, :, t:t + 1], v[:, :, t:t + 1])
        assert np.array_equal(frozen.key_levels.view(np.uint32), lev0.view(np.uint32))
        if step % N == 0:
            r = oracle.nuq_fit_quant(k[:, :, t:t + 1].reshape(2, 1, D), v[:, :, t:t + 1].reshape(2, 1, D), t, 3,
                                     0.05, 8, 4, 1)
            assert np.array_equal(m.key_levels.view(np.uint32), r["key_levels"].view(np.uint32))
            assert not np.array_equal(m.key_levels.view(np.uint32), prev.view(np.uint32))
        else:
            assert np.array_equal(m.key_levels.view(np.uint32), prev.view(np.uint32))
    assert m.sink_kept == frozen.sink_kept == 4


def test_nuq_refit_from_one_token_reconstructs_it_exactly():
    """A per-channel fit over a single sample: no outlier (k = floor(frac*1)
    = 0), every quantile and every Lloyd level equals the sample, so the
    token's keys reconstruct exactly."""
    B, H, D = 1, 2, 32
    k, v = _kv(B, H, 12, D, 10)
    m = NuqCacheModel(3, 0.05, 8, 4, refit_interval=1)
    m.update(k[:, :, :10], v[:, :, :10])
    m.update(k[:, :, 10:11], v[:, :, 10:11])
    lev = m.key_levels.reshape(2, D, 8)
    x = k[:, :, 10].reshape(2, D).view(np.float16).astype(np.float32)
    assert np.array_equal(lev, np.repeat(x[:, :, None], 8, axis=2))
    assert np.array_equal(m.k[:, :, 10], k[:, :, 10])


# ------------------------------------------------------------------ packed KIVI cache model
from oracle.caches import KiviPackedCacheModel  # noqa: E402


def _store_rows(m):
    (kc, ks, kz), (vc, vs, vz) = m.store
    ng = -(-m.nq // m.gs)
    return [kc[:, :, :m.nq], ks[:, :, :ng], kz[:, :, :ng], vc[:, :, :m.nq], vs[:, :, :m.nq], vz[:, :, :m.nq]]


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_kivi_packed_cache_reduces_to_one_pack(bits):
    """Without trims, the cache's fp16 view is the packed round trip of the
    quantized prefix done in one go (flushes are group-aligned, so they cut
    the same key groups) followed by the untouched residual window; and the
    flush sizes do not matter."""
    B, H, D = 2, 2, 64
    k, v = _kv(B, H, 700, D, 11 + bits)
    a = _feed(KiviPackedCacheModel(bits), k, v, [700])
    b = _feed(KiviPackedCacheModel(bits), k, v, [300, 1, 1, 33, 64, 1, 300])
    c = _feed(KiviPackedCacheModel(bits), k, v, [1] * 700)
    nq = (700 - 128) // 32 * 32
    assert a.nq == b.nq == c.nq == nq
    for m in (b, c):
        for x, y in zip(_store_rows(a), _store_rows(m)):
            assert np.array_equal(x, y)
    fk, fv = c.fetch()
    for x, f, per_channel in ((k, fk, 1), (v, fv, 0)):
        codes, sc, zr = oracle.kivi_pack(x, 0, nq, per_channel, bits, 32)
        rec = oracle.kivi_unpack(codes, sc, zr, 0, nq, per_channel, bits, 32, D)
        assert np.array_equal(f[:, :, :nq], rec[:, :, :nq])
        assert np.array_equal(f[:, :, nq:], x[:, :, nq:])


def test_kivi_packed_cache_bytes_are_the_stored_rows():
    """The page's byte formula for the quantized prefix equals the rows of
    the packed arrays that hold it, at every step."""
    B, H, D, bits = 1, 3, 64, 2
    k, v = _kv(B, H, 900, D, 21)
    m, ref = KiviPackedCacheModel(bits), KiviCacheModel(bits)
    t = 0
    for n in (200, 1, 31, 1, 64, 300, 3, 300):
        m.update(k[:, :, t:t + n], v[:, :, t:t + n])
        ref.update(k[:, :, t:t + n], v[:, :, t:t + n])
        t += n
        assert m.nq == ref.nq
        assert m.packed_bytes() == (ref.key_bytes, ref.value_bytes)
        assert m.win[0].shape[2] == ref.offset - ref.nq <= 128 + 32 - 1


@pytest.mark.parametrize("bits", [2, 4])
def test_kivi_packed_cache_trim(bits):
    """A trim changes no value that is kept; below the frontier the tokens
    between the new frontier and the new length return to the window as
    their packed reconstructions; trimming to empty leaves nothing."""
    B, H, D = 1, 2, 64
    k, v = _kv(B, H, 800, D, 31 + bits)
    m = KiviPackedCacheModel(bits)
    m.update(k[:, :, :400], v[:, :, :400])
    assert m.nq == 256
    before = m.fetch()
    assert m.trim(30) == 30 and (m.n, m.nq) == (370, 256)        # into the window
    after = m.fetch()
    assert all(np.array_equal(x[:, :, :370], y) for x, y in zip(before, after))
    assert m.trim(140) == 140 and (m.n, m.nq) == (230, 224)      # into the quantized region
    after = m.fetch()
    assert all(np.array_equal(x[:, :, :230], y) for x, y in zip(before, after))
    assert np.array_equal(m.win[0], before[0][:, :, 224:230])
    m.update(k[:, :, 230:600], v[:, :, 230:600])
    assert m.nq == (600 - 128) // 32 * 32
    straight = _feed(KiviPackedCacheModel(bits), k[:, :, :600], v[:, :, :600], [600])
    assert m.packed_bytes() == straight.packed_bytes()
    # rows quantized before the trim keep their stored values
    f, g = m.fetch(), straight.fetch()
    assert all(np.array_equal(x[:, :, :224], y[:, :, :224]) for x, y in zip(f, g))
    assert m.trim(10 ** 6) == 600 and m.n == 0 and m.win[0].shape[2] == 0
