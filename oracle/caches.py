"""CPU models of the cache lifecycles -- test infrastructure only (imported by
tests/ alone, never by the library).

Plain host implementations, written from the pages, of the two cache objects
the kernels serve. Arrays are fp16 bit patterns (uint16) [B][H][S][D]; each
quantization step calls the oracle's own round trip / NUQ fit.

KiviCacheModel: ["veloxquant_mlx.cache.kivi_cache", KIVIKVCache] tokens age
  out of a fp16 residual window of `residual_length` newest tokens; the
  eligible prefix is flushed only up to a multiple of the group size (keys
  are grouped along tokens, so a flush must hold whole groups); trimming
  pulls the flush frontier down to the group boundary at or below the new
  length; bytes of a quantized stretch of n tokens are b-bit codes plus one
  fp16 (scale, zero) pair per group (_quantized_bytes / _account_bytes).
KiviPackedCacheModel: the same lifecycle with the quantized tokens held only
  as packed storage (b-bit codes plus one fp16 (scale, zero) pair per group,
  kivi_pack), the memory the page's byte accounting charges for (module
  docstring, memory-savings caveat). fp16 is kept for the residual window
  only; the fp16 view is rebuilt with kivi_unpack. A trim below the frontier
  brings the tokens between the new frontier and the new length back into
  the window as their packed reconstructions (they were quantized once and
  are quantized again when they age out).
NuqCacheModel: ["veloxquant_mlx.cache.kvquant_cache module", KVQuantKVCache]
  the first call of a sequence fits and freezes the key tables and keeps
  its first n_sink tokens exact; later calls reuse the frozen key state,
  except that with refit_interval = N > 0 every N-th call after the first
  fits the key tables again from that call's tokens (level lifecycle: the
  page's periodic re-fit on recent tokens, read as a re-fit on the
  tokens of every N-th call); trimming to
  empty starts over; a partial trim keeps the key state.
"""
from __future__ import annotations

import numpy as np

from . import kivi_pack, kivi_param_shape, kivi_round_trip, kivi_unpack, nuq_fit_quant


class KiviCacheModel:
    def __init__(self, bits=2, group_size=32, residual_length=128):
        self.b, self.gs, self.R = bits, group_size, residual_length
        self.k = self.v = None
        self.nq = 0
        self.key_bytes = self.value_bytes = 0          # packed-storage estimate
        self.key_fp16 = self.value_fp16 = 0
        self.residual_bytes = 0

    @property
    def offset(self):
        return 0 if self.k is None else self.k.shape[2]

    def _packed(self, n, B, H, D):
        # b-bit codes of n tokens x D channels, rounded up to whole bytes per (b, h)
        code = -(-(n * D * self.b) // 8) * B * H
        # keys: one (scale, zero) fp16 pair per channel and group of gs tokens
        key_groups = -(-n // self.gs) * D
        # values: one pair per token and group of gs channels
        value_groups = n * -(-D // self.gs)
        return code + key_groups * 4 * B * H, code + value_groups * 4 * B * H

    def update(self, keys, values):
        B, H, S, D = keys.shape
        self.k = keys.copy() if self.k is None else np.concatenate([self.k, keys], axis=2)
        self.v = values.copy() if self.v is None else np.concatenate([self.v, values], axis=2)
        eligible = max(0, self.offset - self.R)
        frontier = eligible - eligible % self.gs
        if frontier > self.nq:
            self.k = kivi_round_trip(self.k, self.nq, frontier, 1, self.b, self.gs)[0]
            self.v = kivi_round_trip(self.v, self.nq, frontier, 0, self.b, self.gs)[0]
            kb, vb = self._packed(frontier - self.nq, B, H, D)
            self.key_bytes += kb
            self.value_bytes += vb
            self.nq = frontier
        self.residual_bytes = (self.offset - self.nq) * B * H * D * 2 * 2
        self.key_fp16 += B * H * S * D * 2
        self.value_fp16 += B * H * S * D * 2
        return self.k, self.v

    def trim(self, n):
        t = min(max(n, 0), self.offset)
        if t == 0:
            return 0
        B, H, _, D = self.k.shape
        keep = self.offset - t
        self.k = self.k[:, :, :keep].copy()
        self.v = self.v[:, :, :keep].copy()
        back = min(self.nq, keep - keep % self.gs)
        if back < self.nq:
            kb, vb = self._packed(self.nq - back, B, H, D)
            self.key_bytes = max(0, self.key_bytes - kb)
            self.value_bytes = max(0, self.value_bytes - vb)
            self.nq = back
        self.key_fp16 = max(0, self.key_fp16 - B * H * t * D * 2)
        self.value_fp16 = max(0, self.value_fp16 - B * H * t * D * 2)
        self.residual_bytes = (self.offset - self.nq) * B * H * D * 2 * 2
        return t


class KiviPackedCacheModel:
    def __init__(self, bits=2, group_size=32, residual_length=128):
        self.b, self.gs, self.R = bits, group_size, residual_length
        self.n = 0            # tokens held
        self.nq = 0           # quantized prefix
        self.win = None       # (keys, values) fp16 bits [B][H][n - nq][D]
        self.store = None     # (key (codes, scale, zero), value (codes, scale, zero)), S_cap = self.cap
        self.cap = 0

    def _grow(self, need, B, H, D):
        if need <= self.cap:
            return
        new = []
        for per_channel in (1, 0):
            shp = kivi_param_shape(B, H, need, D, per_channel, self.gs)
            arrs = (np.zeros((B, H, need, D * self.b // 8), np.uint8), np.zeros(shp, np.uint16),
                    np.zeros(shp, np.uint16))
            if self.store is not None:
                for a, o in zip(arrs, self.store[1 - per_channel]):
                    a[:, :, : o.shape[2]] = o
            new.append(arrs)
        self.store, self.cap = new, need

    def update(self, keys, values):
        B, H, S, D = keys.shape
        if self.win is None:
            self.win = (keys.copy(), values.copy())
        else:
            self.win = (np.concatenate([self.win[0], keys], 2), np.concatenate([self.win[1], values], 2))
        self.n += S
        eligible = max(0, self.n - self.R)
        frontier = eligible - eligible % self.gs
        if frontier > self.nq:
            self._grow(frontier, B, H, D)
            for side, per_channel in ((0, 1), (1, 0)):
                full = np.zeros((B, H, self.cap, D), np.uint16)   # token t in row t
                full[:, :, self.nq:frontier] = self.win[side][:, :, : frontier - self.nq]
                kivi_pack(full, self.nq, frontier, per_channel, self.b, self.gs, into=self.store[side])
            self.win = tuple(w[:, :, frontier - self.nq:].copy() for w in self.win)
            self.nq = frontier
        return self.fetch()

    def fetch(self):
        B, H, _, D = self.win[0].shape
        out = []
        for side, per_channel in ((0, 1), (1, 0)):
            x = np.zeros((B, H, self.n, D), np.uint16)
            if self.nq:
                codes, sc, zr = self.store[side]
                x[:, :, : self.nq] = kivi_unpack(codes, sc, zr, 0, self.nq, per_channel, self.b, self.gs, D)[
                    :, :, : self.nq]
            x[:, :, self.nq:] = self.win[side]
            out.append(x)
        return out[0], out[1]

    def trim(self, n):
        t = min(max(n, 0), self.n)
        if t == 0:
            return 0
        keep = self.n - t
        back = min(self.nq, keep - keep % self.gs)
        if back < self.nq:
            B, H, _, D = self.win[0].shape
            upto = min(self.nq, keep)
            win = []
            for side, per_channel in ((0, 1), (1, 0)):
                codes, sc, zr = self.store[side]
                rec = kivi_unpack(codes, sc, zr, back, upto, per_channel, self.b, self.gs, D)[:, :, back:upto]
                win.append(np.concatenate([rec, self.win[side][:, :, : max(0, keep - self.nq)]], 2))
            self.win = tuple(win)
            self.nq = back
        else:
            self.win = tuple(w[:, :, : keep - self.nq].copy() for w in self.win)
        self.n = keep
        return t

    def packed_bytes(self):
        """(key, value) bytes of the packed rows that hold the quantized prefix."""
        if self.nq == 0:
            return 0, 0
        (kc, ks, kz), (vc, vs, vz) = self.store
        ng = -(-self.nq // self.gs)
        kb = kc[:, :, : self.nq].nbytes + ks[:, :, :ng].nbytes + kz[:, :, :ng].nbytes
        vb = vc[:, :, : self.nq].nbytes + vs[:, :, : self.nq].nbytes + vz[:, :, : self.nq].nbytes
        return kb, vb


class NuqCacheModel:
    def __init__(self, bits=3, outlier_fraction=0.01, lloyd_iters=8, n_sink=4, refit_interval=0):
        self.bits, self.frac, self.iters, self.n_sink = bits, outlier_fraction, lloyd_iters, n_sink
        self.refit_interval = refit_interval
        self.start()

    def start(self):
        self.k = self.v = None
        self.key_levels = self.key_thresh = None
        self.outlier_count = 0
        self.sink_kept = 0
        self.last = None
        self.since_fit = 0

    @property
    def offset(self):
        return 0 if self.k is None else self.k.shape[2]

    def update(self, keys, values):
        B, H, S, D = keys.shape
        first = self.key_levels is None
        fit = first or (self.refit_interval > 0 and self.since_fit + 1 == self.refit_interval)
        r = nuq_fit_quant(keys.reshape(B * H, S, D), values.reshape(B * H, S, D), self.offset, self.bits,
                          self.frac, self.iters, self.n_sink, int(fit), self.key_levels, self.key_thresh)
        if fit:
            self.key_levels, self.key_thresh = r["key_levels"], r["key_thresh"]
        if first:
            self.sink_kept += min(self.n_sink, S)
        self.since_fit = 0 if fit else self.since_fit + 1
        self.outlier_count += len(r["k_out"][0]) + len(r["v_out"][0])
        kr = r["k_recon"].reshape(B, H, S, D)
        vr = r["v_recon"].reshape(B, H, S, D)
        self.k = kr if self.k is None else np.concatenate([self.k, kr], axis=2)
        self.v = vr if self.v is None else np.concatenate([self.v, vr], axis=2)
        self.last = r
        return self.k, self.v

    def trim(self, n):
        t = min(max(n, 0), self.offset)
        if t == self.offset and t > 0:
            self.start()
        elif t > 0:
            keep = self.offset - t
            self.k = self.k[:, :, :keep].copy()
            self.v = self.v[:, :, :keep].copy()
        return t
