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
NuqCacheModel: ["veloxquant_mlx.cache.kvquant_cache module", KVQuantKVCache]
  the first call of a sequence fits and freezes the key tables and keeps
  its first n_sink tokens exact; later calls reuse the frozen key state,
  except that with refit_interval = N > 0 every N-th call after the first
  fits the key tables again from that call's tokens (level lifecycle: levels
  re-fit every N decode steps from the most recent token); trimming to
  empty starts over; a partial trim keeps the key state.
"""
from __future__ import annotations

import numpy as np

from . import kivi_round_trip, nuq_fit_quant


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
