"""Cache objects over the libkvq kernels: the host-side state machines that
decide what to quantize when, and keep the byte accounting.

Every quantization step runs in the HIP kernels (kvq_kivi_quant_dequant,
kvq_nuq_fit_quant, kvq_quant_sym / kvq_dequant_sym); this module only
appends incoming tokens to device-resident buffers (PyTorch memory), moves
frontiers, hands out pages and counts bytes. KIVI / NUQ tensors are fp16
[B][H][S][D] on the current HIP device.

KiviCache  ["veloxquant_mlx.cache.kivi_cache", class KIVIKVCache:
            update_and_fetch, _quantization_boundary, trim with
            _rollback_frontier / _rollback_bytes, _quantized_bytes,
            _account_bytes and the reporting properties]
NuqCache   ["veloxquant_mlx.cache.kvquant_cache module", class
            KVQuantKVCache: update_and_fetch, trim, and the outlier_count,
            sink_kept, key_levels, compressed_*_bytes and effective_bits
            properties]
PagedSymCache [MTPLX pull request #267, "feat(kv-cache): add q6 paged KV
            quantization": paged q8/q6/q4 storage sized by packed_dim; the
            page allocator, appends and trims are a reading, the page
            describes only the storage]
"""
from __future__ import annotations

import math

from . import kvq


def _grow(buf, B, H, need, D, step, like):
    """fp16 [B][H][cap][D] buffer with cap >= need (cap a multiple of step)."""
    import torch

    if buf is not None and buf.shape[2] >= need:
        return buf
    cap = ((need + step - 1) // step) * step
    nb = torch.empty((B, H, cap, D), dtype=torch.float16, device=like.device)
    if buf is not None:
        nb[:, :, : buf.shape[2]].copy_(buf)
    return nb


class KiviCache:
    """KIVI cache: the newest tokens stay fp16 in a residual window, older
    ones are round-tripped in place, keys per channel and values per token,
    in flushes aligned to the group size. The live buffers stay fp16; the
    compressed_* figures are the packed-storage estimate the page defines
    (b-bit codes plus one fp16 (scale, zero) pair per group)."""

    def __init__(self, bits: int = 2, group_size: int = 32, residual_length: int = 128, step: int = 256):
        if bits not in (2, 4, 8):
            raise kvq.KvqError(kvq.KVQ_ERR_BITS, "KIVI bits must be 2, 4 or 8")
        self.bits, self.group_size, self.residual_length, self.step = bits, group_size, residual_length, step
        self.keys = self.values = None
        self.offset = 0
        self.n_quantized = 0
        self._shape = None  # (B, H, D)
        self._kc = self._vc = self._kf = self._vf = self._res = 0
        self.tokens_seen = 0

    # ------------------------------------------------------------- lifecycle
    def update_and_fetch(self, keys, values):
        B, H, S, D = (int(x) for x in keys.shape)
        if self._shape is not None and self._shape != (B, H, D):
            raise kvq.KvqError(kvq.KVQ_ERR_SHAPE, "batch, heads and head_dim are fixed for a cache")
        self._shape = (B, H, D)
        end = self.offset + S
        self.keys = _grow(self.keys, B, H, end, D, self.step, keys)
        self.values = _grow(self.values, B, H, end, D, self.step, values)
        self.keys[:, :, self.offset:end].copy_(keys)
        self.values[:, :, self.offset:end].copy_(values)
        self.offset = end
        hi = kvq.kvq_kivi_boundary(self.offset, self.residual_length, self.group_size)
        n_new = hi - self.n_quantized
        if n_new > 0:
            kvq.kvq_kivi_quant_dequant(self.keys, self.values, self.n_quantized, hi, self.bits, self.group_size)
            self.n_quantized = hi
            k, v = self.packed_bytes(n_new)
            self._kc += k
            self._vc += v
        self._res = self._fp16_bytes(self.offset - self.n_quantized)
        self._kf += B * H * S * D * 2
        self._vf += B * H * S * D * 2
        self.tokens_seen += S
        return self.keys[:, :, : self.offset], self.values[:, :, : self.offset]

    def trim(self, n: int) -> int:
        """Drop the newest n tokens; the quantization frontier falls back to the
        last group boundary at or below the new length (rows between it and the
        new length were quantized once and will be quantized again), and the
        byte accounting of the removed tokens is undone."""
        t = max(0, min(int(n), self.offset))
        if t == 0:
            return 0
        self.offset -= t
        gs = self.group_size
        new_nq = min(self.n_quantized, (self.offset // gs) * gs)
        rolled = self.n_quantized - new_nq
        self.n_quantized = new_nq
        B, H, D = self._shape
        if rolled > 0:
            k, v = self.packed_bytes(rolled)
            self._kc = max(0, self._kc - k)
            self._vc = max(0, self._vc - v)
        self._kf = max(0, self._kf - B * H * t * D * 2)
        self._vf = max(0, self._vf - B * H * t * D * 2)
        self.tokens_seen = max(0, self.tokens_seen - t)
        self._res = self._fp16_bytes(self.offset - self.n_quantized)
        return t

    # ------------------------------------------------------------- accounting
    def packed_bytes(self, n: int):
        """(key, value) bytes of n quantized tokens stored packed: codes at
        `bits` per element, one fp16 scale and one fp16 zero per group (keys:
        per channel over groups of tokens; values: per token over groups of
        channels)."""
        B, H, D = self._shape
        gs, b = self.group_size, self.bits
        codes = math.ceil(n * D * b / 8) * H * B
        k = codes + math.ceil(n / gs) * D * 2 * 2 * H * B
        v = codes + n * math.ceil(D / gs) * 2 * 2 * H * B
        return k, v

    def _fp16_bytes(self, n_tokens: int) -> int:
        B, H, D = self._shape
        return n_tokens * D * 2 * 2 * H * B  # keys + values

    @property
    def compressed_key_bytes(self) -> int:
        return self._kc

    @property
    def compressed_value_bytes(self) -> int:
        return self._vc

    @property
    def fp16_key_bytes(self) -> int:
        return self._kf

    @property
    def fp16_value_bytes(self) -> int:
        return self._vf

    @property
    def residual_fp16_bytes(self) -> int:
        return self._res

    @property
    def assigned_avg_bits(self) -> float:
        return float(self.bits)

    @property
    def effective_compression_ratio(self) -> float:
        full = self._kf + self._vf
        packed = self._kc + self._vc + self._res
        return 1.0 if full == 0 or packed == 0 else full / packed


class NuqCache:
    """KVQuant-style NUQ cache: the first call of a sequence fits and freezes
    the per-channel key levels and |key| thresholds (and keeps its first
    n_sink tokens exact); every call fits fresh per-token value levels; the
    buffers hold the dequantized K/V. With refit_interval = N > 0 the key
    tables are fit again from the tokens of every N-th call after the first
    ("re-fit every N decode steps from the most recent token",
    ["veloxquant_mlx.cache.kvquant_cache module", level lifecycle]).
    Byte accounting (a reading of the page's description): codes at `bits`
    per element, fp32 level tables and fp16 key thresholds (one key table
    held at a time), 6 bytes per outlier (fp16 value + int32 position),
    fp16 sink tokens."""

    def __init__(self, bits: int = 3, outlier_fraction: float = 0.01, lloyd_iters: int = 8, n_sink: int = 4,
                 step: int = 256, refit_interval: int = 0):
        self.bits, self.outlier_fraction, self.lloyd_iters, self.n_sink, self.step = (
            bits, outlier_fraction, lloyd_iters, n_sink, step)
        self.refit_interval = int(refit_interval)
        self._reset()

    def _reset(self):
        self.keys = self.values = None
        self.offset = 0
        self.key_levels = self.key_thresh = None
        self.value_levels = None  # of the latest call
        self.outlier_count = 0
        self.sink_kept = 0
        self._kc = self._vc = self._kf = self._vf = 0
        self._shape = None
        self._since_fit = 0  # calls since the key tables were fit

    def update_and_fetch(self, keys, values):
        import torch

        B, H, S, D = (int(x) for x in keys.shape)
        if self._shape is not None and self._shape != (B, H, D):
            raise kvq.KvqError(kvq.KVQ_ERR_SHAPE, "batch, heads and head_dim are fixed for a cache")
        self._shape = (B, H, D)
        BH, L, d = B * H, 1 << self.bits, keys.device
        first = self.key_levels is None
        fit = first or (self.refit_interval > 0 and self._since_fit + 1 >= self.refit_interval)
        if first:
            self.key_levels = torch.zeros((BH, D, L), dtype=torch.float32, device=d)
            self.key_thresh = torch.zeros((BH, D), dtype=torch.int16, device=d)
        k = keys.reshape(BH, S, D).contiguous()
        v = values.reshape(BH, S, D).contiguous()
        z = lambda *sh, dt: torch.zeros(sh, dtype=dt, device=d)
        cb = D * self.bits // 8
        kc, vc = z(BH, S, cb, dt=torch.uint8), z(BH, S, cb, dt=torch.uint8)
        vl = z(BH, S, L, dt=torch.float32)
        args = (BH, S, D, self.offset, self.n_sink, self.outlier_fraction, int(fit))
        cap = max(1, max(kvq.kvq_nuq_outlier_bound(*args, w) for w in (0, 1)))
        lists = [z(cap, dt=torch.int32), z(cap, dt=torch.int16), z(cap, dt=torch.int32), z(cap, dt=torch.int16)]
        cnt = z(2, dt=torch.int64)
        ws = z(kvq.kvq_nuq_workspace_bytes(BH, S, D, self.bits, self.offset, self.n_sink,
                                           self.outlier_fraction, int(fit)), dt=torch.uint8)
        kr, vr = z(BH, S, D, dt=torch.float16), z(BH, S, D, dt=torch.float16)
        kvq.kvq_nuq_fit_quant(k, v, self.offset, self.bits, self.outlier_fraction, self.lloyd_iters, self.n_sink,
                              fit, self.key_levels, self.key_thresh, vl, kc, vc, *lists, cnt, ws, kr, vr)
        n_out = [int(c) for c in cnt.cpu()]
        sinks = min(self.n_sink, S) if self.offset == 0 else 0
        self.sink_kept += sinks
        self.outlier_count += n_out[0] + n_out[1]
        self.value_levels = vl
        self.last_codes = (kc, vc)
        self.last_outliers = ((lists[0][: n_out[0]], lists[1][: n_out[0]]), (lists[2][: n_out[1]], lists[3][: n_out[1]]))
        codes = BH * S * D * self.bits // 8
        sink_bytes = BH * sinks * D * 2
        self._kc += codes + n_out[0] * 6 + sink_bytes + (BH * D * (L * 4 + 2) if first else 0)
        self._since_fit = 0 if fit else self._since_fit + 1
        self._vc += codes + n_out[1] * 6 + sink_bytes + BH * S * L * 4
        self._kf += BH * S * D * 2
        self._vf += BH * S * D * 2
        end = self.offset + S
        self.keys = _grow(self.keys, B, H, end, D, self.step, keys)
        self.values = _grow(self.values, B, H, end, D, self.step, values)
        self.keys[:, :, self.offset:end].copy_(kr.view(B, H, S, D))
        self.values[:, :, self.offset:end].copy_(vr.view(B, H, S, D))
        self.offset = end
        return self.keys[:, :, : self.offset], self.values[:, :, : self.offset]

    def trim(self, n: int) -> int:
        """Drop the newest n tokens. Trimming to empty resets everything (the
        next call fits afresh and keeps sinks again); a partial trim keeps the
        frozen key state and scales the byte accounting with the token count."""
        t = max(0, min(int(n), self.offset))
        if t == 0:
            return 0
        if t == self.offset:
            self._reset()
            return t
        keep = (self.offset - t) / self.offset
        self._kc, self._vc = int(self._kc * keep), int(self._vc * keep)
        self._kf, self._vf = int(self._kf * keep), int(self._vf * keep)
        self.offset -= t
        return t

    @property
    def nuq_bits(self) -> int:
        return self.bits

    @property
    def compressed_key_bytes(self) -> int:
        return self._kc

    @property
    def compressed_value_bytes(self) -> int:
        return self._vc

    @property
    def fp16_key_bytes(self) -> int:
        return self._kf

    @property
    def fp16_value_bytes(self) -> int:
        return self._vf

    @property
    def effective_bits(self) -> float:
        """Stored key bits per key element (codes, tables, outliers, sinks)."""
        return 0.0 if self._kf == 0 else 16.0 * self._kc / self._kf


class PagedSymCache:
    """Paged symmetric q8/q6/q4 cache for several sequences: per (layer,
    K/V) pools of `num_pages` pages of `page_size` token slots (the layout of
    kvq_quant_sym / kvq_dequant_sym), a free list of pages, and per sequence
    its page list and length. Appends take pages from the free list as a
    sequence grows and quantize the new tokens into their slots; trims give
    back the pages past the new length; fetch dequantizes whole sequences
    through a block table. Page allocation is host bookkeeping; every byte
    of the cache is written and read by the kernels."""

    def __init__(self, layers, num_pages, page_size, kv_heads, head_dim, bits, device=None):
        import torch

        self.lay = kvq.layout(layers, num_pages, page_size, kv_heads, head_dim, bits)
        self.P, self.H, self.D, self.L, self.bits = page_size, kv_heads, head_dim, layers, bits
        pd = kvq.kvq_packed_dim(head_dim, bits)
        if pd <= 0:
            raise kvq.KvqError(kvq.KVQ_ERR_SHAPE, "head_dim %d is not valid for q%d" % (head_dim, bits))
        slots = num_pages * page_size
        dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
        self.device = dev
        self.k_codes = torch.zeros((layers, slots, kv_heads, pd), dtype=torch.uint8, device=dev)
        self.v_codes = torch.zeros_like(self.k_codes)
        self.k_scales = torch.zeros((layers, slots, kv_heads), dtype=torch.int16, device=dev)
        self.v_scales = torch.zeros_like(self.k_scales)
        self.free = list(range(num_pages - 1, -1, -1))  # stack: page 0 is handed out first
        self.pages = {}                                 # seq id -> [page ids]
        self.lengths = {}                               # seq id -> tokens

    def pages_in_use(self) -> int:
        return sum(len(p) for p in self.pages.values())

    def append(self, seq_ids, k, v):
        """k, v: fp16 [layers][n_tokens][kv_heads][head_dim], the new tokens of
        the listed sequences one after another; seq_ids: [(seq id, count)]."""
        import torch

        slots = []
        for sid, n in seq_ids:
            pages = self.pages.setdefault(sid, [])
            length = self.lengths.get(sid, 0)
            need = (length + n + self.P - 1) // self.P - len(pages)
            if need > len(self.free):
                raise kvq.KvqError(kvq.KVQ_ERR_CAPACITY, "page pool exhausted (%d free, %d needed)" %
                                   (len(self.free), need))
            for _ in range(need):
                pages.append(self.free.pop())
            for pos in range(length, length + n):
                slots.append(pages[pos // self.P] * self.P + pos % self.P)
            self.lengths[sid] = length + n
        if len(slots) != int(k.shape[1]):
            raise kvq.KvqError(kvq.KVQ_ERR_SHAPE, "token count does not match the sequence counts")
        sm = torch.tensor(slots, dtype=torch.int32).to(self.device)
        kvq.kvq_quant_sym(self.lay, k, v, sm, self.k_codes, self.k_scales, self.v_codes, self.v_scales)

    def trim(self, sid, n: int) -> int:
        length = self.lengths.get(sid, 0)
        t = max(0, min(int(n), length))
        self.lengths[sid] = length - t
        keep = (length - t + self.P - 1) // self.P
        while len(self.pages[sid]) > keep:
            self.free.append(self.pages[sid].pop())
        return t

    def release(self, sid):
        self.trim(sid, self.lengths.get(sid, 0))
        self.pages.pop(sid, None)
        self.lengths.pop(sid, None)

    def fetch(self, seq_list, max_len=None):
        """fp16 (K, V) [layers][len(seq_list)][max_len][kv_heads][head_dim];
        positions past a sequence's length are +0."""
        import torch

        lens = [self.lengths.get(s, 0) for s in seq_list]
        max_len = max(lens + [1]) if max_len is None else max_len
        mb = max(1, max(len(self.pages.get(s, [])) for s in seq_list))
        bt = torch.full((len(seq_list), mb), -1, dtype=torch.int32)
        for i, s in enumerate(seq_list):
            p = self.pages.get(s, [])
            if p:
                bt[i, : len(p)] = torch.tensor(p, dtype=torch.int32)
        shape = (self.L, len(seq_list), max_len, self.H, self.D)
        ko = torch.empty(shape, dtype=torch.float16, device=self.device)
        vo = torch.empty_like(ko)
        kvq.kvq_dequant_sym(self.lay, self.k_codes, self.k_scales, self.v_codes, self.v_scales,
                            bt.to(self.device), torch.tensor(lens, dtype=torch.int32).to(self.device), ko, vo)
        return ko, vo
