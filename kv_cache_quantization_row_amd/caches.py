"""Cache objects over the libkvq kernels: the host-side state machines that
decide what to quantize when, and keep the byte accounting.

Every quantization step runs in the HIP kernels (kvq_kivi_quant_dequant,
kvq_kivi_pack / kvq_kivi_unpack, kvq_nuq_fit_quant, kvq_quant_sym /
kvq_dequant_sym); this module appends incoming tokens to device-resident
buffers (PyTorch memory), moves frontiers, hands out pages and counts bytes.
KIVI / NUQ tensors are fp16 [B][H][S][D] on the current HIP device.

KiviCache  ["veloxquant_mlx.cache.kivi_cache": module docstring (residual
            window, group-aligned quantization, trim rollback, memory-savings
            caveat) and the KIVIKVCache reporting properties]
NuqCache   ["veloxquant_mlx.cache.kvquant_cache module": level lifecycle,
            attention-sink quantization, byte accounting, and the
            KVQuantKVCache trim and property documentation]
PagedSymCache [MTPLX pull request #267, "feat(kv-cache): add q6 paged KV
            quantization": paged q8/q6/q4 storage sized by packed_dim; the
            page allocator, appends and trims are a reading, the page
            describes only the storage]
"""
from __future__ import annotations

from . import kvq


def _fp16_buffer(old, B, H, need, D, step, device):
    """fp16 [B][H][cap][D] with cap >= need (a multiple of step); the rows of
    `old` are carried over."""
    import torch

    if old is not None and old.shape[2] >= need:
        return old
    cap = -(-need // step) * step
    buf = torch.empty((B, H, cap, D), dtype=torch.float16, device=device)
    if old is not None:
        buf[:, :, : old.shape[2]].copy_(old)
    return buf


class KiviCache:
    """KIVI cache for one batch of sequences.

    State: `offset` tokens are held; the oldest `n_quantized` of them (a
    multiple of the group size) have been quantized, the rest sit in an fp16
    residual window. Three rules drive it:
      - ageing: once a token is more than `residual_length` tokens old it is
        eligible, but quantization only ever takes whole groups of
        `group_size` tokens, since keys are grouped along tokens
        (kvq_kivi_boundary gives the frontier);
      - storage: storage="fp16" round-trips the eligible tokens in place in a
        growing fp16 buffer (what the kivi_cache page's own cache keeps, so
        its compressed sizes are what packed storage would take);
        storage="packed" keeps the quantized tokens only as b-bit codes plus
        one fp16 (scale, zero) pair per group (kvq_kivi_pack), fp16 only for
        the residual window, and rebuilds the fp16 view through
        kvq_kivi_unpack when fetched;
      - trim: dropping tokens pulls the frontier down to the group boundary at
        or below the new length; the tokens between that boundary and the
        new length keep their quantized values and are quantized again when
        they age out (a rolled-back group is requantized once).
    Byte accounting follows from (offset, n_quantized): compressed sizes are
    the packed sizes of the quantized prefix (b-bit codes plus one fp16
    scale and one fp16 zero per group: keys per channel and group of tokens,
    values per token and group of channels), fp16 sizes are those of the
    tokens held, and the residual is the fp16 window."""

    def __init__(self, bits: int = 2, group_size: int = 32, residual_length: int = 128, storage: str = "fp16",
                 step: int = 256):
        if bits not in (2, 4, 8):
            raise kvq.KvqError(kvq.KVQ_ERR_BITS, "KIVI bits must be 2, 4 or 8")
        if group_size <= 0 or residual_length < 0 or step <= 0:
            raise kvq.KvqError(kvq.KVQ_ERR_ARG, "group_size and step must be positive, residual_length >= 0")
        if storage not in ("fp16", "packed"):
            raise kvq.KvqError(kvq.KVQ_ERR_ARG, "storage must be 'fp16' or 'packed'")
        if storage == "packed" and group_size % 8:
            raise kvq.KvqError(kvq.KVQ_ERR_ARG, "packed storage needs group_size a multiple of 8")
        self.bits, self.group_size, self.residual_length = bits, group_size, residual_length
        self.storage, self.step = storage, -(-step // group_size) * group_size
        self._start()

    def _start(self):
        self._len = 0          # tokens held
        self._front = 0        # quantized prefix
        self._geom = None      # (B, H, D, device)
        self.keys = self.values = None      # fp16 storage: full buffers
        self._win = None                    # packed storage: fp16 window [B][H][wcap][D] x2, tokens [front, len)
        self._store = None                  # packed storage: per side (codes, scale, zero), capacity self._cap
        self._cap = 0

    # ------------------------------------------------------------- state
    @property
    def offset(self) -> int:
        return self._len

    @property
    def n_quantized(self) -> int:
        return self._front

    def _admit_geometry(self, keys, values):
        B, H, S, D = (int(x) for x in keys.shape)
        if tuple(values.shape) != tuple(keys.shape):
            raise kvq.KvqError(kvq.KVQ_ERR_SHAPE, "keys and values must have the same shape")
        if self._geom is not None and self._geom[:3] != (B, H, D):
            raise kvq.KvqError(kvq.KVQ_ERR_SHAPE, "batch, heads and head_dim are fixed for a cache")
        if self.storage == "packed" and (D % 8 or D * self.bits % 8):
            raise kvq.KvqError(kvq.KVQ_ERR_SHAPE, "packed storage needs head_dim a multiple of 8")
        self._geom = (B, H, D, keys.device)
        return S

    def _eligible_frontier(self) -> int:
        return kvq.kvq_kivi_boundary(self._len, self.residual_length, self.group_size)

    # ------------------------------------------------------------- fp16 storage
    def _append_fp16(self, keys, values, S):
        B, H, D, dev = self._geom
        end = self._len + S
        self.keys = _fp16_buffer(self.keys, B, H, end, D, self.step, dev)
        self.values = _fp16_buffer(self.values, B, H, end, D, self.step, dev)
        self.keys[:, :, self._len:end].copy_(keys)
        self.values[:, :, self._len:end].copy_(values)

    def _quantize_fp16(self, lo, hi):
        kvq.kvq_kivi_quant_dequant(self.keys, self.values, lo, hi, self.bits, self.group_size)

    # ------------------------------------------------------------- packed storage
    def _reserve_store(self, tokens):
        import torch

        if tokens <= self._cap:
            return
        B, H, D, dev = self._geom
        cap = max(-(-tokens // self.step) * self.step, 2 * self._cap)
        g = self.group_size
        new = []
        for per_channel in (True, False):
            codes = torch.empty((B, H, cap, D * self.bits // 8), dtype=torch.uint8, device=dev)
            shp = kvq.kivi_param_shape(B, H, cap, D, per_channel, g)
            sc = torch.empty(shp, dtype=torch.int16, device=dev)
            zr = torch.empty(shp, dtype=torch.int16, device=dev)
            if self._store is not None:
                oc, os_, oz = self._store[0 if per_channel else 1]
                codes[:, :, : oc.shape[2]].copy_(oc)
                sc[:, :, : os_.shape[2]].copy_(os_)
                zr[:, :, : oz.shape[2]].copy_(oz)
            new.append((codes, sc, zr))
        self._store, self._cap = new, cap

    def _window_rows(self):
        return self._len - self._front

    def _append_packed(self, keys, values, S):
        B, H, D, dev = self._geom
        held = self._window_rows()
        win = [_fp16_buffer(None if self._win is None else self._win[i], B, H, held + S, D, self.step, dev)
               for i in range(2)]
        win[0][:, :, held:held + S].copy_(keys)
        win[1][:, :, held:held + S].copy_(values)
        self._win = win

    def _quantize_packed(self, lo, hi):
        self._reserve_store(hi)
        (kc, ks, kz), (vc, vs, vz) = self._store
        kvq.kvq_kivi_pack(self._win[0], self._win[1], lo, hi, self.bits, self.group_size, k_codes=kc, k_scale=ks,
                          k_zero=kz, v_codes=vc, v_scale=vs, v_zero=vz, x_t0=self._front)
        # the window keeps tokens [hi, len): move them to its first rows, into
        # a smaller buffer when a long prefill left it far larger than the
        # residual window needs
        keep, off = self._len - hi, hi - self._front
        B, H, D, dev = self._geom
        small = -(-(self.residual_length + self.group_size) // self.step) * self.step + self.step
        for i, w in enumerate(self._win):
            if w.shape[2] > 2 * small:
                nw = _fp16_buffer(None, B, H, max(keep, small), D, self.step, dev)
                nw[:, :, :keep].copy_(w[:, :, off:off + keep])
                self._win[i] = nw
            elif keep:
                w[:, :, :keep].copy_(w[:, :, off:off + keep].clone())

    def _unpack_into(self, out_k, out_v, lo, hi, out_t0):
        (kc, ks, kz), (vc, vs, vz) = self._store
        kvq.kvq_kivi_unpack(kc, ks, kz, vc, vs, vz, lo, hi, self.bits, self.group_size, out_k, out_v,
                            out_t0=out_t0)

    def _fetch_packed(self):
        import torch

        B, H, D, dev = self._geom
        k = torch.empty((B, H, self._len, D), dtype=torch.float16, device=dev)
        v = torch.empty_like(k)
        if self._front:
            self._unpack_into(k, v, 0, self._front, 0)
        n = self._window_rows()
        if n:
            k[:, :, self._front:].copy_(self._win[0][:, :, :n])
            v[:, :, self._front:].copy_(self._win[1][:, :, :n])
        return k, v

    # ------------------------------------------------------------- lifecycle
    def update_and_fetch(self, keys, values):
        """Append keys/values fp16 [B][H][S][D]; quantize what aged out of the
        residual window in whole groups; return fp16 (K, V) [B][H][offset][D]."""
        S = self._admit_geometry(keys, values)
        keys, values = keys.contiguous(), values.contiguous()
        if self.storage == "fp16":
            self._append_fp16(keys, values, S)
        else:
            self._append_packed(keys, values, S)
        self._len += S
        target = self._eligible_frontier()
        if target > self._front:
            if self.storage == "fp16":
                self._quantize_fp16(self._front, target)
            else:
                self._quantize_packed(self._front, target)
            self._front = target
        return self.fetch()

    def fetch(self):
        if self._len == 0:
            return None, None
        if self.storage == "fp16":
            return self.keys[:, :, : self._len], self.values[:, :, : self._len]
        return self._fetch_packed()

    def trim(self, n: int) -> int:
        """Drop the newest n tokens (at most offset); returns how many."""
        t = max(0, min(int(n), self._len))
        if t == 0:
            return 0
        new_len = self._len - t
        g = self.group_size
        new_front = min(self._front, new_len - new_len % g)
        if self.storage == "packed" and new_front < self._front:
            # tokens [new_front, min(front, new_len)) come back into the window
            # as their quantized values; window tokens past new_len are dropped
            B, H, D, dev = self._geom
            back = min(self._front, new_len) - new_front
            kept = max(0, new_len - self._front)
            win = [_fp16_buffer(None, B, H, back + kept, D, self.step, dev) for _ in range(2)]
            for i in range(2):
                if kept:
                    win[i][:, :, back:back + kept].copy_(self._win[i][:, :, :kept])
            if back:
                self._unpack_into(win[0], win[1], new_front, new_front + back, new_front)
            self._win = win
        self._len, self._front = new_len, new_front
        if self._len == 0:
            self._start()
        return t

    # ------------------------------------------------------------- accounting
    def packed_bytes(self, n: int):
        """(key, value) bytes of n quantized tokens stored packed."""
        if self._geom is None:
            return 0, 0
        B, H, D, _ = self._geom
        g, b = self.group_size, self.bits
        codes = -(-(n * D * b) // 8)
        key_pairs = -(-n // g) * D
        value_pairs = n * -(-D // g)
        return B * H * (codes + 4 * key_pairs), B * H * (codes + 4 * value_pairs)

    def _fp16_bytes(self, n_tokens: int) -> int:
        if self._geom is None:
            return 0
        B, H, D, _ = self._geom
        return B * H * n_tokens * D * 2

    @property
    def compressed_key_bytes(self) -> int:
        return self.packed_bytes(self._front)[0]

    @property
    def compressed_value_bytes(self) -> int:
        return self.packed_bytes(self._front)[1]

    @property
    def fp16_key_bytes(self) -> int:
        return self._fp16_bytes(self._len)

    @property
    def fp16_value_bytes(self) -> int:
        return self._fp16_bytes(self._len)

    @property
    def residual_fp16_bytes(self) -> int:
        return 2 * self._fp16_bytes(self._len - self._front)

    @property
    def assigned_avg_bits(self) -> float:
        return float(self.bits)

    @property
    def effective_compression_ratio(self) -> float:
        full = self.fp16_key_bytes + self.fp16_value_bytes
        stored = self.compressed_key_bytes + self.compressed_value_bytes + self.residual_fp16_bytes
        return 1.0 if full == 0 or stored == 0 else full / stored

    def stored_quantized_bytes(self) -> int:
        """Device bytes that hold the quantized tokens: with packed storage,
        the rows of the codes and (scale, zero) arrays that the quantized
        prefix occupies (equal to compressed_key_bytes +
        compressed_value_bytes); with fp16 storage, their fp16 rows."""
        if self._front == 0:
            return 0
        if self.storage == "fp16":
            return 2 * self._fp16_bytes(self._front)
        (kc, ks, kz), (vc, vs, vz) = self._store
        g = self.group_size
        nk = -(-self._front // g)
        total = 0
        for t, rows in ((kc, self._front), (vc, self._front), (vs, self._front), (vz, self._front),
                        (ks, nk), (kz, nk)):
            total += t[:, :, :rows].numel() * t.element_size()
        return total

    def device_bytes(self) -> int:
        """All device memory the cache holds (storage at capacity plus buffers)."""
        tensors = []
        if self.storage == "fp16":
            tensors = [t for t in (self.keys, self.values) if t is not None]
        else:
            if self._store is not None:
                tensors += [t for side in self._store for t in side]
            if self._win is not None:
                tensors += list(self._win)
        return sum(t.numel() * t.element_size() for t in tensors)


class NuqCache:
    """KVQuant-style NUQ cache for one batch of sequences.

    The first call of a sequence fits the per-channel key levels and |key|
    thresholds and freezes them, and keeps its first n_sink tokens exact;
    every call fits fresh per-token value levels; the buffers hold the
    dequantized K/V. With refit_interval = N > 0 the key tables are fit again
    on every N-th call after the one that last fit them, from that call's
    tokens (level lifecycle, read for decode calls of one token).
    Nothing in a call waits for the device: each call writes its outlier
    counts to its own slot of a device log (summed on the device every
    _CLOG calls) that is read only when outlier_count or the byte
    properties are asked for; the per-call buffers for a given call length
    are allocated once and reused; keys and values share one fp16 buffer,
    so one copy appends a call's reconstructions.
    Byte accounting (a reading of the page's byte-accounting description):
    codes at `bits` per element, fp32 level tables and fp16 key thresholds
    (one key table held at a time), 6 bytes per outlier (fp16 value + int32
    position), fp16 sink tokens."""

    def __init__(self, bits: int = 3, outlier_fraction: float = 0.01, lloyd_iters: int = 8, n_sink: int = 4,
                 step: int = 256, refit_interval: int = 0):
        self.bits, self.outlier_fraction, self.lloyd_iters, self.n_sink, self.step = (
            bits, float(outlier_fraction), lloyd_iters, n_sink, step)
        self.refit_interval = int(refit_interval)
        self._bufs = {}  # (S, fit, start == 0) -> per-call buffers
        self._reset()

    _CLOG = 1024  # count-log slots

    def _reset(self):
        self.keys = self.values = None
        self._kv = None         # fp16 [2][B][H][cap][D]: keys, values
        self.offset = 0
        self.key_levels = self.key_thresh = None
        self.value_levels = None  # of the latest call
        self.sink_kept = 0
        self._kc = self._vc = self._kf = self._vf = 0  # host-known byte parts
        self._counts = None     # device int64 [2]: outliers of folded-in count-log rounds
        self._clog = None       # device int64 [_CLOG][2]: one slot per call
        self._ci = 0            # next count-log slot
        self._folded = [0, 0]   # outliers already folded into the host totals
        self._shape = None
        self._since_fit = 0     # calls since the key tables were fit
        self._last = None

    def _call_buffers(self, BH, S, D, fit, device):
        import torch

        key = (BH, S, D, bool(fit), self.offset == 0)
        b = self._bufs.get(key)
        if b is None:
            L, cb = 1 << self.bits, D * self.bits // 8
            e = lambda *sh, dt: torch.empty(sh, dtype=dt, device=device)
            args = (BH, S, D, self.offset, self.n_sink, self.outlier_fraction, int(fit))
            cap = max(1, max(kvq.kvq_nuq_outlier_bound(*args, w) for w in (0, 1)))
            wsb = kvq.kvq_nuq_workspace_bytes(BH, S, D, self.bits, self.offset, self.n_sink,
                                              self.outlier_fraction, int(fit))
            b = dict(kc=e(BH, S, cb, dt=torch.uint8), vc=e(BH, S, cb, dt=torch.uint8),
                     lists=[e(cap, dt=torch.int32), e(cap, dt=torch.int16), e(cap, dt=torch.int32),
                            e(cap, dt=torch.int16)],
                     ws=e(wsb, dt=torch.uint8), kvr=e(2, BH, S, D, dt=torch.float16))
            self._bufs[key] = b
        return b

    def update_and_fetch(self, keys, values):
        import torch

        B, H, S, D = (int(x) for x in keys.shape)
        if self._shape is not None and self._shape != (B, H, D):
            raise kvq.KvqError(kvq.KVQ_ERR_SHAPE, "batch, heads and head_dim are fixed for a cache")
        if tuple(values.shape) != tuple(keys.shape):
            raise kvq.KvqError(kvq.KVQ_ERR_SHAPE, "keys and values must have the same shape")
        self._shape = (B, H, D)
        BH, L, d = B * H, 1 << self.bits, keys.device
        first = self.key_levels is None
        fit = first or (self.refit_interval > 0 and self._since_fit + 1 >= self.refit_interval)
        if first:
            self.key_levels = torch.empty((BH, D, L), dtype=torch.float32, device=d)
            self.key_thresh = torch.empty((BH, D), dtype=torch.int16, device=d)
            self._counts = torch.zeros(2, dtype=torch.int64, device=d)
            self._clog = torch.zeros((self._CLOG, 2), dtype=torch.int64, device=d)
            self._ci = 0
        if self._ci == self._CLOG:  # a full log: fold it on the device
            self._counts += self._clog.sum(0)
            self._ci = 0
        k = keys.reshape(BH, S, D).contiguous()
        v = values.reshape(BH, S, D).contiguous()
        b = self._call_buffers(BH, S, D, fit, d)
        vl = torch.empty((BH, S, L), dtype=torch.float32, device=d)  # kept as value_levels
        cnt = self._clog[self._ci]
        kvq.kvq_nuq_fit_quant(k, v, self.offset, self.bits, self.outlier_fraction, self.lloyd_iters, self.n_sink,
                              fit, self.key_levels, self.key_thresh, vl, b["kc"], b["vc"], *b["lists"], cnt,
                              b["ws"], b["kvr"][0], b["kvr"][1])
        self._ci += 1
        sinks = min(self.n_sink, S) if self.offset == 0 else 0
        self.sink_kept += sinks
        self.value_levels = vl
        self._last = dict(b, cnt=cnt)
        codes = BH * S * D * self.bits // 8
        sink_bytes = BH * sinks * D * 2
        self._kc += codes + sink_bytes + (BH * D * (L * 4 + 2) if first else 0)
        self._vc += codes + sink_bytes + BH * S * L * 4
        self._since_fit = 0 if fit else self._since_fit + 1
        self._kf += BH * S * D * 2
        self._vf += BH * S * D * 2
        end = self.offset + S
        if self._kv is None or self._kv.shape[3] < end:
            cap = -(-end // self.step) * self.step
            kv = torch.empty((2, B, H, cap, D), dtype=torch.float16, device=d)
            if self._kv is not None:
                kv[:, :, :, : self._kv.shape[3]].copy_(self._kv)
            self._kv = kv
            self.keys, self.values = kv[0], kv[1]
        self._kv[:, :, :, self.offset:end].copy_(b["kvr"].view(2, B, H, S, D))
        self.offset = end
        return self.keys[:, :, : self.offset], self.values[:, :, : self.offset]

    # ---- values that need the device counts (read when asked for)
    def _fold(self):
        """Move the device outlier counts into the host totals (one sync)."""
        if self._counts is None:
            return
        c = [int(x) for x in (self._counts + self._clog[: self._ci].sum(0)).cpu()]
        self._counts.zero_()
        self._ci = 0
        self._kc += 6 * c[0]
        self._vc += 6 * c[1]
        self._folded[0] += c[0]
        self._folded[1] += c[1]

    @property
    def outlier_count(self) -> int:
        self._fold()
        return self._folded[0] + self._folded[1]

    @property
    def last_codes(self):
        return None if self._last is None else (self._last["kc"], self._last["vc"])

    @property
    def last_outliers(self):
        """((key positions, values), (value positions, values)) of the latest call."""
        if self._last is None:
            return None
        kp, kv_, vp, vv = self._last["lists"]
        n = [int(x) for x in self._last["cnt"].cpu()]
        return (kp[: n[0]], kv_[: n[0]]), (vp[: n[1]], vv[: n[1]])

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
        self._fold()
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
        self._fold()
        return self._kc

    @property
    def compressed_value_bytes(self) -> int:
        self._fold()
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
        return 0.0 if self._kf == 0 else 16.0 * self.compressed_key_bytes / self._kf


class PagedSymCache:
    """Paged symmetric q8/q6/q4 cache for several sequences: per (layer,
    K/V) pools of `num_pages` pages of `page_size` token slots (the layout of
    kvq_quant_sym / kvq_dequant_sym), a free list of pages, and per sequence
    its page list and length. Appends take pages from the free list as a
    sequence grows and quantize the new tokens into their slots; trims give
    back the pages past the new length; fetch dequantizes whole sequences
    through a block table. The block table and lengths of up to `max_seqs`
    sequences are mirrored in device memory (rows are assigned on first
    append), so fetches and one-token-per-sequence decode appends build
    nothing on the host. Page allocation is host bookkeeping; every byte of
    the cache is written and read by the kernels."""

    def __init__(self, layers, num_pages, page_size, kv_heads, head_dim, bits, device=None, max_seqs=64):
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
        self.max_seqs = max_seqs
        self.rows = {}                                  # seq id -> row of the device tables
        self.bt = torch.full((max_seqs + 1, num_pages), -1, dtype=torch.int32, device=dev)
        self.lens = torch.zeros(max_seqs + 1, dtype=torch.int32, device=dev)
        self._rows_version = 0

    def pages_in_use(self) -> int:
        return sum(len(p) for p in self.pages.values())

    def _row(self, sid, taken):
        if sid in self.rows:
            return self.rows[sid]
        used = set(self.rows.values()) | taken
        for r in range(self.max_seqs):
            if r not in used:
                return r
        raise kvq.KvqError(kvq.KVQ_ERR_CAPACITY, "more than %d sequences" % self.max_seqs)

    def append(self, seq_ids, k, v):
        """k, v: fp16 [layers][n_tokens][kv_heads][head_dim], the new tokens of
        the listed sequences one after another; seq_ids: [(seq id, count)].
        Nothing changes unless the whole append succeeds."""
        import torch

        n_tok = sum(int(n) for _, n in seq_ids)
        if n_tok != int(k.shape[1]) or (v is not None and tuple(v.shape) != tuple(k.shape)):
            raise kvq.KvqError(kvq.KVQ_ERR_SHAPE, "token count does not match the sequence counts")
        if len({sid for sid, _ in seq_ids}) != len(seq_ids):
            raise kvq.KvqError(kvq.KVQ_ERR_ARG, "a sequence is listed twice")
        # plan: pages to take and slots, without touching the cache
        free = list(self.free)
        plan, slots, taken = [], [], set()
        for sid, n in seq_ids:
            pages = list(self.pages.get(sid, []))
            length = self.lengths.get(sid, 0)
            need = (length + n + self.P - 1) // self.P - len(pages)
            if need > len(free):
                raise kvq.KvqError(kvq.KVQ_ERR_CAPACITY, "page pool exhausted (%d free, %d needed)" %
                                   (len(free), need))
            new_pages = [free.pop() for _ in range(need)]
            pages += new_pages
            row = self._row(sid, taken)
            taken.add(row)
            for pos in range(length, length + n):
                slots.append(pages[pos // self.P] * self.P + pos % self.P)
            plan.append((sid, row, pages, length + n, len(pages) - len(new_pages)))
        sm = torch.tensor(slots, dtype=torch.int32).pin_memory().to(self.device, non_blocking=True) \
            if self.device.type == "cuda" else torch.tensor(slots, dtype=torch.int32)
        kvq.kvq_quant_sym(self.lay, k, v, sm, self.k_codes, self.k_scales, self.v_codes, self.v_scales)
        self._commit(plan, free)

    def _commit(self, plan, free):
        import torch

        self.free = free
        for sid, row, pages, length, first_new in plan:
            if sid not in self.rows:
                self._rows_version += 1
            self.pages[sid], self.lengths[sid], self.rows[sid] = pages, length, row
            if first_new < len(pages):
                self.bt[row, first_new:len(pages)] = torch.tensor(pages[first_new:], dtype=torch.int32).to(
                    self.device, non_blocking=True)
            self.lens[row] = length

    def append_decode(self, seq_list, k, v):
        """One new token for each sequence of seq_list (k, v: fp16
        [layers][len(seq_list)][kv_heads][head_dim]). Slots come from the
        device block table and lengths; only a sequence that crosses into a
        new page changes the host bookkeeping."""
        import torch

        if len(seq_list) != int(k.shape[1]):
            raise kvq.KvqError(kvq.KVQ_ERR_SHAPE, "one token per listed sequence")
        crossing = [s for s in seq_list if self.lengths.get(s, 0) % self.P == 0 or s not in self.rows]
        if crossing:  # new pages: the general path
            return self.append([(s, 1) for s in seq_list], k, v)
        key = tuple(seq_list)
        if getattr(self, "_dec_key", None) != (key, self._rows_version):
            self._dec_rows = torch.tensor([self.rows[s] for s in seq_list], dtype=torch.int64).to(self.device)
            self._dec_key = (key, self._rows_version)
        rows = self._dec_rows
        pos = self.lens[rows].to(torch.int64)
        page = self.bt[rows, pos // self.P].to(torch.int64)
        sm = (page * self.P + pos % self.P).to(torch.int32)
        kvq.kvq_quant_sym(self.lay, k, v, sm, self.k_codes, self.k_scales, self.v_codes, self.v_scales)
        self.lens[rows] += 1
        for s in seq_list:
            self.lengths[s] += 1

    def trim(self, sid, n: int) -> int:
        length = self.lengths.get(sid, 0)
        t = max(0, min(int(n), length))
        self.lengths[sid] = length - t
        keep = (length - t + self.P - 1) // self.P
        while len(self.pages.get(sid, [])) > keep:
            self.free.append(self.pages[sid].pop())
        if sid in self.rows:
            row = self.rows[sid]
            self.bt[row, keep:] = -1
            self.lens[row] = length - t
        return t

    def release(self, sid):
        self.trim(sid, self.lengths.get(sid, 0))
        self.pages.pop(sid, None)
        self.lengths.pop(sid, None)
        if self.rows.pop(sid, None) is not None:
            self._rows_version += 1

    def fetch(self, seq_list, max_len=None):
        """fp16 (K, V) [layers][len(seq_list)][max_len][kv_heads][head_dim];
        positions past a sequence's length are +0."""
        import torch

        if max_len is None:
            max_len = max([self.lengths.get(s, 0) for s in seq_list] + [1])
        key = tuple(seq_list)
        if getattr(self, "_fetch_key", None) != key or self._fetch_rows_version != self._rows_version:
            # device rows of the listed sequences; an unknown sequence reads
            # row max_seqs, which stays empty (length 0, no pages)
            self._fetch_idx = torch.tensor([self.rows.get(s, self.max_seqs) for s in seq_list],
                                           dtype=torch.int64).to(self.device)
            self._fetch_key, self._fetch_rows_version = key, self._rows_version
        bt, lens = self.bt[self._fetch_idx], self.lens[self._fetch_idx]
        shape = (self.L, len(seq_list), max_len, self.H, self.D)
        ko = torch.empty(shape, dtype=torch.float16, device=self.device)
        vo = torch.empty_like(ko)
        kvq.kvq_dequant_sym(self.lay, self.k_codes, self.k_scales, self.v_codes, self.v_scales, bt, lens, ko, vo)
        return ko, vo
