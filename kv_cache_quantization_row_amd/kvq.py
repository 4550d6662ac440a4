"""Python binding of libkvq (ctypes). Argument marshalling only: every step of
the quantization path runs in the HIP kernels of libkvq.so.

Functions carry the C names (kvq_quant_sym, ...) and take torch tensors that
live on the current HIP device; PyTorch provides device memory and streams.
If the shared library is missing the import of this module still works, but
every call raises -- there is no CPU fallback.
"""
from __future__ import annotations

import ctypes as C
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "kvq.h")

KVQ_OK, KVQ_ERR_NULL, KVQ_ERR_BITS, KVQ_ERR_SHAPE, KVQ_ERR_ALIGN, KVQ_ERR_CAPACITY, \
    KVQ_ERR_HIP, KVQ_ERR_MODE, KVQ_ERR_ARG = range(9)


class KvqError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("kvq error %d: %s" % (code, msg))
        self.code = code


class PagedLayout(C.Structure):
    _fields_ = [("layers", C.c_int32), ("num_pages", C.c_int32), ("page_size", C.c_int32),
                ("kv_heads", C.c_int32), ("head_dim", C.c_int32), ("bits", C.c_int32)]


_P = C.c_void_p
_I = C.c_int32
_L = C.c_int64
_F = C.c_float
_SIGS = {
    "kvq_last_error": (C.c_char_p, []),
    "kvq_version": (C.c_char_p, []),
    "kvq_parse_mode": (C.c_int, [C.c_char_p, C.POINTER(C.c_int32)]),
    "kvq_sym_qmax": (_I, [_I]),
    "kvq_packed_dim": (_L, [_I, _I]),
    "kvq_sym_cache_bytes": (_L, [_L, _I, _I, _I, _I]),
    "kvq_quant_sym": (C.c_int, [C.POINTER(PagedLayout), _P, _P, _I, _I, _I, _P, _P, _P, _P, _P, _P]),
    "kvq_dequant_sym": (C.c_int, [C.POINTER(PagedLayout), _P, _P, _P, _P, _I, _I, _P, _I, _P, _I, _I,
                                  _P, _P, _P]),
    "kvq_attn_workspace_bytes": (_L, [_I, _I, _I, _I]),
    "kvq_attn_decode_sym": (C.c_int, [C.POINTER(PagedLayout), _P, _P, _P, _P, _I, _P, _I, _P, _I, _P, _I, _I,
                                      _F, _P, _P, _L, _P]),
    "kvq_kivi_boundary": (_L, [_L, _I, _I]),
    "kvq_kivi_quant_dequant": (C.c_int, [_P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F,
                                         _P, _P, _P, _P, _P, _P, _P]),
    "kvq_kivi_pack": (C.c_int, [_P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P, _P, _P, _P]),
    "kvq_kivi_unpack": (C.c_int, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P]),
    "kvq_nuq_workspace_bytes": (_L, [_I, _I, _I, _I, _I, _I, _F, _I]),
    "kvq_nuq_outlier_bound": (_L, [_I, _I, _I, _I, _I, _F, _I, _I]),
    "kvq_nuq_fit_quant": (C.c_int, [_P, _P, _I, _I, _I, _I, _I, _F, _I, _I, _I,
                                    _P, _P, _P, _P, _P, _P, _P, _P, _P, _L, _P, _P, _P, _P, _L, _P]),
}

_lib = None


def declared_symbols() -> list[str]:
    """Function names declared in include/kvq.h."""
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z0-9_]+)\s*\(", txt)))


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise KvqError(KVQ_ERR_HIP, "libkvq.so is not built (python -m kv_cache_quantization_row_amd.build)")
        L = C.CDLL(LIB_PATH)
        for name in declared_symbols():
            fn = getattr(L, name)
            if name in _SIGS:
                fn.restype, fn.argtypes = _SIGS[name]
        _lib = L
    return _lib


def _err(rc: int):
    if rc != KVQ_OK:
        raise KvqError(rc, lib().kvq_last_error().decode())


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return C.c_void_p(stream if isinstance(stream, int) else stream.cuda_stream)
    import torch
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise KvqError(KVQ_ERR_ARG, "tensors must be on the GPU")
            if not t.is_contiguous():
                raise KvqError(KVQ_ERR_ARG, "tensors must be contiguous")


# ------------------------------------------------------------------ host helpers
def kvq_version() -> str:
    return lib().kvq_version().decode()


def kvq_parse_mode(mode: str) -> int:
    b = C.c_int32(0)
    _err(lib().kvq_parse_mode(mode.encode(), C.byref(b)))
    return b.value


def kvq_sym_qmax(bits: int) -> int:
    return lib().kvq_sym_qmax(bits)


def kvq_packed_dim(head_dim: int, bits: int) -> int:
    return lib().kvq_packed_dim(head_dim, bits)


def kvq_sym_cache_bytes(tokens, layers, kv_heads, head_dim, bits) -> int:
    return lib().kvq_sym_cache_bytes(tokens, layers, kv_heads, head_dim, bits)


def kvq_kivi_boundary(offset: int, residual_length: int, group_size: int) -> int:
    return lib().kvq_kivi_boundary(offset, residual_length, group_size)


# ------------------------------------------------------------------ symmetric
def layout(layers, num_pages, page_size, kv_heads, head_dim, bits) -> PagedLayout:
    return PagedLayout(layers, num_pages, page_size, kv_heads, head_dim, bits)


def kvq_quant_sym(lay: PagedLayout, k, v, slot_mapping, k_codes, k_scales, v_codes, v_scales,
                  layer0: int = 0, stream=None):
    """k, v: fp16 [n_layers][n_tokens][kv_heads][head_dim] (either may be None with its pools)."""
    x = k if k is not None else v
    _dev(k, v, slot_mapping, k_codes, k_scales, v_codes, v_scales)
    n_layers, n_tokens = int(x.shape[0]), int(x.shape[1])
    _err(lib().kvq_quant_sym(C.byref(lay), _ptr(k), _ptr(v), layer0, n_layers, n_tokens,
                             _ptr(slot_mapping), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes),
                             _ptr(v_scales), _stream(stream)))


def kvq_dequant_sym(lay: PagedLayout, k_codes, k_scales, v_codes, v_scales, block_table, seq_lens,
                    k_out, v_out, layer0: int = 0, stream=None):
    """k_out/v_out: fp16 [n_layers][n_seqs][max_len][kv_heads][head_dim]."""
    o = k_out if k_out is not None else v_out
    _dev(k_codes, k_scales, v_codes, v_scales, block_table, seq_lens, k_out, v_out)
    n_layers, n_seqs, max_len = int(o.shape[0]), int(o.shape[1]), int(o.shape[2])
    _err(lib().kvq_dequant_sym(C.byref(lay), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes),
                               _ptr(v_scales), layer0, n_layers, _ptr(block_table),
                               int(block_table.shape[1]), _ptr(seq_lens), n_seqs, max_len,
                               _ptr(k_out), _ptr(v_out), _stream(stream)))


# ------------------------------------------------------------------ decode attention
def kvq_attn_workspace_bytes(n_seqs, q_heads, head_dim, max_len) -> int:
    return lib().kvq_attn_workspace_bytes(n_seqs, q_heads, head_dim, max_len)


def kvq_attn_decode_sym(lay: PagedLayout, k_codes, k_scales, v_codes, v_scales, layer: int, q, block_table,
                        seq_lens, max_len: int, softmax_scale: float, out, workspace, stream=None):
    """q, out: fp16 [n_seqs][q_heads][head_dim]; pools as in kvq_dequant_sym."""
    _dev(k_codes, k_scales, v_codes, v_scales, q, block_table, seq_lens, out, workspace)
    n_seqs, q_heads = int(q.shape[0]), int(q.shape[1])
    _err(lib().kvq_attn_decode_sym(C.byref(lay), _ptr(k_codes), _ptr(k_scales), _ptr(v_codes), _ptr(v_scales),
                                   layer, _ptr(q), q_heads, _ptr(block_table), int(block_table.shape[1]),
                                   _ptr(seq_lens), n_seqs, max_len, softmax_scale, _ptr(out), _ptr(workspace),
                                   int(workspace.numel() * workspace.element_size()), _stream(stream)))


# ------------------------------------------------------------------ KIVI
def kvq_kivi_quant_dequant(keys, values, lo: int, hi: int, bits: int, group_size: int = 32,
                           eps: float = 1e-8, k_codes=None, k_scale=None, k_min=None,
                           v_codes=None, v_scale=None, v_min=None, stream=None):
    """In place on fp16 [B][H][S_cap][D] keys/values (either may be None)."""
    x = keys if keys is not None else values
    _dev(keys, values, k_codes, k_scale, k_min, v_codes, v_scale, v_min)
    B, H, S_cap, D = (int(s) for s in x.shape)
    _err(lib().kvq_kivi_quant_dequant(_ptr(keys), _ptr(values), B, H, S_cap, D, lo, hi, bits,
                                      group_size, eps, _ptr(k_codes), _ptr(k_scale), _ptr(k_min),
                                      _ptr(v_codes), _ptr(v_scale), _ptr(v_min), _stream(stream)))


def kivi_param_shape(B, H, S_cap, D, per_channel, group_size):
    """Shape of the fp16 scale / zero arrays of packed KIVI storage."""
    if per_channel:
        return (B, H, (S_cap + group_size - 1) // group_size, D)
    return (B, H, S_cap, (D + group_size - 1) // group_size)


def kvq_kivi_pack(keys, values, lo: int, hi: int, bits: int, group_size: int = 32, eps: float = 1e-8,
                  k_codes=None, k_scale=None, k_zero=None, v_codes=None, v_scale=None, v_zero=None,
                  stream=None):
    """keys/values fp16 [B][H][S_cap][D] (either None); codes uint8
    [B][H][S_cap][D*bits/8]; scale/zero int16 holding fp16 bits, shapes of
    kivi_param_shape."""
    x = keys if keys is not None else values
    _dev(keys, values, k_codes, k_scale, k_zero, v_codes, v_scale, v_zero)
    B, H, S_cap, D = (int(s) for s in x.shape)
    _err(lib().kvq_kivi_pack(_ptr(keys), _ptr(values), B, H, S_cap, D, lo, hi, bits, group_size, eps,
                             _ptr(k_codes), _ptr(k_scale), _ptr(k_zero), _ptr(v_codes), _ptr(v_scale),
                             _ptr(v_zero), _stream(stream)))


def kvq_kivi_unpack(k_codes, k_scale, k_zero, v_codes, v_scale, v_zero, lo: int, hi: int, bits: int,
                    group_size: int, k_out, v_out, stream=None):
    """Tokens [lo, hi) into k_out / v_out, fp16 [B][H][S_cap][D] (either None)."""
    o = k_out if k_out is not None else v_out
    _dev(k_codes, k_scale, k_zero, v_codes, v_scale, v_zero, k_out, v_out)
    B, H, S_cap, D = (int(s) for s in o.shape)
    _err(lib().kvq_kivi_unpack(_ptr(k_codes), _ptr(k_scale), _ptr(k_zero), _ptr(v_codes), _ptr(v_scale),
                               _ptr(v_zero), B, H, S_cap, D, lo, hi, bits, group_size, _ptr(k_out),
                               _ptr(v_out), _stream(stream)))


# ------------------------------------------------------------------ NUQ
def kvq_nuq_outlier_bound(BH, S, D, start_pos, n_sink, frac, fit_keys, which) -> int:
    return lib().kvq_nuq_outlier_bound(BH, S, D, start_pos, n_sink, frac, int(fit_keys), which)


def kvq_nuq_workspace_bytes(BH, S, D, bits, start_pos, n_sink, frac, fit_keys) -> int:
    return lib().kvq_nuq_workspace_bytes(BH, S, D, bits, start_pos, n_sink, frac, int(fit_keys))


def kvq_nuq_fit_quant(keys, values, start_pos, bits, frac, lloyd_iters, n_sink, fit_keys,
                      key_levels, key_thresh, value_levels, k_codes, v_codes, k_opos, k_oval,
                      v_opos, v_oval, out_counts, workspace, k_recon=None, v_recon=None, stream=None):
    """keys/values fp16 [BH][S][D]; all outputs preallocated device tensors (see include/kvq.h)."""
    _dev(keys, values, key_levels, key_thresh, value_levels, k_codes, v_codes, k_opos, k_oval,
         v_opos, v_oval, out_counts, workspace, k_recon, v_recon)
    BH, S, D = (int(x) for x in keys.shape)
    out_cap = min(int(k_opos.numel()), int(k_oval.numel()), int(v_opos.numel()), int(v_oval.numel()))
    _err(lib().kvq_nuq_fit_quant(_ptr(keys), _ptr(values), BH, S, D, start_pos, bits, frac,
                                 lloyd_iters, n_sink, int(fit_keys), _ptr(key_levels),
                                 _ptr(key_thresh), _ptr(value_levels), _ptr(k_codes), _ptr(v_codes),
                                 _ptr(k_opos), _ptr(k_oval), _ptr(v_opos), _ptr(v_oval), out_cap,
                                 _ptr(out_counts), _ptr(k_recon), _ptr(v_recon), _ptr(workspace),
                                 int(workspace.numel() * workspace.element_size()), _stream(stream)))
