"""CPU oracle (test infrastructure).

Plain single-threaded C++ reference for the KV-cache quantization path, loaded
through ctypes. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it; the product library never imports it. All arrays are
numpy, host memory, C-contiguous. fp16 data travels as uint16 bit patterns.

Sources are cited per function in kvq_oracle.cpp (page title + section);
attn_decode (decode attention over dequantized rows) is plain numpy in
float64, and caches.py holds CPU models of the cache lifecycles.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

CXXFLAGS = ["-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall"]


def build(force: bool = True) -> str:
    """Compile the oracle with the host compiler (no HIP involved)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["g++", *CXXFLAGS, "-o", tmp, _SRC])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None

_P = C.c_void_p
_I = C.c_int
_LL = C.c_longlong
_F = C.c_float

_SIGS = {
    "orc_h2f": (C.c_float, [C.c_uint16]),
    "orc_f2h": (C.c_uint16, [C.c_float]),
    "orc_h2f_array": (None, [_P, _P, _LL]),
    "orc_f2h_array": (None, [_P, _P, _LL]),
    "orc_sym_qmax": (_I, [_I]),
    "orc_packed_dim": (_LL, [_I, _I]),
    "orc_sym_cache_bytes": (_LL, [_LL, _I, _I, _I, _I]),
    "orc_sym_quant_rows": (_I, [_P, _LL, _I, _I, _P, _P]),
    "orc_sym_dequant_rows": (_I, [_P, _P, _LL, _I, _I, _P]),
    "orc_sym_unpack_rows": (_I, [_P, _LL, _I, _I, _P]),
    "orc_sym_quant_paged": (_I, [_P, _I, _I, _I, _I, _P, _LL, _P, _P]),
    "orc_sym_dequant_paged": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _I, _P, _I, _I, _P]),
    "orc_kivi_boundary": (_LL, [_LL, _I, _I]),
    "orc_kivi_round_trip": (_I, [_P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P]),
    "orc_nuq_fit": (None, [_P, _I, _I, _I, _P]),
    "orc_nuq_threshold": (C.c_uint16, [_P, _I, C.c_double]),
    "orc_nuq_nearest": (_I, [C.c_uint16, _P, _I]),
    "orc_kivi_pack": (_I, [_P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P]),
    "orc_kivi_unpack": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _P]),
    "orc_nuq_fit_quant": (_I, [_P, _P, _I, _I, _I, _I, _I, C.c_double, _I, _I, _I,
                               _P, _P, _P, _P, _P, _P, _P, _P, _P, _LL, _P, _P, _P]),
}


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = C.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    assert a.dtype == np.uint16, a.dtype
    return a


# ------------------------------------------------------------------ fp16
def h2f(h):
    h = _u16(h)
    out = np.empty(h.shape, np.float32)
    lib().orc_h2f_array(_p(h), _p(out), h.size)
    return out


def f2h(f):
    f = np.ascontiguousarray(f, dtype=np.float32)
    out = np.empty(f.shape, np.uint16)
    lib().orc_f2h_array(_p(f), _p(out), f.size)
    return out


# ------------------------------------------------------------------ symmetric
def sym_qmax(bits):
    return lib().orc_sym_qmax(bits)


def packed_dim(D, bits):
    return lib().orc_packed_dim(D, bits)


def sym_cache_bytes(tokens, layers, kv_heads, D, bits):
    return lib().orc_sym_cache_bytes(tokens, layers, kv_heads, D, bits)


def sym_quant_rows(x, bits):
    """x: fp16 [..., D] -> (codes uint8 [..., packed_dim], scales uint16 [...])."""
    x = _u16(x)
    D = x.shape[-1]
    n = x.size // D
    pd = packed_dim(D, bits)
    assert pd > 0
    codes = np.zeros(x.shape[:-1] + (pd,), np.uint8)
    scales = np.zeros(x.shape[:-1], np.uint16)
    rc = lib().orc_sym_quant_rows(_p(x), n, D, bits, _p(codes), _p(scales))
    assert rc == 0
    return codes, scales


def sym_dequant_rows(codes, scales, D, bits):
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = _u16(scales)
    n = scales.size
    out = np.zeros(scales.shape + (D,), np.uint16)
    rc = lib().orc_sym_dequant_rows(_p(codes), _p(scales), n, D, bits, _p(out))
    assert rc == 0
    return out


def sym_unpack_rows(codes, D, bits):
    codes = np.ascontiguousarray(codes, np.uint8)
    pd = packed_dim(D, bits)
    n = codes.size // pd
    q = np.zeros(codes.shape[:-1] + (D,), np.int32)
    rc = lib().orc_sym_unpack_rows(_p(codes), n, D, bits, _p(q))
    assert rc == 0
    return q


def sym_quant_paged(x, bits, slot_mapping, codes, scales):
    """One layer: x fp16 [T][H][D]; codes uint8 [slots][H][pd], scales uint16 [slots][H] (updated in place)."""
    x = _u16(x)
    T, H, D = x.shape
    sm = np.ascontiguousarray(slot_mapping, np.int32)
    assert codes.flags.c_contiguous and scales.flags.c_contiguous
    n_slots = scales.shape[0]
    rc = lib().orc_sym_quant_paged(_p(x), T, H, D, bits, _p(sm), n_slots, _p(codes), _p(scales))
    assert rc == 0


def sym_dequant_paged(codes, scales, page_size, D, bits, block_table, seq_lens, max_len):
    """One layer: codes [num_pages*page_size][H][pd] -> fp16 bits [n_seqs][max_len][H][D]."""
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = _u16(scales)
    H = scales.shape[1]
    num_pages = scales.shape[0] // page_size
    bt = np.ascontiguousarray(block_table, np.int32)
    sl = np.ascontiguousarray(seq_lens, np.int32)
    n_seqs, max_blocks = bt.shape
    out = np.empty((n_seqs, max_len, H, D), np.uint16)
    rc = lib().orc_sym_dequant_paged(_p(codes), _p(scales), num_pages, page_size, H, D, bits,
                                     _p(bt), max_blocks, _p(sl), n_seqs, max_len, _p(out))
    assert rc == 0
    return out


# ------------------------------------------------------------------ KIVI
def kivi_boundary(offset, residual_length, group_size):
    return lib().orc_kivi_boundary(offset, residual_length, group_size)


def kivi_round_trip(x, lo, hi, per_channel, bits, group_size, eps=1e-8, want_params=False):
    """x: fp16 bits [B][H][S_cap][D]; returns (recon, codes, scale, min) with recon a new array."""
    x = _u16(x).copy()
    B, H, S_cap, D = x.shape
    n = hi - lo
    codes = scale = mn = None
    if want_params:
        cpr = (D * bits + 7) // 8
        codes = np.zeros((B, H, n, cpr), np.uint8)
        if per_channel:
            ng = (n + group_size - 1) // group_size
            scale = np.zeros((B, H, ng, D), np.float32)
        else:
            ng = (D + group_size - 1) // group_size
            scale = np.zeros((B, H, n, ng), np.float32)
        mn = np.zeros_like(scale)
    rc = lib().orc_kivi_round_trip(_p(x), B, H, S_cap, D, lo, hi, int(per_channel), bits,
                                   group_size, eps, _p(codes), _p(scale), _p(mn))
    assert rc == 0, rc
    return x, codes, scale, mn


def kivi_param_shape(B, H, S_cap, D, per_channel, group_size):
    """Shape of the fp16 scale / zero arrays of packed KIVI storage."""
    if per_channel:
        return (B, H, (S_cap + group_size - 1) // group_size, D)
    return (B, H, S_cap, (D + group_size - 1) // group_size)


def kivi_pack(x, lo, hi, per_channel, bits, group_size, eps=1e-8, into=None):
    """Packed KIVI storage of tokens [lo, hi) of x (fp16 bits [B][H][S_cap][D]).

    Returns (codes uint8 [B][H][S_cap][D*bits/8], scale uint16, zero uint16)
    with the parameter shapes of kivi_param_shape; `into` = such a triple to
    update in place (other tokens kept)."""
    x = _u16(x)
    B, H, S_cap, D = x.shape
    if into is None:
        shp = kivi_param_shape(B, H, S_cap, D, per_channel, group_size)
        into = (np.zeros((B, H, S_cap, D * bits // 8), np.uint8), np.zeros(shp, np.uint16),
                np.zeros(shp, np.uint16))
    codes, sc, zr = into
    assert codes.flags.c_contiguous and sc.flags.c_contiguous and zr.flags.c_contiguous
    rc = lib().orc_kivi_pack(_p(x), B, H, S_cap, D, lo, hi, int(per_channel), bits, group_size, eps,
                             _p(codes), _p(sc), _p(zr))
    assert rc == 0, rc
    return codes, sc, zr


def kivi_unpack(codes, scale, zero, lo, hi, per_channel, bits, group_size, D):
    """fp16 bits [B][H][S_cap][D]: tokens [lo, hi) reconstructed, others 0."""
    codes = np.ascontiguousarray(codes, np.uint8)
    B, H, S_cap = codes.shape[:3]
    out = np.zeros((B, H, S_cap, D), np.uint16)
    rc = lib().orc_kivi_unpack(_p(codes), _p(_u16(scale)), _p(_u16(zero)), B, H, S_cap, D, lo, hi,
                               int(per_channel), bits, group_size, _p(out))
    assert rc == 0, rc
    return out


# ------------------------------------------------------------------ decode attention
def attn_decode(q, k, v, scale):
    """One decode step of attention over dequantized rows, in float64.

    [MTPLX pull request #267, "feat(kv-cache): add q6 paged KV quantization",
     PR description: the cache's rows are dequantized and handed to
     scaled-dot-product attention] out = sum_t softmax_t(scale * q.k_t) v_t,
    the softmax taken after subtracting the largest score; no rows -> zeros.
    q: fp16 bits [D]; k, v: fp16 bits [T][D] (the dequantized cache rows).
    """
    qf = _u16(q).view(np.float16).astype(np.float64)
    kf = _u16(k).view(np.float16).astype(np.float64).reshape(-1, qf.size)
    vf = _u16(v).view(np.float16).astype(np.float64).reshape(-1, qf.size)
    if kf.shape[0] == 0:
        return np.zeros(qf.size)
    s = (kf @ qf) * float(scale)
    w = np.exp(s - s.max())
    return (w[:, None] * vf).sum(axis=0) / w.sum()


# ------------------------------------------------------------------ NUQ
def nuq_fit(u, L, iters):
    u = _u16(u)
    lev = np.zeros(L, np.float32)
    lib().orc_nuq_fit(_p(u), u.size, L, iters, _p(lev))
    return lev


def nuq_threshold(x, frac):
    x = _u16(x)
    return lib().orc_nuq_threshold(_p(x), x.size, frac)


def nuq_nearest(u_bits, levels):
    levels = np.ascontiguousarray(levels, np.float32)
    return lib().orc_nuq_nearest(int(u_bits), _p(levels), levels.size)


def nuq_fit_quant(keys, values, start_pos, bits, frac, iters, n_sink, fit_keys,
                  key_levels=None, key_thresh=None, out_cap=None):
    """Mirror of the library's NUQ call on host arrays. keys/values fp16 bits [BH][S][D].

    Returns a dict with key_levels, key_thresh, value_levels, k_codes, v_codes,
    k_out (pos, val), v_out (pos, val), k_recon, v_recon.
    """
    keys = _u16(keys)
    values = _u16(values)
    BH, S, D = keys.shape
    L = 1 << bits
    if key_levels is None:
        key_levels = np.zeros((BH, D, L), np.float32)
    else:
        key_levels = np.ascontiguousarray(key_levels, np.float32).copy()
    if key_thresh is None:
        key_thresh = np.zeros((BH, D), np.uint16)
    else:
        key_thresh = _u16(key_thresh).copy()
    value_levels = np.zeros((BH, S, L), np.float32)
    cpr = D * bits // 8
    k_codes = np.zeros((BH, S, cpr), np.uint8)
    v_codes = np.zeros((BH, S, cpr), np.uint8)
    cap = BH * S * D if out_cap is None else out_cap
    k_opos = np.zeros(max(cap, 1), np.int32)
    k_oval = np.zeros(max(cap, 1), np.uint16)
    v_opos = np.zeros(max(cap, 1), np.int32)
    v_oval = np.zeros(max(cap, 1), np.uint16)
    counts = np.zeros(2, np.int64)
    k_recon = np.zeros((BH, S, D), np.uint16)
    v_recon = np.zeros((BH, S, D), np.uint16)
    rc = lib().orc_nuq_fit_quant(_p(keys), _p(values), BH, S, D, start_pos, bits, frac, iters,
                                 n_sink, int(fit_keys), _p(key_levels), _p(key_thresh),
                                 _p(value_levels), _p(k_codes), _p(v_codes), _p(k_opos),
                                 _p(k_oval), _p(v_opos), _p(v_oval), cap, _p(counts),
                                 _p(k_recon), _p(v_recon))
    if rc != 0:
        raise ValueError("oracle nuq_fit_quant failed: %d" % rc)
    nk, nv = int(counts[0]), int(counts[1])
    return dict(key_levels=key_levels, key_thresh=key_thresh, value_levels=value_levels,
                k_codes=k_codes, v_codes=v_codes,
                k_out=(k_opos[:nk].copy(), k_oval[:nk].copy()),
                v_out=(v_opos[:nv].copy(), v_oval[:nv].copy()),
                k_recon=k_recon, v_recon=v_recon)
