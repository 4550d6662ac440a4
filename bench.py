"""Benchmark of the KV-cache quantize -> pack -> unpack -> dequantize path on one MI355X.

Default workload (the one the headline metric is quoted on): paged symmetric
q8/q6/q4 cache, 16 layers x 4 KV heads x head_dim 256, page size 16; 16
sequences x 32,768-token prefill quantized into pages (one launch covers all
16 layers), 256 single-token decode appends per sequence (one launch per step,
all layers), then a full-cache dequant sweep of 16 x 33,024 tokens. fp16 input
N(0,1) with 1% of channels x10 per (layer, head) and 5% of token positions
drawn from Laplace(0,1). One step = that whole sequence for each width in
--bits. Inputs are generated on the GPU and resident in HBM before timing.

Output: one JSON line (metric, value in GB/s of fp16-equivalent KV processed,
roofline of the dominant kernel, CPU-oracle baseline on a bounded sample).
Other workloads (--workload kivi | kivi_packed | long_context | single_layer |
nuq | attn_decode) print a line of the same form for their own configuration.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak, 8 TB/s
METRIC = "KV quant+pack / unpack+dequant GB/s (fp16-equiv) and % of HBM peak, 1 GPU"


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_sym_kivi.md")
ATTN_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_attn_decode.md")
CSRC = os.path.join(ROOT, "kv_cache_quantization_row_amd", "csrc")


def measured_traffic(kernel_class):
    """HBM bytes of one timed span of a kernel class from the committed
    rocprofv3 FETCH_SIZE/WRITE_SIZE summaries, or None when there is no entry
    or the kernel source changed since the counters were taken."""
    import hashlib
    import re

    launches, traffic_file = 1, TRAFFIC_FILE
    grid = {}  # a kernel launched at several grid sizes: the grid this span runs
    if kernel_class.startswith("attn_decode_q"):  # span: one launch pair per layer
        b = kernel_class.split("_q")[1].split("_")[0]
        launches = int(kernel_class.rsplit("_x", 1)[1])
        names, src = ["attn_decode_chunk_pg<%s, 256>" % b, "attn_decode_merge<256>"], "attn.hip"
        traffic_file = ATTN_TRAFFIC_FILE
    elif kernel_class.startswith("quant_prefill_q"):
        b = kernel_class[-1]
        names, src = ["sym_quant_v8<%s, 32, %d>" % (b, 1 if b == "8" else 2)], "sym.hip"
    elif kernel_class.startswith("dequant_sweep_q"):
        b = kernel_class[-1]
        names, src = ["sym_dequant_page<%s, 256>" % b], "sym.hip"
    elif kernel_class.startswith("kivi_keys_values_b"):
        b = kernel_class[-1]
        names, src = ["kivi_keys_fast<%s, 8, 4, false>" % b, "kivi_values_fast<%s, 8, 4, 1, false>" % b], "kivi.hip"
    elif kernel_class.startswith("kivi_pack_b"):
        b = kernel_class[-1]
        names, src = ["kivi_keys_fast<%s, 8, 4, true>" % b, "kivi_values_fast<%s, 8, 4, 4, true>" % b], "kivi.hip"
    elif kernel_class.startswith("kivi_unpack_b"):
        b = kernel_class[-1]
        names, src = ["kivi_unpack<%s, true>" % b, "kivi_unpack<%s, false>" % b], "kivi.hip"
    elif kernel_class == "quant_chunks_q6_x64":  # 64 chunk launches of the long-context cache
        launches, names, src = 64, ["sym_quant_v8<6, 32, 2>"], "sym.hip"
        grid = {"sym_quant_v8<6, 32, 2>": 8388608}
    elif kernel_class == "dequant_full_q6":
        names, src = ["sym_dequant_page<6, 256>"], "sym.hip"
        grid = {"sym_dequant_page<6, 256>": 538968064}
    else:
        return None
    if not os.path.exists(traffic_file):
        return None
    sha = hashlib.sha1(open(os.path.join(CSRC, src), "rb").read()).hexdigest()
    best = {}
    for line in open(traffic_file):
        m = re.match(r"traffic (.+?) grid=(\d+) bytes=(\d+) src_sha1=([0-9a-f]+)", line.strip())
        if m and m.group(1) in names and m.group(4) == sha:
            g = int(m.group(2))
            if m.group(1) in grid and g != grid[m.group(1)]:
                continue
            if g > best.get(m.group(1), (0, 0))[0]:
                best[m.group(1)] = (g, int(m.group(3)))
    if len(best) != len(names):
        return None
    return launches * sum(v[1] for v in best.values())


VALU_FILE = os.path.join(ROOT, "profiles", "valu_nuq_3bit_BH32_S4096_D128.md")
# VALU issue peak: each CU issues one wave64 VALU instruction per clock (4
# SIMDs, each taking 4 clocks for the 64 lanes of a wave on its 16 lanes):
# 256 CUs x 64 lanes x 2.4 GHz = 39.3 T lane-instructions per second
# (the 157.3 TFLOP/s fp32 figure counts an fma as 2 and packed fp32 as 2 more).
VALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12


def measured_valu(call):
    """VALU instructions (SQ_INSTS_VALU, summed over the kernels of one call)
    from the committed rocprofv3 counter summary, or None when absent or when
    the kernel source changed since the counters were taken."""
    import hashlib
    import re

    if not os.path.exists(VALU_FILE):
        return None
    sha = hashlib.sha1(open(os.path.join(CSRC, "nuq.hip"), "rb").read()).hexdigest()
    for line in open(VALU_FILE):
        m = re.match(r"valu_call (\S+) insts=(\d+) src_sha1=([0-9a-f]+)", line.strip())
        if m and m.group(1) == call and m.group(3) == sha:
            return int(m.group(2))
    return None


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


CPU_SHARE = 16  # host cores the GPU machine gives one GPU's jobs, whatever the machine has
CPU_CAP_NOTE = "threads = min(cores available to the process, 16): the host's CPU share for one GPU"


def cpu_threads():
    return max(1, min(CPU_SHARE, len(os.sched_getaffinity(0))))


def run_threads(fn, parts):
    """fn over parts, one thread each (the oracle's C calls release the GIL)."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(len(parts)) as ex:
        return list(ex.map(fn, parts))


class Timers:
    """Per-kernel-class HIP event pairs recorded on the launch stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def span(self, name):
        torch = self.torch
        timers = self

        class _S:
            def __enter__(self_):
                self_.a = torch.cuda.Event(enable_timing=True)
                self_.b = torch.cuda.Event(enable_timing=True)
                self_.a.record()

            def __exit__(self_, *exc):
                self_.b.record()
                timers.pairs.setdefault(name, []).append((self_.a, self_.b))

        return _S()

    def mean_ms(self):
        return {k: sum(a.elapsed_time(b) for a, b in v) / len(v) for k, v in self.pairs.items()}

    def count(self):
        return {k: len(v) for k, v in self.pairs.items()}


# --------------------------------------------------------------------------- paged symmetric
class PagedSym:
    """16 layers x 4 heads x 256, page 16, 16 seqs x 32,768 prefill + 256 appends + sweep."""

    def __init__(self, torch, args):
        self.torch = torch
        self.L, self.H, self.D, self.P = 16, 4, 256, 16
        self.S, self.T, self.N_DEC = 16, args.prefill_tokens, args.decode_steps
        self.bits_list = [int(b) for b in args.bits.split(",")]
        self.total = self.T + self.N_DEC
        self.name = "paged_sym"
        self.page_order = args.page_order

    def setup(self):
        torch = self.torch
        from kv_cache_quantization_row_amd import inputs, kvq

        self.kvq = kvq
        d = torch.device("cuda:0")
        L, H, D, P, S, T = self.L, self.H, self.D, self.P, self.S, self.T
        self.bt, self.num_pages = inputs.paged_block_table(S, self.total, P, seed=2002)
        if self.page_order == "identity":  # pages of each sequence consecutive in the pool
            import torch as _t
            self.bt = _t.arange(self.bt.numel(), dtype=_t.int32).view(self.bt.shape).contiguous()
        self.max_blocks = self.bt.shape[1]
        self.slot_prefill = inputs.slot_mapping_for(self.bt, P, 0, T).to(d)
        self.slot_dec = [inputs.slot_mapping_for(self.bt, P, T + i, 1).to(d) for i in range(self.N_DEC)]
        log("generating %d layers x %d tokens x %d x %d fp16 K and V" % (L, S * T, H, D))
        self.k = torch.empty((L, S * T, H, D), dtype=torch.float16, device=d)
        self.v = torch.empty_like(self.k)
        for l in range(L):
            self.k[l] = inputs.sym_layer(S * T, H, D, seed=2100 + l, device=d, laplace_token_frac=0.05,
                                         channel_seed=3100 + l)
            self.v[l] = inputs.sym_layer(S * T, H, D, seed=2200 + l, device=d, laplace_token_frac=0.05,
                                         channel_seed=3200 + l)
        self.kd = inputs.sym_layer(self.N_DEC * L * S, H, D, seed=2300, device=d,
                                   laplace_token_frac=0.05).view(self.N_DEC, L, S, H, D)
        self.vd = inputs.sym_layer(self.N_DEC * L * S, H, D, seed=2400, device=d,
                                   laplace_token_frac=0.05).view(self.N_DEC, L, S, H, D)
        # per-step views built here so the timed loop holds only the library calls
        self.kd_steps = [self.kd[i] for i in range(self.N_DEC)]
        self.vd_steps = [self.vd[i] for i in range(self.N_DEC)]
        slots = self.num_pages * P
        self.kc = torch.empty((L * slots * H * D,), dtype=torch.uint8, device=d)  # sized for q8
        self.vc = torch.empty_like(self.kc)
        self.ks = torch.empty((L, slots, H), dtype=torch.int16, device=d)
        self.vs = torch.empty_like(self.ks)
        self.ko = torch.empty((L, S, self.total, H, D), dtype=torch.float16, device=d)
        self.vo = torch.empty_like(self.ko)
        self.bt_d = self.bt.to(d)
        self.lens = torch.full((S,), self.total, dtype=torch.int32, device=d)
        self.lay = {b: kvq.layout(L, self.num_pages, P, H, D, b) for b in self.bits_list}
        torch.cuda.synchronize()

    def step(self, tm):
        kvq = self.kvq
        for b in self.bits_list:
            lay = self.lay[b]
            with tm.span("quant_prefill_q%d" % b):
                kvq.kvq_quant_sym(lay, self.k, self.v, self.slot_prefill, self.kc, self.ks, self.vc, self.vs)
            with tm.span("decode_append_q%d_x%d" % (b, self.N_DEC)):
                for i in range(self.N_DEC):
                    kvq.kvq_quant_sym(lay, self.kd_steps[i], self.vd_steps[i], self.slot_dec[i], self.kc, self.ks,
                                      self.vc, self.vs)
            with tm.span("dequant_sweep_q%d" % b):
                kvq.kvq_dequant_sym(lay, self.kc, self.ks, self.vc, self.vs, self.bt_d, self.lens,
                                    self.ko, self.vo)

    # elements processed per step (fp16 values quantized + values dequantized, K and V)
    def elems(self):
        per_bits = 2 * self.L * self.H * self.D * (self.S * self.T + self.N_DEC * self.S + self.S * self.total)
        return per_bits * len(self.bits_list)

    def kernel_bytes(self, name):
        """Algorithmic HBM bytes of one launch of a kernel class."""
        L, H, D, S = self.L, self.H, self.D, self.S
        b = int(name.split("_q")[1].split("_")[0])
        per_elem = 2 + b / 8 + 2 / D  # fp16 in/out + packed code + fp16 scale per row
        if name.startswith("quant_prefill"):
            return 2 * L * S * self.T * H * D * per_elem
        if name.startswith("dequant_sweep"):
            return 2 * L * S * self.total * H * D * per_elem
        return 2 * L * S * H * D * per_elem * self.N_DEC

    def config(self):
        return {"workload": "paged symmetric q8/q6/q4 KV cache: 16 layers x 4 KV heads x D=256, page 16, "
                            "16 seqs x %d-token prefill + %d decode appends + full dequant sweep"
                            % (self.T, self.N_DEC),
                "bits": self.bits_list, "layers": self.L, "kv_heads": self.H, "head_dim": self.D,
                "page_size": self.P, "seqs": self.S, "prefill_tokens": self.T,
                "decode_steps": self.N_DEC, "tokens_per_seq_after_decode": self.total}

    def cpu_baseline(self, budget_tokens):
        """Oracle (single thread) on layer 0, the first budget_tokens/16 tokens of each sequence."""
        import numpy as np
        import oracle
        from kv_cache_quantization_row_amd import inputs

        n = budget_tokens
        k = inputs.sym_layer(n, self.H, self.D, seed=2100, laplace_token_frac=0.05, channel_seed=3100)
        v = inputs.sym_layer(n, self.H, self.D, seed=2200, laplace_token_frac=0.05, channel_seed=3200)
        kk = k.view(__import__("torch").int16).numpy().view(np.uint16)
        vv = v.view(__import__("torch").int16).numpy().view(np.uint16)
        def run(parts):  # quantize + dequantize every part at every width; fp16-equivalent elements
            elems = 0
            for b in self.bits_list:
                for x in parts:
                    c, s = oracle.sym_quant_rows(x, b)
                    oracle.sym_dequant_rows(c, s, self.D, b)
                    elems += 2 * x.size
            return elems

        t0 = time.perf_counter()
        elems = run((kk, vv))
        dt1 = time.perf_counter() - t0
        # all cores: one thread per core over disjoint token ranges, each
        # calling the unmodified oracle (its C calls release the GIL)
        from concurrent.futures import ThreadPoolExecutor
        cores = cpu_threads()
        cut = [n * i // cores for i in range(cores + 1)]
        parts = [(kk[cut[i]:cut[i + 1]], vv[cut[i]:cut[i + 1]]) for i in range(cores)]
        t0 = time.perf_counter()
        with ThreadPoolExecutor(cores) as ex:
            elems_all = sum(ex.map(run, parts))
        dtn = time.perf_counter() - t0
        return {"value": round(2 * elems_all / dtn / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
                "value_1core": round(2 * elems / dt1 / 1e9, 4),
                "sample": "layer 0, %d tokens x 4 heads x 256 of K and V, quantize + dequantize at q%s: "
                          "%.1f s on one thread, %.2f s on %d threads over disjoint token ranges (%s)"
                          % (n, "/q".join(map(str, self.bits_list)), dt1, dtn, cores, CPU_CAP_NOTE)}


# --------------------------------------------------------------------------- KIVI
class Kivi:
    """B=8 x 16 layers folded (128), 8 heads, 8192 tokens, D=64, gs 32, residual 128, b in --kivi-bits."""

    def __init__(self, torch, args):
        self.torch = torch
        self.B, self.H, self.S, self.D, self.gs = 128, 8, 8192, 64, 32
        self.bits_list = [int(b) for b in args.kivi_bits.split(",")]
        self.steps, self.warmup = args.steps, args.warmup
        self.name = "kivi"

    def setup(self):
        torch = self.torch
        from kv_cache_quantization_row_amd import inputs, kvq

        self.kvq = kvq
        d = torch.device("cuda:0")
        self.hi = kvq.kvq_kivi_boundary(self.S, 128, self.gs)
        k0, v0 = inputs.kivi_kv(self.B, self.H, self.S, self.D, seed=1003, device=d)
        # the round trip is in place and its output sits on the quantization
        # grid (where the near-tie division fallback never fires), so every
        # timed call gets its own fresh copy of the input: 2 GiB per call
        n = len(self.bits_list) * (self.steps + self.warmup)
        log("KIVI: %d fresh input copies (%.0f GiB)" % (n, n * 2 * k0.numel() * 2 / 2 ** 30))
        self.copies = [(k0.clone(), v0.clone()) for _ in range(n)]
        del k0, v0
        self.i = 0
        torch.cuda.synchronize()

    def step(self, tm):
        for b in self.bits_list:
            k, v = self.copies[self.i % len(self.copies)]
            self.i += 1
            with tm.span("kivi_keys_values_b%d" % b):
                self.kvq.kvq_kivi_quant_dequant(k, v, 0, self.hi, b, self.gs)

    def elems(self):
        return 2 * self.B * self.H * self.hi * self.D * len(self.bits_list)

    def kernel_bytes(self, name):
        return 2 * self.B * self.H * self.hi * self.D * 4.0

    def config(self):
        return {"workload": "KIVI round trip: batch 8 x 16 layers (B=128) x 8 KV heads x 8192 tokens x D=64, "
                            "group 32, residual 128 (tokens [0, %d)), keys per channel, values per token" % self.hi,
                "bits": self.bits_list}

    def cpu_baseline(self, budget_tokens):
        import numpy as np
        import oracle
        from kv_cache_quantization_row_amd import inputs

        nbh = max(1, budget_tokens // self.S)
        k, v = inputs.kivi_kv(nbh, 1, self.S, self.D, seed=1003)
        t0 = time.perf_counter()
        elems = 0
        for b in self.bits_list:
            oracle.kivi_round_trip(k.numpy().view(np.uint16), 0, self.hi, 1, b, self.gs)
            oracle.kivi_round_trip(v.numpy().view(np.uint16), 0, self.hi, 0, b, self.gs)
            elems += 2 * nbh * self.hi * self.D
        dt = time.perf_counter() - t0
        return {"value": round(2 * elems / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": "%d (batch, head) slices of 8192 x 64 keys and values (%.1f s)" % (nbh, dt)}


# --------------------------------------------------------------------------- KIVI packed
class KiviPacked:
    """Packed KIVI storage on the KIVI shape: B=128 (batch 8 x 16 layers), 8
    heads, 8192 tokens, D=64, group 32, tokens [0, 8064) (residual 128):
    pack keys and values (codes + fp16 scale/zero), then unpack both, per b."""

    def __init__(self, torch, args):
        self.torch = torch
        self.B, self.H, self.S, self.D, self.gs = 128, 8, 8192, 64, 32
        self.bits_list = [int(b) for b in args.kivi_bits.split(",")]
        self.name = "kivi_packed"

    def setup(self):
        torch = self.torch
        from kv_cache_quantization_row_amd import inputs, kvq

        self.kvq = kvq
        d = torch.device("cuda:0")
        B, H, S, D, gs = self.B, self.H, self.S, self.D, self.gs
        self.hi = kvq.kvq_kivi_boundary(S, 128, gs)
        self.k, self.v = inputs.kivi_kv(B, H, S, D, seed=1003, device=d)
        self.st = {}
        for b in self.bits_list:
            kc = torch.empty((B, H, S, D * b // 8), dtype=torch.uint8, device=d)
            ks = torch.empty(kvq.kivi_param_shape(B, H, S, D, 1, gs), dtype=torch.int16, device=d)
            vs = torch.empty(kvq.kivi_param_shape(B, H, S, D, 0, gs), dtype=torch.int16, device=d)
            self.st[b] = (kc, ks, torch.empty_like(ks), torch.empty_like(kc), vs, torch.empty_like(vs))
        self.ko, self.vo = torch.empty_like(self.k), torch.empty_like(self.v)
        torch.cuda.synchronize()

    def step(self, tm):
        for b in self.bits_list:
            kc, ks, kz, vc, vs, vz = self.st[b]
            with tm.span("kivi_pack_b%d" % b):
                self.kvq.kvq_kivi_pack(self.k, self.v, 0, self.hi, b, self.gs, k_codes=kc, k_scale=ks, k_zero=kz,
                                       v_codes=vc, v_scale=vs, v_zero=vz)
            with tm.span("kivi_unpack_b%d" % b):
                self.kvq.kvq_kivi_unpack(kc, ks, kz, vc, vs, vz, 0, self.hi, b, self.gs, self.ko, self.vo)

    def elems(self):  # fp16 K and V elements packed plus unpacked
        return 2 * 2 * self.B * self.H * self.hi * self.D * len(self.bits_list)

    def kernel_bytes(self, name):
        """fp16 in (pack) or out (unpack), b-bit codes, fp16 (scale, zero) pairs."""
        b = int(name.rsplit("_b", 1)[1])
        BH, n, D, gs = self.B * self.H, self.hi, self.D, self.gs
        elems = 2 * BH * n * D
        params = BH * (-(-n // gs)) * D * 4 + BH * n * (-(-D // gs)) * 4
        return elems * 2 + elems * b / 8 + params

    def config(self):
        return {"workload": "KIVI packed storage: batch 8 x 16 layers (B=128) x 8 KV heads x 8192 tokens x D=64, "
                            "group 32, tokens [0, %d): pack keys + values to b-bit codes with fp16 scale/zero, "
                            "then unpack both" % self.hi, "bits": self.bits_list}

    def cpu_baseline(self, budget_tokens):
        import numpy as np
        import oracle
        from kv_cache_quantization_row_amd import inputs

        nbh = max(1, budget_tokens // self.S)
        k, v = inputs.kivi_kv(nbh, 1, self.S, self.D, seed=1003)
        kn, vn = k.numpy().view(np.uint16), v.numpy().view(np.uint16)
        t0 = time.perf_counter()
        elems = 0
        for b in self.bits_list:
            pk = oracle.kivi_pack(kn, 0, self.hi, 1, b, self.gs)
            pv = oracle.kivi_pack(vn, 0, self.hi, 0, b, self.gs)
            oracle.kivi_unpack(*pk, 0, self.hi, 1, b, self.gs, self.D)
            oracle.kivi_unpack(*pv, 0, self.hi, 0, b, self.gs, self.D)
            elems += 2 * 2 * nbh * self.hi * self.D
        dt = time.perf_counter() - t0
        return {"value": round(2 * elems / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": "%d (batch, head) slices of 8192 x 64 keys and values, pack + unpack (%.1f s)" % (nbh, dt)}


# --------------------------------------------------------------------------- NUQ
class Nuq:
    """Batch 4 x 8 KV heads (BH=32), 4096-token prefill, D=128, 3 bits, 1% outliers,
    8 Lloyd iterations, 4 sinks; then 64 single-token decode calls against the
    frozen key levels. Student-t(4) K/V. The 64 MiB working set is rotated over
    16 resident copies (~1 GiB) so the 256 MB last-level cache does not serve it."""

    def __init__(self, torch, args):
        self.torch = torch
        self.BH, self.S, self.D, self.bits = 32, 4096, 128, 3
        self.frac, self.iters, self.ns, self.n_dec = 0.01, args.lloyd_iters, 4, 64
        self.copies = 16
        self.name = "nuq"

    def setup(self):
        torch = self.torch
        from kv_cache_quantization_row_amd import inputs, kvq

        self.kvq = kvq
        d = torch.device("cuda:0")
        BH, S, D, L = self.BH, self.S, self.D, 1 << self.bits
        self.k = [inputs.student_t((BH, S, D), 4, seed=1004 + 10 * i, device=d) for i in range(self.copies)]
        self.v = [inputs.student_t((BH, S, D), 4, seed=1005 + 10 * i, device=d) for i in range(self.copies)]
        self.kd = inputs.student_t((self.n_dec, BH, 1, D), 4, seed=5000, device=d)
        self.vd = inputs.student_t((self.n_dec, BH, 1, D), 4, seed=6000, device=d)
        self.kd_steps = [self.kd[t] for t in range(self.n_dec)]  # views built before timing
        self.vd_steps = [self.vd[t] for t in range(self.n_dec)]
        z = lambda *sh, dt=torch.float32: torch.zeros(sh, dtype=dt, device=d)
        self.kl, self.kt = z(BH, D, L), z(BH, D, dt=torch.int16)
        self.vl, self.vl1 = z(BH, S, L), z(BH, 1, L)
        cb = D * self.bits // 8
        self.kc, self.vc = z(BH, S, cb, dt=torch.uint8), z(BH, S, cb, dt=torch.uint8)
        self.kc1, self.vc1 = z(BH, 1, cb, dt=torch.uint8), z(BH, 1, cb, dt=torch.uint8)
        cap = max(kvq.kvq_nuq_outlier_bound(BH, S, D, 0, self.ns, self.frac, 1, w) for w in (0, 1))
        cap1 = max(kvq.kvq_nuq_outlier_bound(BH, 1, D, S, self.ns, self.frac, 0, w) for w in (0, 1))
        self.lists = [z(cap, dt=torch.int32), z(cap, dt=torch.int16), z(cap, dt=torch.int32), z(cap, dt=torch.int16)]
        self.lists1 = [z(cap1, dt=torch.int32), z(cap1, dt=torch.int16), z(cap1, dt=torch.int32), z(cap1, dt=torch.int16)]
        self.cnt, self.cnt1 = z(2, dt=torch.int64), z(2, dt=torch.int64)
        self.ws = z(kvq.kvq_nuq_workspace_bytes(BH, S, D, self.bits, 0, self.ns, self.frac, 1), dt=torch.uint8)
        self.ws1 = z(kvq.kvq_nuq_workspace_bytes(BH, 1, D, self.bits, S, self.ns, self.frac, 0), dt=torch.uint8)
        self.i = 0
        torch.cuda.synchronize()

    def step(self, tm):
        kvq = self.kvq
        c = self.i % self.copies
        self.i += 1
        with tm.span("nuq_prefill"):
            kvq.kvq_nuq_fit_quant(self.k[c], self.v[c], 0, self.bits, self.frac, self.iters, self.ns, 1,
                                  self.kl, self.kt, self.vl, self.kc, self.vc, *self.lists, self.cnt, self.ws)
        with tm.span("nuq_decode_x%d" % self.n_dec):
            for t in range(self.n_dec):
                kvq.kvq_nuq_fit_quant(self.kd_steps[t], self.vd_steps[t], self.S + t, self.bits, self.frac, self.iters,
                                      self.ns, 0, self.kl, self.kt, self.vl1, self.kc1, self.vc1,
                                      *self.lists1, self.cnt1, self.ws1)

    def elems(self):
        return 2 * self.BH * self.D * (self.S + self.n_dec)

    def kernel_bytes(self, name):
        BH, S, D, L = self.BH, self.S, self.D, 1 << self.bits
        n_out = int(self.cnt.sum().item())
        if name == "nuq_prefill":
            return (2 * 2 * BH * S * D + 2 * BH * S * D * self.bits / 8 + BH * D * (4 * L + 2)
                    + BH * S * 4 * L + 6 * n_out)
        n_out1 = int(self.cnt1.sum().item())
        return self.n_dec * (2 * 2 * BH * D + 2 * BH * D * self.bits / 8 + BH * D * (4 * L + 2)
                             + BH * 4 * L + 6 * n_out1)

    def roofline(self, dom, kernels, means):
        """The prefill call is bound by the fits' VALU work, not by HBM: report
        its VALU issue rate (counted instructions x 64 lanes over the live call
        time) against the VALU peak; the HBM fraction stays beside it."""
        if dom != "nuq_prefill":
            return None
        insts = measured_valu("nuq_prefill")
        if insts is None:
            return None
        achieved = insts * 64 / (means[dom] / 1e3) / 1e12
        return {"bound": "alu", "kernel": dom, "achieved": round(achieved, 3), "peak": round(VALU_PEAK_TOPS, 2),
                "unit": "TOP/s (VALU lane-instructions)", "frac": round(achieved / VALU_PEAK_TOPS, 4),
                "traffic": None, "valu_instructions": insts, "frac_hbm": kernels[dom]["frac_hbm"],
                "algorithmic_bytes": int(self.kernel_bytes(dom))}

    def config(self):
        return {"workload": "KVQuant-style NUQ 3-bit: batch 4 x 8 KV heads, D=128, 4096-token prefill "
                            "(1%% outliers, %d Lloyd iterations, 4 sinks) + %d decode calls" % (self.iters, self.n_dec),
                "bits": self.bits, "outlier_fraction": self.frac, "lloyd_iters": self.iters,
                "n_sink": self.ns, "rotation_copies": self.copies}

    def cpu_baseline(self, budget_tokens):
        import numpy as np
        import oracle
        from kv_cache_quantization_row_amd import inputs

        nbh = 1
        k = inputs.student_t((nbh, self.S, self.D), 4, seed=1004).numpy().view(np.uint16)
        v = inputs.student_t((nbh, self.S, self.D), 4, seed=1005).numpy().view(np.uint16)
        t0 = time.perf_counter()
        oracle.nuq_fit_quant(k, v, 0, self.bits, self.frac, self.iters, self.ns, 1)
        dt = time.perf_counter() - t0
        return {"value": round(2 * 2 * nbh * self.S * self.D / dt / 1e9, 5), "unit": "GB/s", "cores": 1,
                "kind": "oracle", "sample": "prefill of 1 of 32 (batch, head) slices, 4096 x 128 K and V (%.1f s)" % dt}


# --------------------------------------------------------------------------- long context
class LongContext:
    """One 262,144-token sequence, 16 layers x 4 KV heads x D=256, q6, page 16:
    quantized in 64 chunks of 4096 tokens (one launch per chunk, all layers,
    alternating over two streams), 1,024 single-token appends, then a full
    dequant of 263,168 tokens."""

    def __init__(self, torch, args):
        self.torch = torch
        self.L, self.H, self.D, self.P, self.bits = 16, 4, 256, 16, 6
        self.T, self.CH, self.N_DEC = 262144, 4096, args.decode_steps_long
        self.total = self.T + self.N_DEC
        self.name = "long_context"

    def setup(self):
        torch = self.torch
        from kv_cache_quantization_row_amd import inputs, kvq

        self.kvq = kvq
        d = torch.device("cuda:0")
        L, H, D, P = self.L, self.H, self.D, self.P
        self.bt, self.num_pages = inputs.paged_block_table(1, self.total, P, seed=5005)
        nch = self.T // self.CH
        self.slots = [inputs.slot_mapping_for(self.bt, P, c * self.CH, self.CH).to(d) for c in range(nch)]
        self.slot_dec = inputs.slot_mapping_for(self.bt, P, self.T, self.N_DEC).to(d)
        log("generating %d chunks of %d layers x %d tokens" % (nch, L, self.CH))
        self.k = torch.empty((nch, L, self.CH, H, D), dtype=torch.float16, device=d)
        self.v = torch.empty_like(self.k)
        for l in range(L):
            self.k[:, l] = inputs.sym_layer(self.T, H, D, seed=7100 + l, device=d, channel_seed=8100 + l).view(nch, self.CH, H, D)
            self.v[:, l] = inputs.sym_layer(self.T, H, D, seed=7200 + l, device=d, channel_seed=8200 + l).view(nch, self.CH, H, D)
        self.kd = inputs.sym_layer(self.N_DEC * L, H, D, seed=7300, device=d).view(self.N_DEC, L, 1, H, D)
        self.vd = inputs.sym_layer(self.N_DEC * L, H, D, seed=7400, device=d).view(self.N_DEC, L, 1, H, D)
        # per-step views built here so the timed loop holds only the library calls
        self.kd_steps = [self.kd[i] for i in range(self.N_DEC)]
        self.vd_steps = [self.vd[i] for i in range(self.N_DEC)]
        self.sm_steps = [self.slot_dec[i:i + 1] for i in range(self.N_DEC)]
        slots = self.num_pages * P
        pd = kvq.kvq_packed_dim(D, self.bits)
        self.kc = torch.empty((L, slots, H, pd), dtype=torch.uint8, device=d)
        self.vc = torch.empty_like(self.kc)
        self.ks = torch.empty((L, slots, H), dtype=torch.int16, device=d)
        self.vs = torch.empty_like(self.ks)
        self.ko = torch.empty((L, 1, self.total, H, D), dtype=torch.float16, device=d)
        self.vo = torch.empty_like(self.ko)
        self.bt_d = self.bt.to(d)
        self.lens = torch.full((1,), self.total, dtype=torch.int32, device=d)
        self.lay = kvq.layout(L, self.num_pages, P, H, D, self.bits)
        self.side = torch.cuda.Stream()  # default priority
        torch.cuda.synchronize()

    def step(self, tm):
        kvq, torch = self.kvq, self.torch
        with tm.span("quant_chunks_q6_x%d" % len(self.slots)):
            # consecutive chunks are independent: even chunks on the timing
            # stream, odd ones on a second stream of the same (default)
            # priority, so one launch's drain overlaps the next one's ramp;
            # the second stream is forked from and joined back into the first
            main = torch.cuda.current_stream()
            fork = torch.cuda.Event()
            fork.record(main)
            self.side.wait_event(fork)
            for c, sm in enumerate(self.slots):
                st = main if c % 2 == 0 else self.side
                kvq.kvq_quant_sym(self.lay, self.k[c], self.v[c], sm, self.kc, self.ks, self.vc, self.vs, stream=st)
            join = torch.cuda.Event()
            join.record(self.side)
            main.wait_event(join)
        with tm.span("decode_append_q6_x%d" % self.N_DEC):
            for i in range(self.N_DEC):
                kvq.kvq_quant_sym(self.lay, self.kd_steps[i], self.vd_steps[i], self.sm_steps[i], self.kc, self.ks,
                                  self.vc, self.vs)
        with tm.span("dequant_full_q6"):
            kvq.kvq_dequant_sym(self.lay, self.kc, self.ks, self.vc, self.vs, self.bt_d, self.lens, self.ko, self.vo)

    def elems(self):
        return 2 * self.L * self.H * self.D * (self.T + self.N_DEC + self.total)

    def kernel_bytes(self, name):
        per = 2 + self.bits / 8 + 2 / self.D
        rows = 2 * self.L * self.H
        if name.startswith("quant_chunks"):
            return rows * self.T * self.D * per
        if name.startswith("dequant_full"):
            return rows * self.total * self.D * per
        return rows * self.N_DEC * self.D * per

    def config(self):
        return {"workload": "long-context q6 paged cache: one 262,144-token sequence, 16 layers x 4 KV heads x "
                            "D=256, 64 chunks of 4096 tokens + %d appends + full dequant of %d tokens"
                            % (self.N_DEC, self.total), "bits": self.bits,
                "packed_GiB": round(self.kvq.kvq_sym_cache_bytes(self.T, 16, 4, 256, 6) / 2 ** 30, 4)}

    def cpu_baseline(self, budget_tokens):
        """Oracle on chunks 0-3 of layer 0 (16,384 tokens: quantize into pages,
        then dequantize them), on all CPU_SHARE threads over disjoint token
        ranges; extrapolated linearly to the whole workload."""
        import numpy as np
        import oracle
        from kv_cache_quantization_row_amd import inputs

        n = 4 * self.CH
        k = inputs.sym_layer(n, self.H, self.D, seed=7100, channel_seed=8100)
        v = inputs.sym_layer(n, self.H, self.D, seed=7200, channel_seed=8200)
        kk = k.view(__import__("torch").int16).numpy().view(np.uint16)
        vv = v.view(__import__("torch").int16).numpy().view(np.uint16)

        def run(part):
            elems = 0
            for x in part:
                c, sc = oracle.sym_quant_rows(x, self.bits)
                oracle.sym_dequant_rows(c, sc, self.D, self.bits)
                elems += 2 * x.size
            return elems

        cores = cpu_threads()
        cut = [n * i // cores for i in range(cores + 1)]
        t0 = time.perf_counter()
        elems = sum(run_threads(run, [(kk[cut[i]:cut[i + 1]], vv[cut[i]:cut[i + 1]]) for i in range(cores)]))
        dt = time.perf_counter() - t0
        rate = 2 * elems / dt / 1e9
        whole_s = 2 * self.elems() / (rate * 1e9)
        return {"value": round(rate, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
                "sample": "chunks 0-3 of layer 0 (16,384 tokens x 4 heads x 256, K and V): quantize + dequantize, "
                          "%.2f s on %d threads (%s); extrapolated linearly: %.0f s for the whole workload"
                          % (dt, cores, CPU_CAP_NOTE, whole_s)}


# --------------------------------------------------------------------------- decode attention
class AttnDecode:
    """Decode attention over the packed pools of the paged configuration:
    16 layers x 4 KV heads x D=256, page 16, 16 sequences x 33,024 tokens
    (32,768 prefill + 256 appends) in randomly assigned pages, 4 query heads
    per KV head; one step = one decode token of every sequence through all 16
    layers (one launch per layer) for each width in --bits."""

    def __init__(self, torch, args):
        self.torch = torch
        self.L, self.H, self.D, self.P, self.G = 16, 4, 256, 16, args.attn_group
        self.S, self.len = 16, args.prefill_tokens + args.decode_steps
        self.bits_list = [int(b) for b in args.bits.split(",")]
        self.name = "attn_decode"

    def setup(self):
        torch = self.torch
        from kv_cache_quantization_row_amd import inputs, kvq

        self.kvq = kvq
        d = torch.device("cuda:0")
        L, H, D, P, S, T = self.L, self.H, self.D, self.P, self.S, self.len
        bt, self.num_pages = inputs.paged_block_table(S, T, P, seed=2002)
        slots = self.num_pages * P
        slot_map = inputs.slot_mapping_for(bt, P, 0, T).to(d)
        self.bt = bt.to(d)
        self.lens = torch.full((S,), T, dtype=torch.int32, device=d)
        self.pools = {}
        for b in self.bits_list:
            pd = kvq.kvq_packed_dim(D, b)
            lay = kvq.layout(L, self.num_pages, P, H, D, b)
            kc = torch.empty((L, slots, H, pd), dtype=torch.uint8, device=d)
            vc = torch.empty_like(kc)
            ks = torch.empty((L, slots, H), dtype=torch.int16, device=d)
            vs = torch.empty_like(ks)
            self.pools[b] = (lay, kc, ks, vc, vs)
        for l in range(L):
            log("filling layer %d of the pools (%d tokens)" % (l, S * T))
            k = inputs.sym_layer(S * T, H, D, seed=2100 + l, device=d, laplace_token_frac=0.05,
                                 channel_seed=3100 + l)[None]
            v = inputs.sym_layer(S * T, H, D, seed=2200 + l, device=d, laplace_token_frac=0.05,
                                 channel_seed=3200 + l)[None]
            for b, (lay, kc, ks, vc, vs) in self.pools.items():
                kvq.kvq_quant_sym(lay, k, v, slot_map, kc, ks, vc, vs, layer0=l)
            del k, v
        self.q = inputs.sym_layer(L * S, H * self.G, D, seed=2500, device=d, outlier_frac=0).view(L, S, H * self.G, D)
        self.out = torch.empty((S, H * self.G, D), dtype=torch.float16, device=d)
        self.ws = torch.empty(kvq.kvq_attn_workspace_bytes(S, H * self.G, D, T), dtype=torch.uint8, device=d)
        self.scale = 1.0 / D ** 0.5
        torch.cuda.synchronize()

    def step(self, tm):
        kvq = self.kvq
        for b in self.bits_list:
            lay, kc, ks, vc, vs = self.pools[b]
            with tm.span("attn_decode_q%d_x%d" % (b, self.L)):
                for l in range(self.L):
                    kvq.kvq_attn_decode_sym(lay, kc, ks, vc, vs, l, self.q[l], self.bt, self.lens, self.len,
                                            self.scale, self.out, self.ws)

    # fp16-equivalent K and V elements read per step
    def elems(self):
        return 2 * self.L * self.S * self.len * self.H * self.D * len(self.bits_list)

    def kernel_bytes(self, name):
        """Algorithmic bytes of the 16 launches of one width: packed codes and
        fp16 scales of every cached K and V row, the queries and the outputs."""
        b = int(name.split("_q")[1].split("_")[0])
        rows = 2 * self.S * self.len * self.H
        qo = 2 * self.S * self.H * self.G * self.D * 2
        return self.L * (rows * (self.D * b // 8 + 2) + qo)

    def config(self):
        return {"workload": "paged decode attention over packed q8/q6/q4 codes: 16 layers x 4 KV heads x D=256, "
                            "page 16, 16 seqs x %d tokens, %d query heads per KV head, one decode token per "
                            "sequence through all layers" % (self.len, self.G),
                "bits": self.bits_list, "layers": self.L, "kv_heads": self.H, "q_heads": self.H * self.G,
                "head_dim": self.D, "page_size": self.P, "seqs": self.S, "tokens_per_seq": self.len}

    def cpu_baseline(self, budget_tokens):
        """Oracle on layer 0 of one sequence (budget_tokens/4 tokens): dequantize
        the rows, then attention for every query head, per width."""
        import numpy as np
        import torch as _t
        import oracle
        from kv_cache_quantization_row_amd import inputs

        n = max(budget_tokens // 4, 1)
        H, D, G = self.H, self.D, self.G
        k = inputs.sym_layer(n, H, D, seed=2100, laplace_token_frac=0.05, channel_seed=3100)
        v = inputs.sym_layer(n, H, D, seed=2200, laplace_token_frac=0.05, channel_seed=3200)
        q = inputs.sym_layer(1, H * G, D, seed=2500, outlier_frac=0)[0]
        kk, vv, qq = (x.contiguous().view(_t.int16).numpy().view(np.uint16) for x in (k, v, q))
        t0 = time.perf_counter()
        for b in self.bits_list:
            for h in range(H):
                kd = oracle.sym_dequant_rows(*oracle.sym_quant_rows(kk[:, h], b), D, b)
                vd = oracle.sym_dequant_rows(*oracle.sym_quant_rows(vv[:, h], b), D, b)
                for j in range(G):
                    oracle.attn_decode(qq[h * G + j], kd, vd, self.scale)
        dt = time.perf_counter() - t0
        elems = 2 * n * H * D * len(self.bits_list)
        return {"value": round(2 * elems / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": "layer 0, one sequence of %d tokens x 4 KV heads x 256, %d query heads per KV head, "
                          "quantize + dequantize + attention at q%s (%.1f s; quantization included, so an "
                          "upper bound on the oracle's time)" % (n, G, "/q".join(map(str, self.bits_list)), dt)}


# --------------------------------------------------------------------------- single layer
class SingleLayer:
    """One layer, K and V each [1024][4][256], q6, 64 pages of 16 (slots in token
    order), then the read-back; 256 resident copies (~1 GiB) rotated per call."""

    def __init__(self, torch, args):
        self.torch = torch
        self.T, self.H, self.D, self.P, self.bits, self.copies = 1024, 4, 256, 16, 6, 256
        self.name = "single_layer"

    def setup(self):
        torch = self.torch
        from kv_cache_quantization_row_amd import inputs, kvq

        self.kvq = kvq
        d = torch.device("cuda:0")
        T, H, D, P, C = self.T, self.H, self.D, self.P, self.copies
        self.k = torch.stack([inputs.sym_layer(T, H, D, seed=1001 + 2 * i, device=d) for i in range(C)])[:, None]
        self.v = torch.stack([inputs.sym_layer(T, H, D, seed=1002 + 2 * i, device=d) for i in range(C)])[:, None]
        pd = kvq.kvq_packed_dim(D, self.bits)
        self.kc = torch.empty((C, T, H, pd), dtype=torch.uint8, device=d)
        self.vc = torch.empty_like(self.kc)
        self.ks = torch.empty((C, T, H), dtype=torch.int16, device=d)
        self.vs = torch.empty_like(self.ks)
        self.ko = torch.empty((C, 1, 1, T, H, D), dtype=torch.float16, device=d)
        self.vo = torch.empty_like(self.ko)
        self.slot = torch.arange(T, dtype=torch.int32, device=d)
        self.bt = torch.arange(T // P, dtype=torch.int32, device=d)[None]
        self.lens = torch.full((1,), T, dtype=torch.int32, device=d)
        self.lay = kvq.layout(1, T // P, P, H, D, self.bits)
        # the same 256-call loops captured once as HIP graphs (launch-bound
        # work replayed without a host call per kernel); the first pass runs
        # on a side stream of default priority, as capture expects
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self._quant_all()
            self._dequant_all()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.gq, self.gd = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.gq):
            self._quant_all()
        with torch.cuda.graph(self.gd):
            self._dequant_all()
        torch.cuda.synchronize()

    def _quant_all(self):
        for c in range(self.copies):
            self.kvq.kvq_quant_sym(self.lay, self.k[c], self.v[c], self.slot, self.kc[c], self.ks[c], self.vc[c],
                                   self.vs[c])

    def _dequant_all(self):
        for c in range(self.copies):
            self.kvq.kvq_dequant_sym(self.lay, self.kc[c], self.ks[c], self.vc[c], self.vs[c], self.bt, self.lens,
                                     self.ko[c], self.vo[c])

    def step(self, tm):
        """The round trip twice: 256 calls from the host, then the captured graphs."""
        with tm.span("quant_q6_x%d" % self.copies):
            self._quant_all()
        with tm.span("dequant_q6_x%d" % self.copies):
            self._dequant_all()
        with tm.span("quant_q6_graph_x%d" % self.copies):
            self.gq.replay()
        with tm.span("dequant_q6_graph_x%d" % self.copies):
            self.gd.replay()

    def roofline(self, dom, kernels, means):
        """The kernels' own rate: the graph replays, where a launch is not
        separated from the next by a host call (the host-called loops beside
        them measure the binding and launch path, about 10 us per call)."""
        name = max(("quant_q6_graph_x%d" % self.copies, "dequant_q6_graph_x%d" % self.copies),
                   key=lambda n: means[n])
        return {"bound": "hbm", "kernel": name, "achieved": kernels[name]["GB/s"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": kernels[name]["frac_hbm"], "traffic": None,
                "algorithmic_bytes": int(self.kernel_bytes(name))}

    def elems(self):  # both passes of the step
        return 2 * 2 * 2 * self.T * self.H * self.D * self.copies

    def kernel_bytes(self, name):
        return 2 * self.T * self.H * self.D * (2 + self.bits / 8 + 2 / self.D) * self.copies

    def config(self):
        return {"workload": "single-layer q6 round trip: K and V [1024][4][256], 64 pages of 16, rotated over "
                            "%d resident copies" % self.copies, "bits": self.bits}

    def cpu_baseline(self, budget_tokens):
        """The oracle on the whole configuration (one layer, K and V [1024][4][256]:
        quantize into pages, dequantize back), single thread, repeated."""
        import numpy as np
        import torch as _t
        import oracle
        from kv_cache_quantization_row_amd import inputs

        T, H, D, P = self.T, self.H, self.D, self.P
        k = inputs.sym_layer(T, H, D, seed=1001).view(_t.int16).numpy().view(np.uint16)
        v = inputs.sym_layer(T, H, D, seed=1002).view(_t.int16).numpy().view(np.uint16)
        pd = oracle.packed_dim(D, self.bits)
        slot = np.arange(T, dtype=np.int32)
        bt = np.arange(T // P, dtype=np.int32)[None]
        reps, t0 = 0, time.perf_counter()
        while reps < 3 or time.perf_counter() - t0 < 2.0:
            for x in (k, v):
                codes = np.zeros((T, H, pd), np.uint8)
                sc = np.zeros((T, H), np.uint16)
                oracle.sym_quant_paged(x, self.bits, slot, codes, sc)
                oracle.sym_dequant_paged(codes, sc, P, D, self.bits, bt, np.array([T], np.int32), T)
            reps += 1
        dt = (time.perf_counter() - t0) / reps
        return {"value": round(2 * 2 * 2 * T * H * D / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": "the whole configuration (quantize into 64 pages + dequantize, K and V), %d repetitions, "
                          "%.1f ms each, one thread" % (reps, dt * 1e3)}


class Caches:
    """The cache objects over the kernels, in decode: a NuqCache with a
    4096-token prefill (batch 4 x 8 KV heads, D=128, 3 bits, 1% outliers, 8
    Lloyd iterations, 4 sinks) takes 64 one-token decode steps
    (update_and_fetch: fit, quantize, reconstruction appended; no host sync);
    a packed KiviCache on the KIVI shape (batch 8 x 16 layers folded, 8 KV
    heads, D=64, b=2, group 32, residual 128) with an 8192-token prefill
    takes 32 one-token decode steps, each returning the whole fp16 K/V
    (kvq_kivi_unpack of the packed prefix plus the fp16 window; one step in
    32 also packs a new group)."""

    def __init__(self, torch, args):
        self.torch = torch
        self.name = "caches"
        self.n_nuq, self.n_kivi = 64, 32

    def setup(self):
        torch = self.torch
        from kv_cache_quantization_row_amd import caches, inputs

        d = torch.device("cuda:0")
        self.caches = caches
        B, H, D = 4, 8, 128
        self.nk = inputs.student_t((B * H, 4096, D), 4, seed=1004, device=d).view(B, H, 4096, D)
        self.nv = inputs.student_t((B * H, 4096, D), 4, seed=1005, device=d).view(B, H, 4096, D)
        n_dec = self.n_nuq * 64
        self.nkd = inputs.student_t((B * H, n_dec, D), 4, seed=5000, device=d).view(B, H, n_dec, D)
        self.nvd = inputs.student_t((B * H, n_dec, D), 4, seed=6000, device=d).view(B, H, n_dec, D)
        self.nuq_steps = [(self.nkd[:, :, t:t + 1].contiguous(), self.nvd[:, :, t:t + 1].contiguous())
                          for t in range(n_dec)]
        Bk, Hk, Dk = 128, 8, 64
        self.kk, self.kv = inputs.kivi_kv(Bk, Hk, 8192 + 64 * self.n_kivi, Dk, seed=1003, device=d)
        self.kivi_steps = [(self.kk[:, :, 8192 + t:8193 + t].contiguous(), self.kv[:, :, 8192 + t:8193 + t].contiguous())
                           for t in range(64 * self.n_kivi)]
        self._fresh()
        torch.cuda.synchronize()

    def _fresh(self):
        self.nuq = self.caches.NuqCache(3, 0.01, 8, 4)
        self.nuq.update_and_fetch(self.nk, self.nv)
        self.kivi = self.caches.KiviCache(2, 32, 128, storage="packed")
        self.kivi.update_and_fetch(self.kk[:, :, :8192].contiguous(), self.kv[:, :, :8192].contiguous())
        self.t_nuq = self.t_kivi = 0

    def step(self, tm):
        if self.t_nuq + self.n_nuq > len(self.nuq_steps) or self.t_kivi + self.n_kivi > len(self.kivi_steps):
            self._fresh()
        with tm.span("nuq_cache_decode_x%d" % self.n_nuq):
            for i in range(self.n_nuq):
                self.nuq.update_and_fetch(*self.nuq_steps[self.t_nuq + i])
        self.t_nuq += self.n_nuq
        with tm.span("kivi_packed_cache_decode_x%d" % self.n_kivi):
            for i in range(self.n_kivi):
                self.kivi.update_and_fetch(*self.kivi_steps[self.t_kivi + i])
        self.t_kivi += self.n_kivi

    def elems(self):  # fp16 K and V elements handed back by the KIVI fetches
        return 2 * 128 * 8 * 8200 * 64 * self.n_kivi

    def kernel_bytes(self, name):
        if name.startswith("kivi"):  # per step: packed prefix read, fp16 K/V written, window copied
            BH, n, D = 128 * 8, 8200, 64
            return self.n_kivi * 2 * BH * (n * D * 2 + n * D * 2 / 8 + (n // 32) * D * 4 / 2 + n * 4)
        BH, D, L = 32, 128, 8
        return self.n_nuq * (2 * 2 * BH * D + 2 * BH * D * 3 / 8 + BH * D * (4 * L + 2) + BH * 4 * L)

    def config(self):
        return {"workload": "cache objects in decode: NuqCache (batch 4 x 8 KV heads, D=128, 3 bits, 4096-token "
                            "prefill) 64 one-token steps; packed KiviCache (B=128, 8 KV heads, D=64, b=2, group 32, "
                            "8192-token prefill) 32 one-token steps returning the whole fp16 K/V"}

    def cpu_baseline(self, budget_tokens):
        """Oracle cache model (KiviPackedCacheModel) on one of the 128 batch
        rows of the packed KIVI cache: its 8192-token prefill untimed, then
        one-token decode steps, each handing back the whole fp16 K/V (the same
        elements per row as the GPU figure). The NUQ cache steps are not in
        the sample."""
        import numpy as np
        import torch as _t
        from oracle.caches import KiviPackedCacheModel
        from kv_cache_quantization_row_amd import inputs

        H, D, n0, steps = 8, 64, 8192, 64  # two group flushes among the steps, as on the GPU
        kk, vv = inputs.kivi_kv(1, H, n0 + steps, D, seed=1003)
        k, v = (x.contiguous().view(_t.int16).numpy().view(np.uint16) for x in (kk, vv))
        m = KiviPackedCacheModel(2, 32, 128)
        m.update(k[:, :, :n0], v[:, :, :n0])
        t0 = time.perf_counter()
        elems = 0
        for t in range(steps):
            ko, vo = m.update(k[:, :, n0 + t:n0 + t + 1], v[:, :, n0 + t:n0 + t + 1])
            elems += ko.size + vo.size
        dt = time.perf_counter() - t0
        return {"value": round(2 * elems / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": "packed KIVI cache model, one batch row (8 KV heads x D=64, b=2, group 32, residual "
                          "128): %d one-token decode steps after an untimed 8192-token prefill (%.1f s); the "
                          "NUQ cache steps are not in the sample" % (steps, dt)}


class Copy:
    """Plain device-to-device copy of 4 GiB (torch copy kernel): the practical
    HBM ceiling on this machine and the reference for scaling traffic counters."""

    def __init__(self, torch, args):
        self.torch = torch
        self.n = 1 << 31  # fp16 elements = 4 GiB
        self.name = "copy"

    def setup(self):
        torch = self.torch
        d = torch.device("cuda:0")
        self.src = torch.ones(self.n, dtype=torch.float16, device=d)
        self.dst = torch.empty_like(self.src)
        torch.cuda.synchronize()

    def step(self, tm):
        with tm.span("copy_4GiB"):
            self.dst.copy_(self.src)

    def elems(self):
        return self.n

    def kernel_bytes(self, name):
        return 2 * 2 * self.n

    def config(self):
        return {"workload": "plain device copy, 4 GiB read + 4 GiB written"}

    def cpu_baseline(self, budget_tokens):
        return None


WORKLOADS = {"paged_sym": PagedSym, "kivi": Kivi, "nuq": Nuq, "long_context": LongContext,
             "single_layer": SingleLayer, "attn_decode": AttnDecode, "kivi_packed": KiviPacked, "copy": Copy,
             "caches": Caches}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="paged_sym", choices=sorted(WORKLOADS))
    ap.add_argument("--bits", default="8,6,4")
    ap.add_argument("--kivi-bits", default="2,4")
    ap.add_argument("--prefill-tokens", type=int, default=32768)
    ap.add_argument("--decode-steps", type=int, default=256)
    ap.add_argument("--decode-steps-long", type=int, default=1024)
    ap.add_argument("--lloyd-iters", type=int, default=8, help="Lloyd iterations of the NUQ fits (nuq workload)")
    ap.add_argument("--cpu-tokens", type=int, default=65536)
    ap.add_argument("--attn-group", type=int, default=4, help="query heads per KV head (attn_decode)")
    ap.add_argument("--page-order", default="random", choices=["random", "identity"],
                    help="pool page assignment of the paged workload (random = fragmented pool)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(requested --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch

    from kv_cache_quantization_row_amd import kvq

    kvq.lib()  # fails loudly if the HIP library is missing
    torch.cuda.init()
    wl = WORKLOADS[args.workload](torch, args)
    wl.setup()
    log("warmup %d" % args.warmup)
    warm = Timers(torch)
    for _ in range(args.warmup):
        wl.step(warm)
    torch.cuda.synchronize()
    tm = Timers(torch)
    log("timing %d steps" % args.steps)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for _ in range(args.steps):
        wl.step(tm)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    value = 2.0 * wl.elems() / (ms_per_step / 1e3) / 1e9

    means = tm.mean_ms()
    kernels = {}
    for name, ms in means.items():
        nbytes = wl.kernel_bytes(name)
        gbs = nbytes / (ms / 1e3) / 1e9
        kernels[name] = {"avg_ms": round(ms, 4), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
        if "_x" in name and name.rsplit("_x", 1)[1].isdigit():  # a span of N launches or steps
            kernels[name]["us_per_call"] = round(ms * 1e3 / int(name.rsplit("_x", 1)[1]), 2)
    totals = {n: means[n] * c for n, c in tm.count().items()}
    cands = [n for n in totals if "decode" not in n] or list(totals)
    dom = max(cands, key=lambda n: totals[n])
    roof = wl.roofline(dom, kernels, means) if hasattr(wl, "roofline") else None
    if roof is None:
        roof = {"bound": "hbm", "kernel": dom, "achieved": kernels[dom]["GB/s"], "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": kernels[dom]["frac_hbm"], "traffic": measured_traffic(dom),
                "algorithmic_bytes": int(wl.kernel_bytes(dom))}

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline")
        cpu = wl.cpu_baseline(args.cpu_tokens)
    line = {"metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
            "config": wl.config(), "roofline": roof, "cpu_baseline": cpu, "kernels": kernels,
            "wall_s": round(wall, 3)}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
