"""The single-layer q6 round trip (quantize into pages, dequantize back)
captured once in a HIP graph and replayed: the launch-bound inner loop in the
form a serving loop would run it.

Each replay reads new inputs copied into the captured input buffers; eager
library calls and host synchronisations run between the replays, and every
replay's codes, scales and fp16 output are compared bit for bit with the
oracle's for that replay's input. The symmetric entry points only launch
kernels on the caller's stream (no allocation, no memset, no host wait), so
they record into a graph as they are.
"""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_quantization_row_amd import inputs, kvq
from tests.gpu_util import dev, first_diff, say, u16

pytestmark = pytest.mark.gpu


def test_round_trip_replayed_from_a_hip_graph():
    say("sym round trip in a HIP graph")
    d = dev()
    T, H, D, P, bits = 1024, 4, 256, 16, 6
    pd = kvq.kvq_packed_dim(D, bits)
    lay = kvq.layout(1, T // P, P, H, D, bits)
    xk = torch.zeros((1, T, H, D), dtype=torch.float16, device=d)
    xv = torch.zeros_like(xk)
    pools = [torch.zeros((1, T, H, pd), dtype=torch.uint8, device=d), torch.zeros((1, T, H), dtype=torch.int16, device=d)]
    pools += [torch.zeros_like(pools[0]), torch.zeros_like(pools[1])]
    kc, ks, vc, vs = pools
    slot = torch.arange(T, dtype=torch.int32, device=d)
    bt = torch.arange(T // P, dtype=torch.int32, device=d)[None]
    lens = torch.full((1,), T, dtype=torch.int32, device=d)
    ko = torch.zeros((1, 1, T, H, D), dtype=torch.float16, device=d)
    vo = torch.zeros_like(ko)

    def run():
        kvq.kvq_quant_sym(lay, xk, xv, slot, kc, ks, vc, vs)
        kvq.kvq_dequant_sym(lay, kc, ks, vc, vs, bt, lens, ko, vo)

    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()

    # eager work between the replays: the same calls on other buffers
    ek, es = torch.zeros_like(kc), torch.zeros_like(ks)
    for rep in range(3):
        hk = inputs.sym_layer(T, H, D, seed=3001 + 2 * rep)
        hv = inputs.sym_layer(T, H, D, seed=3002 + 2 * rep)
        xk.copy_(hk[None].to(d))
        xv.copy_(hv[None].to(d))
        kvq.kvq_quant_sym(lay, xv, None, slot, ek, es, None, None)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, x, c, s, out in (("K", hk, kc, ks, ko), ("V", hv, vc, vs, vo)):
            exp_c = np.zeros((T, H, pd), np.uint8)
            exp_s = np.zeros((T, H), np.uint16)
            oracle.sym_quant_paged(u16(x), bits, np.arange(T, dtype=np.int32), exp_c, exp_s)
            assert first_diff(c[0].cpu().numpy(), exp_c) is None, (rep, name, "codes")
            assert first_diff(u16(s[0]), exp_s) is None, (rep, name, "scales")
            exp_o = oracle.sym_dequant_paged(exp_c, exp_s, P, D, bits, np.arange(T // P, dtype=np.int32)[None],
                                             np.array([T], np.int32), T)
            assert first_diff(u16(out[0]), exp_o) is None, (rep, name, "dequant")
        # the eager call between replays wrote its own buffers only
        assert first_diff(ek[0].cpu().numpy(), vc[0].cpu().numpy()) is None, (rep, "eager codes")


def test_nuq_decode_step_replayed_from_a_hip_graph():
    """A NUQ decode step (32 (batch, head) vectors, D = 128, 3 bits, keys
    against frozen tables) through the no-allocation entry point, captured
    once and replayed three times with new tokens copied into the captured
    input buffers; each replay's outputs equal, bit for bit, an eager call of
    the workspace entry point on the same inputs (itself checked against the
    oracle in test_gpu_nuq.py)."""
    say("nuq decode step in a HIP graph")
    d = dev()
    BH, S, D, bits, frac, iters, ns = 32, 1, 128, 3, 0.01, 8, 4
    L = 1 << bits
    start = 4096
    # frozen key tables from a prefill
    kp = inputs.student_t((BH, 512, D), 4, seed=701).to(d)
    vp = inputs.student_t((BH, 512, D), 4, seed=702).to(d)
    kl = torch.zeros((BH, D, L), device=d)
    kt = torch.zeros((BH, D), dtype=torch.int16, device=d)

    def outs():
        cap = max(1, max(kvq.kvq_nuq_outlier_bound(BH, S, D, start, ns, frac, 0, w) for w in (0, 1)))
        return dict(value_levels=torch.zeros((BH, S, L), device=d),
                    k_codes=torch.zeros((BH, S, D * bits // 8), dtype=torch.uint8, device=d),
                    v_codes=torch.zeros((BH, S, D * bits // 8), dtype=torch.uint8, device=d),
                    k_opos=torch.zeros(cap, dtype=torch.int32, device=d),
                    k_oval=torch.zeros(cap, dtype=torch.int16, device=d),
                    v_opos=torch.zeros(cap, dtype=torch.int32, device=d),
                    v_oval=torch.zeros(cap, dtype=torch.int16, device=d),
                    out_counts=torch.zeros(2, dtype=torch.int64, device=d))

    capp = max(1, max(kvq.kvq_nuq_outlier_bound(BH, 512, D, 0, ns, frac, 1, w) for w in (0, 1)))
    z = lambda *sh, dt=torch.float32: torch.zeros(sh, dtype=dt, device=d)
    kvq.kvq_nuq_fit_quant_noalloc(kp, vp, 0, bits, frac, iters, ns, 1, kl, kt, z(BH, 512, L),
                                  z(BH, 512, D * bits // 8, dt=torch.uint8), z(BH, 512, D * bits // 8, dt=torch.uint8),
                                  z(capp, dt=torch.int32), z(capp, dt=torch.int16), z(capp, dt=torch.int32),
                                  z(capp, dt=torch.int16), z(2, dt=torch.int64))
    kd = torch.zeros((BH, S, D), dtype=torch.float16, device=d)
    vd = torch.zeros_like(kd)
    g_out = outs()

    def step():
        o = g_out
        kvq.kvq_nuq_fit_quant_noalloc(kd, vd, start, bits, frac, iters, ns, 0, kl, kt, o["value_levels"],
                                      o["k_codes"], o["v_codes"], o["k_opos"], o["k_oval"], o["v_opos"],
                                      o["v_oval"], o["out_counts"])

    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    ws = torch.zeros((kvq.kvq_nuq_workspace_bytes(BH, S, D, bits, start, ns, frac, 0),), dtype=torch.uint8, device=d)
    for rep in range(3):
        kd.copy_(inputs.student_t((BH, S, D), 4, seed=710 + 2 * rep).to(d))
        vd.copy_(inputs.student_t((BH, S, D), 4, seed=711 + 2 * rep).to(d))
        ref = outs()
        kvq.kvq_nuq_fit_quant(kd, vd, start, bits, frac, iters, ns, 0, kl.clone(), kt.clone(), ref["value_levels"],
                              ref["k_codes"], ref["v_codes"], ref["k_opos"], ref["k_oval"], ref["v_opos"],
                              ref["v_oval"], ref["out_counts"], ws)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        cnt = ref["out_counts"].cpu().numpy()
        assert np.array_equal(cnt, g_out["out_counts"].cpu().numpy()), (rep, cnt)
        for name in ref:
            a, b = ref[name], g_out[name]
            if name in ("k_opos", "k_oval"):
                a, b = a[: cnt[0]], b[: cnt[0]]
            if name in ("v_opos", "v_oval"):
                a, b = a[: cnt[1]], b[: cnt[1]]
            xa = a.cpu().contiguous().view(torch.uint8).numpy()
            xb = b.cpu().contiguous().view(torch.uint8).numpy()
            assert first_diff(xa, xb) is None, (rep, name, first_diff(xa, xb))
