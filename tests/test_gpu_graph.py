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
