"""kvq_nuq_fit_quant_noalloc (workspace in the library's static device
array) against kvq_nuq_fit_quant (caller's workspace): every output
bit-for-bit on two calls in a row, the second smaller, through the C ABI;
plus a many-token call (where the caller-workspace entry forks the value fit
onto a second stream and the no-allocation entry stays on one stream)."""
import numpy as np
import pytest
import torch

from kv_cache_quantization_row_amd import inputs, kvq
from tests.gpu_util import dev, first_diff, say, u16

pytestmark = pytest.mark.gpu


def _outputs(BH, S, D, bits, start, n_sink, frac, fit, d, key_levels=None, key_thresh=None):
    L = 1 << bits
    cap = max(1, max(kvq.kvq_nuq_outlier_bound(BH, S, D, start, n_sink, frac, fit, w) for w in (0, 1)))
    o = dict(key_levels=torch.full((BH, D, L), 3.0, device=d) if key_levels is None else key_levels.clone(),
             key_thresh=torch.full((BH, D), 5, dtype=torch.int16, device=d) if key_thresh is None
             else key_thresh.clone(),
             value_levels=torch.full((BH, S, L), 9.0, device=d),
             k_codes=torch.full((BH, S, D * bits // 8), 0xA5, dtype=torch.uint8, device=d),
             v_codes=torch.full((BH, S, D * bits // 8), 0x5A, dtype=torch.uint8, device=d),
             k_opos=torch.full((cap,), -1, dtype=torch.int32, device=d),
             k_oval=torch.zeros(cap, dtype=torch.int16, device=d),
             v_opos=torch.full((cap,), -1, dtype=torch.int32, device=d),
             v_oval=torch.zeros(cap, dtype=torch.int16, device=d),
             out_counts=torch.full((2,), -1, dtype=torch.int64, device=d),
             k_recon=torch.zeros((BH, S, D), dtype=torch.float16, device=d),
             v_recon=torch.ones((BH, S, D), dtype=torch.float16, device=d))
    return o


def _same(a, b, what):
    ca, cb = a["out_counts"].cpu().numpy(), b["out_counts"].cpu().numpy()
    assert np.array_equal(ca, cb), (what, ca, cb)
    for name in a:
        x, y = a[name], b[name]
        if name in ("k_opos", "k_oval"):
            x, y = x[: ca[0]], y[: ca[0]]
        if name in ("v_opos", "v_oval"):
            x, y = x[: ca[1]], y[: ca[1]]
        xa = x.cpu().contiguous().view(torch.uint8).numpy()
        ya = y.cpu().contiguous().view(torch.uint8).numpy()
        assert first_diff(xa, ya) is None, (what, name, first_diff(xa, ya))


def _call_both(k, v, start, bits, frac, iters, n_sink, fit, d, kl=None, kt=None):
    BH, S, D = k.shape
    ref = _outputs(BH, S, D, bits, start, n_sink, frac, fit, d, kl, kt)
    got = _outputs(BH, S, D, bits, start, n_sink, frac, fit, d, kl, kt)
    ws = torch.full((kvq.kvq_nuq_workspace_bytes(BH, S, D, bits, start, n_sink, frac, fit),), 0xEE,
                    dtype=torch.uint8, device=d)
    kvq.kvq_nuq_fit_quant(k, v, start, bits, frac, iters, n_sink, fit, ref["key_levels"], ref["key_thresh"],
                          ref["value_levels"], ref["k_codes"], ref["v_codes"], ref["k_opos"], ref["k_oval"],
                          ref["v_opos"], ref["v_oval"], ref["out_counts"], ws, ref["k_recon"], ref["v_recon"])
    kvq.kvq_nuq_fit_quant_noalloc(k, v, start, bits, frac, iters, n_sink, fit, got["key_levels"], got["key_thresh"],
                                  got["value_levels"], got["k_codes"], got["v_codes"], got["k_opos"], got["k_oval"],
                                  got["v_opos"], got["v_oval"], got["out_counts"], got["k_recon"], got["v_recon"])
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_matches_the_workspace_entry_on_consecutive_calls():
    d = dev()
    bits, frac, iters, ns = 3, 0.01, 8, 4
    # call 1: a prefill of 32 (batch, head) vectors x 1000 tokens x D = 128
    # (more than 4096 tokens: the workspace entry forks the value fit)
    say("noalloc prefill 32x1000x128")
    k = inputs.student_t((32, 1000, 128), 4, seed=501).to(d)
    v = inputs.student_t((32, 1000, 128), 4, seed=502).to(d)
    ref, got = _call_both(k, v, 0, bits, frac, iters, ns, 1, d)
    _same(ref, got, "prefill")
    # call 2, smaller: one decode token against the frozen key tables (the
    # array keeps the previous call's contents; counters must be cleared)
    say("noalloc decode 32x1x128")
    kd = inputs.student_t((32, 1, 128), 4, seed=503).to(d)
    vd = inputs.student_t((32, 1, 128), 4, seed=504).to(d)
    ref2, got2 = _call_both(kd, vd, 1000, bits, frac, iters, ns, 0, d, ref["key_levels"], ref["key_thresh"])
    _same(ref2, got2, "decode")
    # call 3, smaller again: a short prefill with sinks, other widths
    say("noalloc short prefill 3x70x64")
    k3 = inputs.student_t((3, 70, 64), 4, seed=505).to(d)
    v3 = inputs.student_t((3, 70, 64), 4, seed=506).to(d)
    ref3, got3 = _call_both(k3, v3, 0, 2, 0.05, 4, ns, 1, d)
    _same(ref3, got3, "short prefill")


def test_noalloc_refuses_a_call_above_its_workspace():
    d = dev()
    BH, S, D = 64, 2000, 128  # half of every token's values may be outliers: > 32 MiB of value staging
    assert kvq.kvq_nuq_workspace_bytes(BH, S, D, 3, 5, 4, 0.5, 0) > kvq.NUQ_NOALLOC_WORKSPACE_BYTES
    k = torch.zeros((BH, S, D), dtype=torch.float16, device=d)
    o = _outputs(BH, S, D, 3, 5, 4, 0.5, 0, d)
    with pytest.raises(kvq.KvqError) as e:
        kvq.kvq_nuq_fit_quant_noalloc(k, k, 5, 3, 0.5, 8, 4, 0, o["key_levels"], o["key_thresh"],
                                      o["value_levels"], o["k_codes"], o["v_codes"], o["k_opos"], o["k_oval"],
                                      o["v_opos"], o["v_oval"], o["out_counts"])
    assert e.value.code == kvq.KVQ_ERR_CAPACITY
