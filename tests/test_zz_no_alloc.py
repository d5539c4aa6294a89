"""pkv_decode_layer_noalloc -- the layer entry point that allocates nothing
(its split-KV workspace is the library's own device array) -- against
pkv_decode_layer with a caller-allocated workspace, through the C ABI: two
calls in a row, the second with a smaller input, then the first input again
(the array keeps the last call's contents; what must start at zero is
cleared by every call).  Outputs and cache bytes must be identical bit for
bit, and the outputs within the tolerances of the oracle."""
import dataclasses

import numpy as np
import pytest
import torch

import paged_fp8_kv_amd as P
import workloads as W
from gpu_harness import assert_close, device_inputs, oracle_step, poison_stale

pytestmark = pytest.mark.gpu


def _layers(wl, buf, gpu, noalloc):
    c = wl.cfg
    d = device_inputs(wl, gpu)
    ctl = P.pkv_setup_attn_control(d["seq_lens"], d["active"], d["bt_full"], d["bt_swa"],
                                   c.block, c.window, positions=d["positions"])
    step = P.make_step([buf], ctl, d["bt_full"], c.batch, c.hq, c.hkv, c.head_dim, c.block,
                       c.window, wl.nb)
    sm = 1.0 / np.sqrt(c.head_dim)
    tw = ctl["bt_swa_trim"].shape[1]
    outs = []
    for i in range(c.layers):
        out = torch.empty_like(d["q"][i])
        if noalloc:
            P.pkv_decode_layer_noalloc(step, i, d["q"][i], d["k_new"][i], d["v_new"][i],
                                       wl.k_scale[i], wl.v_scale[i], sm, out)
        else:
            ws = P.new_workspace(c.batch, c.hq, c.hkv, c.head_dim, c.block,
                                 tw if i % 2 == 0 else wl.bt_full.shape[1],
                                 c.window if i % 2 == 0 else 0, gpu)
            P.pkv_decode_layer(step, i, d["q"][i], d["k_new"][i], d["v_new"][i], wl.k_scale[i],
                               wl.v_scale[i], sm, out, ws)
        outs.append(out)
    torch.cuda.synchronize()
    return outs


def _compare(wl, gpu, what):
    print(f"[no alloc] {what}: batch {wl.cfg.batch}", flush=True)
    host = W.make_buffers(wl, "cpu")
    poison_stale(host, wl)
    snap = host[0].numpy().copy()
    a_buf, b_buf = host[0].to(gpu), host[0].to(gpu)
    a = _layers(wl, a_buf, gpu, noalloc=True)
    b = _layers(wl, b_buf, gpu, noalloc=False)
    for i, (x, y) in enumerate(zip(a, b)):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16)), f"{what} layer {i}"
    assert torch.equal(a_buf, b_buf), what
    ref, _ = oracle_step(wl, [snap])
    for i in range(wl.cfg.layers):
        assert_close(a[i], ref[i], f"{what} no-alloc layer {i}")
    assert np.array_equal(a_buf.cpu().numpy(), snap), what
    return a


def test_noalloc_layer_equals_layer_with_workspace(gpu):
    # a pair of layers, batch 8, contexts 1024..4096: long items are cut
    # between workgroups, so partials and arrival counters are used
    wl1 = W.make_workload(W.CONFIGS["cfg2"])
    first = _compare(wl1, gpu, "call 1")
    # a smaller input next (3 sequences, 200..700 tokens)
    small = dataclasses.replace(W.CONFIGS["cfg2"], name="cfg2_small_b3", batch=3,
                                ctx=("uniform", 200, 700), seed=21)
    _compare(W.make_workload(small), gpu, "call 2 (smaller)")
    # the first input again: the same bits as its first call
    again = _compare(wl1, gpu, "call 3 (first input again)")
    for x, y in zip(first, again):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
