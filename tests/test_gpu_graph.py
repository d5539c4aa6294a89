"""A whole decode step -- the control setup and every layer -- captured as a
HIP graph on a side stream and replayed.  Every library call enqueues on the
caller's stream and records no memset node (counters are cleared by the
kernels themselves, or by a fill kernel in the no-allocation entry point), so
each replay must reproduce the eager step bit for bit.  Before every replay
the outputs are cleared and an eager step with other queries runs on the same
cache, workspaces and control tensors; outputs and cache bytes are compared
after each of three replays."""
import numpy as np
import pytest
import torch

import paged_fp8_kv_amd as P
import workloads as W
from gpu_harness import csr_lists, device_inputs

pytestmark = pytest.mark.gpu


def _step_fn(wl, bufs, gpu, tables, noalloc):
    c = wl.cfg
    d = device_inputs(wl, gpu)
    if tables == "csr":
        csr = tuple(torch.from_numpy(x).to(gpu) for x in csr_lists(wl))
        ctl = P.pkv_setup_attn_control_csr(*csr, d["active"], c.block, c.window,
                                           wl.bt_full.shape[1], positions=d["positions"])
        bt_full = ctl["bt_full"]

        def setup():
            P.pkv_setup_attn_control_csr(*csr, d["active"], c.block, c.window,
                                         wl.bt_full.shape[1], positions=d["positions"], out=ctl)
    else:
        ctl = P.pkv_setup_attn_control(d["seq_lens"], d["active"], d["bt_full"], d["bt_swa"],
                                       c.block, c.window, positions=d["positions"])
        bt_full = d["bt_full"]

        def setup():
            P.pkv_setup_attn_control(d["seq_lens"], d["active"], d["bt_full"], d["bt_swa"],
                                     c.block, c.window, positions=d["positions"], out=ctl)
    step = P.make_step(bufs, ctl, bt_full, c.batch, c.hq, c.hkv, c.head_dim, c.block, c.window,
                       wl.nb)
    tw = ctl["bt_swa_trim"].shape[1]
    ws = [P.new_workspace(c.batch, c.hq, c.hkv, c.head_dim, c.block, tw, c.window, gpu),
          P.new_workspace(c.batch, c.hq, c.hkv, c.head_dim, c.block, wl.bt_full.shape[1], 0, gpu)]
    sm = 1.0 / np.sqrt(c.head_dim)

    def run(qq, oo):
        setup()
        for i in range(c.layers):
            if noalloc:
                P.pkv_decode_layer_noalloc(step, i, qq[i], d["k_new"][i], d["v_new"][i],
                                           wl.k_scale[i], wl.v_scale[i], sm, oo[i])
            else:
                P.pkv_decode_layer(step, i, qq[i], d["k_new"][i], d["v_new"][i], wl.k_scale[i],
                                   wl.v_scale[i], sm, oo[i], ws[i % 2])

    return run


@pytest.mark.parametrize("name,tables,noalloc", [("cfg2", "padded", False),
                                                 ("cfg5", "csr", False),
                                                 ("cfg5", "padded", True)],
                         ids=["cfg2-padded", "cfg5-pagelists", "cfg5-noalloc"])
def test_graph_replays_equal_the_eager_step(name, tables, noalloc, gpu):
    print(f"[graph] {name} {tables} noalloc={noalloc}", flush=True)
    wl = W.make_workload(W.CONFIGS[name])
    c = wl.cfg
    bufs = [h.to(gpu) for h in W.make_buffers(wl, "cpu")]
    q = wl.q.to(gpu)
    q_other = torch.randn(q.shape, generator=torch.Generator().manual_seed(99)).to(
        torch.bfloat16).to(gpu)
    outs = [torch.empty_like(q[i]) for i in range(c.layers)]
    other = [torch.empty_like(q[i]) for i in range(c.layers)]
    run = _step_fn(wl, bufs, gpu, tables, noalloc)

    run(q, outs)  # writes the step's new tokens; later steps rewrite the same bytes
    run(q, outs)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    ref_bufs = [b.clone() for b in bufs]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run(q, outs)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(q, outs)
    for r in range(3):
        for o in outs:
            o.zero_()
        run(q_other, other)
        g.replay()
        torch.cuda.synchronize()
        for i in range(c.layers):
            assert torch.equal(outs[i].view(torch.int16), ref[i].view(torch.int16)), (r, i)
            assert not torch.equal(other[i].view(torch.int16), ref[i].view(torch.int16)), (r, i)
        for j, b in enumerate(bufs):
            assert torch.equal(b, ref_bufs[j]), (r, j)
