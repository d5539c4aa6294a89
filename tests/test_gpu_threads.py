"""The library is reentrant: two host threads, each driving its own decode
steps on its own HIP stream (own cache, control, workspaces and outputs),
call into it at the same time.  Every output of every step must equal, bit
for bit, what the same step gives when run alone."""
import threading

import numpy as np
import pytest
import torch

import paged_fp8_kv_amd as P
import workloads as W
from gpu_harness import device_inputs

pytestmark = pytest.mark.gpu


def _prepare(name, gpu):
    wl = W.make_workload(W.CONFIGS[name])
    c = wl.cfg
    d = device_inputs(wl, gpu)
    bufs = [h.to(gpu) for h in W.make_buffers(wl, "cpu")]
    ctl = P.pkv_setup_attn_control(d["seq_lens"], d["active"], d["bt_full"], d["bt_swa"],
                                   c.block, c.window, positions=d["positions"])
    step = P.make_step(bufs, ctl, d["bt_full"], c.batch, c.hq, c.hkv, c.head_dim, c.block,
                       c.window, wl.nb)
    tw = ctl["bt_swa_trim"].shape[1]
    ws = [P.new_workspace(c.batch, c.hq, c.hkv, c.head_dim, c.block, tw, c.window, gpu),
          P.new_workspace(c.batch, c.hq, c.hkv, c.head_dim, c.block, wl.bt_full.shape[1], 0, gpu)]
    outs = [torch.empty_like(d["q"][i]) for i in range(c.layers)]
    sm = 1.0 / np.sqrt(c.head_dim)

    def run(stream):
        P.pkv_setup_attn_control(d["seq_lens"], d["active"], d["bt_full"], d["bt_swa"], c.block,
                                 c.window, positions=d["positions"], out=ctl, stream=stream)
        for i in range(c.layers):
            P.pkv_decode_layer(step, i, d["q"][i], d["k_new"][i], d["v_new"][i], wl.k_scale[i],
                               wl.v_scale[i], sm, outs[i], ws[i % 2], stream=stream)

    return run, outs


def test_two_threads_on_two_streams(gpu):
    jobs = [_prepare("cfg2", gpu), _prepare("cfg5", gpu)]
    for run, _ in jobs:
        run(None)  # writes the new tokens; later steps rewrite the same bytes
    torch.cuda.synchronize()
    refs = [[o.clone() for o in outs] for _, outs in jobs]

    errors = []
    mismatches = []

    def worker(k):
        try:
            run, outs = jobs[k]
            s = torch.cuda.Stream()
            for r in range(20):
                with torch.cuda.stream(s):
                    for o in outs:
                        o.zero_()
                    run(s)
                s.synchronize()
                for i, o in enumerate(outs):
                    if not torch.equal(o.view(torch.int16), refs[k][i].view(torch.int16)):
                        mismatches.append((k, r, i))
        except Exception as e:  # reported on the main thread
            errors.append((k, repr(e)))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    assert not mismatches, mismatches[:5]

