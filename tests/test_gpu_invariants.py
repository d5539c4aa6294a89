"""Invariants of the attention that hold bit for bit on the GPU, from the
definition of the method ("GPT-OSS-120B giga-kernel decode", "Kernel
contract": each query head attends its group's KV head; a per-tensor FP8
scale multiplies every dequantized value):
  * query heads of one group with equal queries get bitwise equal rows;
  * doubling v_scale doubles every output exactly (a power of two scales the
    fp32 weighted sum and the bf16 rounding alike);
  * only the product k_scale * sm_scale enters the scores: halving one and
    doubling the other changes no bit.
Each is checked on the window and the full layer of the two-layer batch-8
workload (contexts 1024..4096, block 32) and of the ragged batch-256 one
(contexts 100..600, block 16, 25% inactive rows), through the stand-alone
attention call."""
import numpy as np
import pytest
import torch

import paged_fp8_kv_amd as P
import workloads as W
from gpu_harness import device_inputs

pytestmark = pytest.mark.gpu


def _attend(wl, buf, ctl, d, q, window, k_scale, v_scale, sm):
    c = wl.cfg
    if window:
        return P.pkv_paged_decode_attn(q, buf, ctl["bt_swa_trim"], ctl["pos_swa"], c.block, wl.nb,
                                       window, k_scale, v_scale, sm, c.hkv)
    return P.pkv_paged_decode_attn(q, buf, d["bt_full"], ctl["pos_full"], c.block, wl.nb, 0,
                                   k_scale, v_scale, sm, c.hkv)


def _setup(name, gpu):
    wl = W.make_workload(W.CONFIGS[name])
    c = wl.cfg
    d = device_inputs(wl, gpu)
    buf = W.make_buffers(wl, "cpu")[0].to(gpu)
    ctl = P.pkv_setup_attn_control(d["seq_lens"], d["active"], d["bt_full"], d["bt_swa"],
                                   c.block, c.window, positions=d["positions"])
    return wl, buf, ctl, d


@pytest.mark.parametrize("window", [128, 0], ids=["window", "full"])
@pytest.mark.parametrize("name", ["cfg2", "cfg5"])
def test_equal_queries_in_a_group_give_equal_rows(name, window, gpu):
    wl, buf, ctl, d = _setup(name, gpu)
    c = wl.cfg
    G = c.hq // c.hkv
    q = d["q"][1].clone()
    qg = q.view(c.batch, c.hkv, G, c.head_dim)
    qg[:, :, 1:] = qg[:, :, :1]
    out = _attend(wl, buf, ctl, d, q, window, wl.k_scale[1], wl.v_scale[1], 0.125)
    torch.cuda.synchronize()
    o = out.view(c.batch, c.hkv, G, c.head_dim).view(torch.int16)
    assert torch.equal(o, o[:, :, :1].expand_as(o))


@pytest.mark.parametrize("window", [128, 0], ids=["window", "full"])
@pytest.mark.parametrize("name", ["cfg2", "cfg5"])
def test_doubling_v_scale_doubles_every_output(name, window, gpu):
    wl, buf, ctl, d = _setup(name, gpu)
    q = d["q"][0]
    ks, vs = wl.k_scale[0], wl.v_scale[0]
    a = _attend(wl, buf, ctl, d, q, window, ks, vs, 0.125)
    b = _attend(wl, buf, ctl, d, q, window, ks, 2.0 * vs, 0.125)
    torch.cuda.synchronize()
    af = a.float()
    assert torch.isfinite(af).all() and af.abs().max() > 0
    assert torch.equal(b.float(), 2.0 * af)


@pytest.mark.parametrize("window", [128, 0], ids=["window", "full"])
@pytest.mark.parametrize("name", ["cfg2", "cfg5"])
def test_scores_depend_on_the_product_of_k_scale_and_sm_scale(name, window, gpu):
    wl, buf, ctl, d = _setup(name, gpu)
    q = d["q"][0]
    ks, vs = wl.k_scale[0], wl.v_scale[0]
    a = _attend(wl, buf, ctl, d, q, window, ks, vs, 0.125)
    b = _attend(wl, buf, ctl, d, q, window, 2.0 * ks, vs, 0.0625)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
