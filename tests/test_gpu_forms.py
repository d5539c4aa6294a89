"""The layer entry point's two KV forms and its update indices, on the GPU.

"GPT-OSS-120B giga-kernel decode", "Kernel contract": the kernel accepts the
per-buffer K/V arguments or the stacked cache (exactly one of them), and each
step writes the new token's K/V through two update indices.
"""
import numpy as np
import pytest
import torch

import paged_fp8_kv_amd as P
import workloads as W
from gpu_harness import assert_close, device_inputs, gpu_step, oracle_step, poison_stale

pytestmark = pytest.mark.gpu


def _case(name, gpu):
    wl = W.make_workload(W.CONFIGS[name])
    host = W.make_buffers(wl, "cpu")
    poison_stale(host, wl)
    return wl, host


@pytest.mark.parametrize("name", ["cfg2", "cfg5"])
def test_stacked_form_matches_oracle_and_per_buffer_form(name, gpu):
    """One allocation of all buffers back to back, handed over as the stacked
    form: outputs and every byte equal the oracle's, and bit for bit the
    per-buffer form's."""
    print(f"[stacked] {name}", flush=True)
    wl, host = _case(name, gpu)
    snaps = [h.numpy().copy() for h in host]
    total = host[0].numel()
    stacked = torch.cat(host).to(gpu)
    views = [stacked[j * total:(j + 1) * total] for j in range(len(host))]
    a, _ = gpu_step(wl, views, gpu, stacked=stacked)
    per = [h.to(gpu) for h in host]
    b, _ = gpu_step(wl, per, gpu)
    ref, _ = oracle_step(wl, snaps)
    for i in range(wl.cfg.layers):
        assert_close(a[i], ref[i], f"{name} stacked layer {i}")
        assert torch.equal(a[i].view(torch.int16), b[i].view(torch.int16)), i
    for j in range(len(host)):
        got = views[j].cpu().numpy()
        assert np.array_equal(got, snaps[j]), f"buffer {j}: {int((got != snaps[j]).sum())} bytes differ"
        assert torch.equal(views[j], per[j])


def test_stacked_form_with_more_buffers_than_layers_use(gpu):
    """Stacked form with three buffers: the pair of layers reads and writes
    only the first; the others keep their bytes."""
    wl, host = _case("cfg2", gpu)
    total = host[0].numel()
    extra = [torch.full_like(host[0], 0x3C), torch.full_like(host[0], 0x44)]
    stacked = torch.cat([host[0]] + extra).to(gpu)
    views = [stacked[j * total:(j + 1) * total] for j in range(3)]
    per = [host[0].to(gpu)]
    a, _ = gpu_step(wl, views[:1], gpu, stacked=stacked)
    b, _ = gpu_step(wl, per, gpu)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert torch.equal(views[0], per[0])
    assert torch.equal(views[1].cpu(), extra[0]) and torch.equal(views[2].cpu(), extra[1])


def _layer_vs_separate(name, gpu, edit):
    """Run layers 0 and 1 of a pair through pkv_decode_layer with the update
    indices edited by `edit(ctl)`, and the same layers as a separate update
    (with the edited indices) plus attention.  Returns both results."""
    wl, host = _case(name, gpu)
    c = wl.cfg
    d = device_inputs(wl, gpu)
    ctl = P.pkv_setup_attn_control(d["seq_lens"], d["active"], d["bt_full"], d["bt_swa"],
                                   c.block, c.window, positions=d["positions"])
    edit(ctl)
    sm = 1.0 / np.sqrt(c.head_dim)
    tw = ctl["bt_swa_trim"].shape[1]
    ws = [P.new_workspace(c.batch, c.hq, c.hkv, c.head_dim, c.block, tw, c.window, gpu),
          P.new_workspace(c.batch, c.hq, c.hkv, c.head_dim, c.block, wl.bt_full.shape[1], 0, gpu)]
    fused = host[0].to(gpu)
    step = P.make_step([fused], ctl, d["bt_full"], c.batch, c.hq, c.hkv, c.head_dim, c.block,
                       c.window, wl.nb)
    outs_f = []
    for i in range(2):
        out = torch.empty_like(d["q"][i])
        P.pkv_decode_layer(step, i, d["q"][i], d["k_new"][i], d["v_new"][i], wl.k_scale[i],
                           wl.v_scale[i], sm, out, ws[i])
        outs_f.append(out)
    sep = host[0].to(gpu)
    outs_s = []
    for i in range(2):
        swa = i == 0
        P.pkv_kv_cache_update(sep, d["k_new"][i], d["v_new"][i],
                              ctl["upd_swa"] if swa else ctl["upd_full"], c.block, wl.nb,
                              wl.k_scale[i], wl.v_scale[i])
        if swa:
            o = P.pkv_paged_decode_attn(d["q"][i], sep, ctl["bt_swa_trim"], ctl["pos_swa"],
                                        c.block, wl.nb, c.window, wl.k_scale[i], wl.v_scale[i],
                                        sm, c.hkv)
        else:
            o = P.pkv_paged_decode_attn(d["q"][i], sep, d["bt_full"], ctl["pos_full"], c.block,
                                        wl.nb, 0, wl.k_scale[i], wl.v_scale[i], sm, c.hkv)
        outs_s.append(o)
    torch.cuda.synchronize()
    return wl, host[0], ctl, fused, outs_f, sep, outs_s


def test_minus_one_update_index_skips_the_write(gpu):
    """Rows whose update index is -1 are not written and attend the cache as
    it is: bytes and outputs equal the separate update (which skips them too)
    followed by attention, bit for bit."""
    rows = torch.tensor([1, 4, 6])

    def edit(ctl):
        ctl["upd_swa"][rows[:2].to(ctl["upd_swa"].device)] = -1
        ctl["upd_full"][rows[1:].to(ctl["upd_full"].device)] = -1

    wl, before, ctl, fused, of, sep, os_ = _layer_vs_separate("cfg2", gpu, edit)
    assert torch.equal(fused, sep)
    for a, b in zip(of, os_):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # the skipped rows left their slots as they were (poisoned: NaN output)
    for r in rows.tolist():
        assert torch.isnan(of[0][r].float()).all() == (r in (1, 4))
        assert torch.isnan(of[1][r].float()).all() == (r in (4, 6))


def test_foreign_update_index_gives_nan_and_no_write(gpu):
    """An update index that is neither -1 nor the table's slot of the frame
    position: that row is NaN and nothing is written for it; every other row
    and byte is as in an unedited step."""
    moved = {}

    def edit(ctl):
        # point row 3's full-layer write at another valid slot of its own block
        u = int(ctl["upd_full"][3])
        moved["orig"] = u
        ctl["upd_full"][3] = u - 1 if u % 32 else u + 1

    wl, before, ctl, fused, of, _, _ = _layer_vs_separate("cfg2", gpu, edit)
    assert torch.isnan(of[1][3].float()).all()
    # reference: the same step with row 3's full write skipped (-1)
    def edit_ref(ctl):
        ctl["upd_full"][3] = -1
    _, _, _, fused_ref, of_ref, _, _ = _layer_vs_separate("cfg2", gpu, edit_ref)
    assert torch.equal(fused, fused_ref)
    keep = [r for r in range(wl.cfg.batch) if r != 3]
    assert torch.equal(of[1][keep].view(torch.int16), of_ref[1][keep].view(torch.int16))
    assert torch.equal(of[0].view(torch.int16), of_ref[0].view(torch.int16))
