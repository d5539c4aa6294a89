"""Rotary embedding on the GPU path: the queries turned before the scores,
the new K turned in fp32 before its FP8 code is taken (bit-exact against the
oracle, including inputs where a fused multiply-add would flip the code), on
the fused layer entry point and on the separate update + attention calls."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_harness import ROPE_GUARDS, assert_close, gpu_step, oracle_step, poison_stale
from oracle import control as OC
from oracle import layout as OL
from paged_build import rope_fma_trap

pytestmark = pytest.mark.gpu


def _case(name, gpu):
    wl = W.make_workload(W.CONFIGS[name])
    host = W.make_buffers(wl, "cpu")
    poison_stale(host, wl)
    snaps = [h.numpy().copy() for h in host]
    return wl, [h.to(gpu) for h in host], snaps


def _check(wl, outs, bufs, ref, snaps, what):
    for i in range(wl.cfg.layers):
        assert_close(outs[i], ref[i], f"{what} layer {i}", **ROPE_GUARDS)
    for j, b in enumerate(bufs):
        got = b.cpu().numpy()
        assert np.array_equal(got, snaps[j]), f"{what} buffer {j}: {int((got != snaps[j]).sum())} bytes differ"


@pytest.mark.parametrize("layer_api", [True, False])
@pytest.mark.parametrize("name", ["cfg1", "cfg2", "cfg5"])
def test_step_with_rope_matches_oracle(name, layer_api, gpu):
    print(f"[rope] {name} layer_api={layer_api}", flush=True)
    wl, bufs, snaps = _case(name, gpu)
    rope = W.rope_tables(wl)
    outs, _ = gpu_step(wl, bufs, gpu, use_layer_api=layer_api, rope=rope)
    ref, _ = oracle_step(wl, snaps, rope=rope)
    _check(wl, outs, bufs, ref, snaps, name)


@pytest.mark.parametrize("layer_api", [True, False])
def test_rope_k_code_is_taken_from_unfused_fp32(layer_api, gpu):
    """Rows 0 and 1 carry the four ties of rope_fma_trap, scaled by the K scale
    1/8 (a power of two, so every product, tie and quotient scales exactly):
    the unfused fp32 evaluation codes them 0x38, a fused multiply-add 0x39."""
    print(f"[rope] fma trap layer_api={layer_api}", flush=True)
    wl, bufs, snaps = _case("cfg2", gpu)
    cos, sin = W.rope_tables(wl)
    x, c, s, traps = rope_fma_trap()
    cos[:2], sin[:2] = c, s
    assert all(k == 0.125 for k in wl.k_scale)
    xs = x * np.float32(0.125)
    wl.k_new[:, :2] = torch.from_numpy(xs).to(torch.bfloat16)[None, :, None, :]
    assert torch.equal(wl.k_new[0, :2, 0].float(), torch.from_numpy(xs))  # bf16-exact inputs
    outs, _ = gpu_step(wl, bufs, gpu, use_layer_api=layer_api, rope=(cos, sin))
    ref, _ = oracle_step(wl, snaps, rope=(cos, sin))
    _check(wl, outs, bufs, ref, snaps, "trap")
    # the oracle's codes at the traps (the GPU bytes equal them) are the unfused ones
    ctl = OC.attention_control(wl.seq_lens, wl.active, wl.bt_full, wl.bt_swa, wl.cfg.block,
                               wl.cfg.window)
    half = wl.half_bytes
    for layer, key in ((0, "upd_swa"), (1, "upd_full")):
        for b, d in traps:
            blk, tok = divmod(int(ctl[key][b]), wl.cfg.block)
            for h in range(wl.cfg.hkv):
                off = OL.k_offset(blk, h, tok, d, wl.cfg.hkv, wl.cfg.block, wl.cfg.head_dim, True)
                assert snaps[0][off] == 0x38, (layer, b, d, h, hex(snaps[0][off]))


def test_rope_changes_the_result(gpu):
    """Guard against a silently ignored rotation: turned and unturned steps differ."""
    wl, bufs, _ = _case("cfg2", gpu)
    bufs2 = [b.clone() for b in bufs]
    a, _ = gpu_step(wl, bufs, gpu, rope=W.rope_tables(wl))
    b, _ = gpu_step(wl, bufs2, gpu)
    assert not torch.equal(a[1], b[1])
    assert not all(torch.equal(x, y) for x, y in zip(bufs, bufs2))
