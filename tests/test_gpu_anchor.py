"""The window frame's anchor lag ("GPT-OSS-120B giga-kernel decode", "DI
wiring (NIXL)": both nodes operate at N - 1), on the GPU: the control
bit-exact against the oracle's, and whole steps against the oracle."""
import numpy as np
import pytest
import torch

import paged_fp8_kv_amd as P
import workloads as W
from gpu_harness import assert_close, csr_lists, device_inputs, gpu_step, oracle_step, poison_stale
from oracle import control as OC

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("tables", ["padded", "csr"])
@pytest.mark.parametrize("name", ["cfg2", "cfg3", "cfg5"])
def test_lagged_control_matches_oracle(name, tables, gpu):
    wl = W.make_workload(W.CONFIGS[name])
    c = wl.cfg
    d = device_inputs(wl, gpu)
    if tables == "csr":
        ip, fi, si, lp = (torch.from_numpy(x).to(gpu) for x in csr_lists(wl))
        got = P.pkv_setup_attn_control_csr(ip, fi, si, lp, d["active"], c.block, c.window,
                                           wl.bt_full.shape[1], positions=d["positions"],
                                           anchor_lag=1)
    else:
        got = P.pkv_setup_attn_control(d["seq_lens"], d["active"], d["bt_full"], d["bt_swa"],
                                       c.block, c.window, positions=d["positions"], anchor_lag=1)
    torch.cuda.synchronize()
    ref = OC.attention_control(wl.seq_lens, wl.active, wl.bt_full, wl.bt_swa, c.block, c.window,
                               positions=wl.positions, anchor_lag=1)
    for k in ("pos_full", "pos_swa", "bt_swa_trim", "upd_full", "upd_swa", "pos_abs"):
        assert np.array_equal(got[k].cpu().numpy(), ref[k]), k


def test_lagged_control_at_every_boundary_offset(gpu):
    """One sequence per token index p in [0, 600) at block 16: the lagged
    trimmed table and frame positions equal the oracle's everywhere, so every
    p % 16 around every eviction boundary is covered."""
    Bk, Wn = 16, 128
    p = np.arange(600)
    B = p.size
    width = -(-600 // Bk) + 1
    rng = np.random.default_rng(9)
    bt_full = rng.integers(0, 1 << 20, size=(B, width)).astype(np.int32)
    bt_swa = rng.integers(1 << 20, 1 << 21, size=(B, width)).astype(np.int32)
    lens = (p + 1).astype(np.int32)
    act = np.ones(B, np.uint8)
    t = lambda x: torch.from_numpy(x).to(gpu)
    for lag in (0, 1):
        got = P.pkv_setup_attn_control(t(lens), t(act), t(bt_full), t(bt_swa), Bk, Wn,
                                       anchor_lag=lag)
        torch.cuda.synchronize()
        ref = OC.attention_control(lens, act, bt_full, bt_swa, Bk, Wn, anchor_lag=lag)
        for k in ("pos_swa", "bt_swa_trim", "upd_swa"):
            assert np.array_equal(got[k].cpu().numpy(), ref[k]), (lag, k)


@pytest.mark.parametrize("name", ["cfg2", "cfg5"])
def test_lagged_step_matches_oracle(name, gpu):
    """A whole step with the lagged frame: outputs against the oracle run with
    the same lag, cache bytes bit-exact; with block 32 the window layer is
    also bitwise the unlagged one (frames shift by whole 32-token sub-tiles)."""
    print(f"[anchor lag] {name}", flush=True)
    wl = W.make_workload(W.CONFIGS[name])
    host = W.make_buffers(wl, "cpu")
    poison_stale(host, wl)
    snaps = [h.numpy().copy() for h in host]
    bufs = [h.to(gpu) for h in host]
    base = [h.to(gpu) for h in host]
    outs, _ = gpu_step(wl, bufs, gpu, anchor_lag=1)
    outs0, _ = gpu_step(wl, base, gpu)
    ref, _ = oracle_step(wl, snaps, anchor_lag=1)
    for i in range(wl.cfg.layers):
        assert_close(outs[i], ref[i], f"{name} lag 1 layer {i}")
    for j, b in enumerate(bufs):
        got = b.cpu().numpy()
        assert np.array_equal(got, snaps[j]), f"buffer {j}: {int((got != snaps[j]).sum())} bytes differ"
        assert torch.equal(b, base[j])
    if wl.cfg.block == 32:
        assert torch.equal(outs[0].view(torch.int16), outs0[0].view(torch.int16))
    assert torch.equal(outs[1].view(torch.int16), outs0[1].view(torch.int16))
