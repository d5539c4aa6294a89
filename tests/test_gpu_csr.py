"""Control from compressed page lists equals the control from padded tables,
bit for bit, and the padded table it writes drives the same attention."""
import numpy as np
import pytest
import torch

import paged_fp8_kv_amd as P
import workloads as W
from gpu_harness import assert_close, device_inputs, gpu_step, oracle_step, poison_stale
from oracle import control as OC

pytestmark = pytest.mark.gpu


def _csr(wl):
    """Compress the workload's padded tables (plain loops)."""
    Bk = wl.cfg.block
    indptr, full, swa, last = [0], [], [], []
    for b in range(wl.cfg.batch):
        n = -(-int(wl.seq_lens[b]) // Bk)
        full += [int(x) for x in wl.bt_full[b, :n]]
        swa += [int(x) for x in wl.bt_swa[b, :n]]
        indptr.append(indptr[-1] + n)
        last.append(int(wl.seq_lens[b]) - (n - 1) * Bk if n else 0)
    a = lambda x: np.asarray(x, dtype=np.int32)
    return a(indptr), a(full), a(swa), a(last)


@pytest.mark.parametrize("name", ["cfg2", "cfg4", "cfg5"])
def test_csr_control_equals_padded(name, gpu):
    cfg = W.CONFIGS[name]
    wl = W.make_workload(cfg, hbm_bytes=torch.cuda.mem_get_info(gpu)[1])
    print(f"[csr] {name}", flush=True)
    win = cfg.window if "swa" in cfg.kinds else 0
    d = device_inputs(wl, gpu)
    ref = P.pkv_setup_attn_control(d["seq_lens"], d["active"], d["bt_full"], d["bt_swa"],
                                   cfg.block, win, positions=d["positions"])
    ip, fi, si, lp = _csr(wl)
    t = lambda x: torch.from_numpy(x).to(gpu)
    width = wl.bt_full.shape[1]
    got = P.pkv_setup_attn_control_csr(t(ip), t(fi), t(si), t(lp), d["active"], cfg.block, win,
                                       width, positions=d["positions"])
    torch.cuda.synchronize()
    keys = ["pos_full", "upd_full", "pos_abs"] + (["pos_swa", "upd_swa", "bt_swa_trim"] if win else [])
    for k in keys:
        assert torch.equal(got[k], ref[k]), k
    sl, bf, _ = OC.csr_to_tables(ip, fi, si, lp, cfg.block, width)
    assert np.array_equal(got["seq_lens"].cpu().numpy(), sl)
    assert np.array_equal(got["bt_full"].cpu().numpy(), bf)
    assert np.array_equal(bf, wl.bt_full)


def test_csr_tables_drive_identical_attention(gpu):
    cfg = W.CONFIGS["cfg2"]
    wl = W.make_workload(cfg)
    buf = W.make_buffers(wl, "cpu")[0].to(gpu)
    d = device_inputs(wl, gpu)
    ip, fi, si, lp = _csr(wl)
    t = lambda x: torch.from_numpy(x).to(gpu)
    c = P.pkv_setup_attn_control_csr(t(ip), t(fi), t(si), t(lp), d["active"], cfg.block,
                                     cfg.window, wl.bt_full.shape[1])
    r = P.pkv_setup_attn_control(d["seq_lens"], d["active"], d["bt_full"], d["bt_swa"],
                                 cfg.block, cfg.window)
    outs = []
    for ctl, table in ((c, c["bt_full"]), (r, d["bt_full"])):
        full = P.pkv_paged_decode_attn(d["q"][1], buf, table, ctl["pos_full"], cfg.block, wl.nb, 0,
                                       0.125, 0.0625, 0.125, cfg.hkv)
        swa = P.pkv_paged_decode_attn(d["q"][0], buf, ctl["bt_swa_trim"], ctl["pos_swa"], cfg.block,
                                      wl.nb, cfg.window, 0.125, 0.0625, 0.125, cfg.hkv)
        outs.append((full, swa))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("name", ["cfg2", "cfg4", "cfg5"])
def test_csr_control_matches_oracle(name, gpu):
    """The control built from page lists against the oracle's control of the
    oracle's own conversion of the same lists (not against the padded HIP
    setup)."""
    cfg = W.CONFIGS[name]
    wl = W.make_workload(cfg, hbm_bytes=torch.cuda.mem_get_info(gpu)[1])
    win = cfg.window if "swa" in cfg.kinds else 0
    ip, fi, si, lp = _csr(wl)
    width = wl.bt_full.shape[1]
    t = lambda x: torch.from_numpy(x).to(gpu)
    got = P.pkv_setup_attn_control_csr(t(ip), t(fi), t(si), t(lp), t(wl.active), cfg.block, win,
                                       width, positions=t(wl.positions.astype(np.int64)))
    torch.cuda.synchronize()
    sl, bf, bs = OC.csr_to_tables(ip, fi, si if win else None, lp, cfg.block, width)
    ref = OC.attention_control(sl, wl.active, bf, bs, cfg.block, max(win, 1),
                               positions=wl.positions)
    keys = ["pos_full", "upd_full", "pos_abs"] + (["pos_swa", "upd_swa", "bt_swa_trim"] if win else [])
    for k in keys:
        assert np.array_equal(got[k].cpu().numpy(), ref[k]), k
    assert np.array_equal(got["seq_lens"].cpu().numpy(), sl)
    assert np.array_equal(got["bt_full"].cpu().numpy(), bf)


@pytest.mark.parametrize("name", ["cfg2", "cfg5"])
def test_csr_step_matches_oracle(name, gpu):
    """A whole step driven by page lists, against the oracle."""
    print(f"[csr step] {name}", flush=True)
    wl = W.make_workload(W.CONFIGS[name])
    host = W.make_buffers(wl, "cpu")
    poison_stale(host, wl)
    snaps = [h.numpy().copy() for h in host]
    bufs = [h.to(gpu) for h in host]
    outs, _ = gpu_step(wl, bufs, gpu, tables="csr")
    ref, _ = oracle_step(wl, snaps)
    for i in range(wl.cfg.layers):
        assert_close(outs[i], ref[i], f"{name} csr layer {i}")
    for j, b in enumerate(bufs):
        got = b.cpu().numpy()
        assert np.array_equal(got, snaps[j]), f"buffer {j}: {int((got != snaps[j]).sum())} bytes differ"
