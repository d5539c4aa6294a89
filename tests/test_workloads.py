"""Checks of the seeded input generators (CPU only)."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import control as C


@pytest.mark.parametrize("name", ["cfg1", "cfg2", "cfg3", "cfg5"])
def test_tables_are_disjoint_in_range_and_cover_the_window(name):
    cfg = W.CONFIGS[name]
    wl = W.make_workload(cfg)
    full = wl.bt_full[wl.bt_full >= 0]
    swa = wl.bt_swa[wl.bt_swa >= 0]
    assert np.unique(np.concatenate([full, swa])).size == full.size + swa.size
    assert full.max() < wl.nb and (swa.size == 0 or swa.max() < wl.nb)
    for b in range(cfg.batch):
        n = -(-int(wl.seq_lens[b]) // cfg.block)
        assert np.all(wl.bt_full[b, :n] >= 0) and np.all(wl.bt_full[b, n:] == -1)
    if "swa" in cfg.kinds:
        ctl = C.attention_control(wl.seq_lens, wl.active, wl.bt_full, wl.bt_swa, cfg.block, cfg.window)
        for b in range(cfg.batch):
            if wl.active[b]:
                wf = int(ctl["pos_swa"][b])
                assert np.all(ctl["bt_swa_trim"][b, : wf // cfg.block + 1] >= 0)


def test_config_specifics():
    c1 = W.make_workload(W.CONFIGS["cfg1"])
    assert c1.nb == 64 and c1.seq_lens[0] == 256 and c1.k_scale[0] == c1.v_scale[0] == 0.125
    c5 = W.make_workload(W.CONFIGS["cfg5"])
    assert int((c5.active == 0).sum()) == 64
    assert np.all(c5.positions >= c5.seq_lens - 1)
    assert np.all(c5.positions <= c5.seq_lens - 1 + 100000)
    assert c5.seq_lens.min() >= 100 and c5.seq_lens.max() <= 600
    c4 = W.make_workload(W.CONFIGS["cfg4"], hbm_bytes=288 * 10 ** 9)
    assert c4.nb == int(0.30 * 288 * 10 ** 9) // (2 * 8 * 32 * 64)
    assert c4.seq_lens.min() >= 128 and c4.seq_lens.max() <= 32768


def test_deterministic():
    a = W.make_workload(W.CONFIGS["cfg2"])
    b = W.make_workload(W.CONFIGS["cfg2"])
    assert np.array_equal(a.bt_full, b.bt_full) and torch.equal(a.q, b.q)
    ba = W.make_buffers(a)
    bb = W.make_buffers(b)
    assert all(torch.equal(x, y) for x, y in zip(ba, bb))


def test_buffer_fill_poisons_unreferenced_blocks():
    wl = W.make_workload(W.CONFIGS["cfg2"])
    buf = W.make_buffers(wl)[0].view(2, wl.nb, -1)
    unref = np.setdiff1d(np.arange(wl.nb), wl.referenced)
    assert torch.all(buf[:, torch.from_numpy(unref)] == W.POISON)
