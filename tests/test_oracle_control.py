"""Pins of the oracle's attention-control setup (CPU only)."""
import json
import os

import numpy as np
import pytest

from oracle import control as C

GOLD = os.path.join(os.path.dirname(__file__), "golden")
W = 128


def _run(block, n_tok=3000):
    p = np.arange(n_tok)
    B = p.size
    width = -(-n_tok // block) + 1
    bt_full = np.tile(np.arange(width, dtype=np.int32) + 10_000, (B, 1))
    bt_swa = np.tile(np.arange(width, dtype=np.int32) + 50_000, (B, 1))
    ctl = C.attention_control(p + 1, np.ones(B, np.uint8), bt_full, bt_swa, block, W)
    return p, bt_full, bt_swa, ctl


@pytest.mark.parametrize("block", [16, 32, 128])
def test_trimmed_frame_covers_exactly_the_window(block):
    p, bt_full, bt_swa, ctl = _run(block)
    n_swa = C.trimmed_width(W, block)
    assert ctl["bt_swa_trim"].shape[1] == n_swa
    for b in range(p.size):
        pb = int(p[b])
        wf = int(ctl["pos_swa"][b])
        origin = pb - wf                       # token index of frame position 0
        assert origin % block == 0 and 0 <= origin <= max(0, pb - W + 1)
        assert origin > pb - W + 1 - block     # frame starts at the block of the oldest key
        lo = max(0, wf - W + 1)
        window = range(max(0, pb - W + 1), pb + 1)
        assert len(window) == wf - lo + 1
        trim = ctl["bt_swa_trim"][b]
        for t in window:
            f = t - origin
            assert trim[f // block] == bt_swa[b, t // block]
        used = int((trim >= 0).sum())
        assert used == pb // block - origin // block + 1 <= n_swa
        assert np.all(trim[used:] == -1)
        assert ctl["pos_full"][b] == pb
        assert ctl["upd_full"][b] == bt_full[b, pb // block] * block + pb % block
        assert ctl["upd_swa"][b] == bt_swa[b, pb // block] * block + pb % block


@pytest.mark.parametrize("block", [16, 32, 128])
def test_oldest_block_is_dropped_at_the_printed_boundary(block):
    g = json.load(open(os.path.join(GOLD, "swa_eviction_boundary.json")))
    assert g["window"] == W and block in g["block_sizes"]
    p, _, bt_swa, ctl = _run(block)
    first = ctl["bt_swa_trim"][:, 0]
    for b in range(1, p.size):
        advanced = first[b] != first[b - 1]
        assert advanced == (p[b] % block == block - 1 and p[b] >= W), int(p[b])


def test_inactive_and_missing_blocks():
    bt = np.arange(8, dtype=np.int32).reshape(2, 4)
    swa = np.full((2, 4), -1, dtype=np.int32)
    ctl = C.attention_control([40, 40], [1, 0], bt, swa, 16, W, positions=[1000, 5])
    assert ctl["upd_full"][1] == -1 and ctl["pos_full"][1] == -1 and ctl["pos_swa"][1] == -1
    assert np.all(ctl["bt_swa_trim"][1] == -1)
    assert ctl["upd_swa"][0] == -1          # no window block allocated: no write
    assert ctl["upd_full"][0] == bt[0, 2] * 16 + 7
    assert list(ctl["pos_abs"]) == [1000, -1]


def test_trimmed_width_values():
    assert [C.trimmed_width(W, b) for b in (16, 32, 128)] == [9, 5, 2]
