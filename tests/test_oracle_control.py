"""Pins of the oracle's attention-control setup (CPU only)."""
import json
import os

import numpy as np
import pytest

from oracle import control as C

GOLD = os.path.join(os.path.dirname(__file__), "golden")
W = 128


def _run(block, n_tok=3000, window=W):
    p = np.arange(n_tok)
    B = p.size
    width = -(-n_tok // block) + 1
    bt_full = np.tile(np.arange(width, dtype=np.int32) + 10_000, (B, 1))
    bt_swa = np.tile(np.arange(width, dtype=np.int32) + 50_000, (B, 1))
    ctl = C.attention_control(p + 1, np.ones(B, np.uint8), bt_full, bt_swa, block, window)
    return p, bt_full, bt_swa, ctl


# the pages' window of 128 at every supported block, and other windows (the
# setup takes the window as an argument): 1 key, 33 keys, 1000 keys
@pytest.mark.parametrize("block,window", [(16, 128), (32, 128), (128, 128), (16, 1), (16, 33),
                                          (64, 33), (32, 1000), (64, 1000)])
def test_trimmed_frame_covers_exactly_the_window(block, window):
    W = window
    p, bt_full, bt_swa, ctl = _run(block, 3000 if W < 1000 else 2500, W)
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


def _to_csr(seq_lens, bt_full, bt_swa, block):
    """Compress padded tables by hand (plain loops, independent of the oracle)."""
    indptr, full, swa, last = [0], [], [], []
    for b in range(len(seq_lens)):
        n = -(-int(seq_lens[b]) // block)
        for c in range(n):
            full.append(int(bt_full[b, c])); swa.append(int(bt_swa[b, c]))
        indptr.append(indptr[-1] + n)
        last.append(int(seq_lens[b]) - (n - 1) * block if n else 0)
    return np.array(indptr), np.array(full), np.array(swa), np.array(last)


@pytest.mark.parametrize("block", [16, 32, 128])
def test_csr_round_trip_and_lengths(block):
    """Padded tables -> compressed page lists -> padded tables is the identity
    on every referenced column, and lengths follow (pages-1)*block + last."""
    rng = np.random.default_rng(block)
    B, width = 40, 70
    L = rng.integers(0, width * block + 1, size=B).astype(np.int32)
    L[:3] = [0, 1, width * block]
    bt_full = np.full((B, width), -1, np.int32)
    bt_swa = np.full((B, width), -1, np.int32)
    for b in range(B):
        n = -(-int(L[b]) // block)
        bt_full[b, :n] = rng.integers(0, 10**6, n)
        keep = max(0, n - 5)
        bt_swa[b, keep:n] = rng.integers(0, 10**6, n - keep)
    ip, fi, si, lp = _to_csr(L, bt_full, bt_swa, block)
    sl, f2, s2 = C.csr_to_tables(ip, fi, si, lp, block, width)
    assert np.array_equal(sl, L)
    assert np.array_equal(f2, bt_full) and np.array_equal(s2, bt_swa)
    # the control built from either form is the same
    act = (L > 0).astype(np.uint8)
    a = C.attention_control(L, act, bt_full, bt_swa, block, 128)
    b_ = C.attention_control(sl, act, f2, s2, block, 128)
    for k in a:
        assert np.array_equal(a[k], b_[k]), k


def test_csr_hand_example():
    """Two sequences, block 4: 3 pages with 2 tokens in the last (10 tokens),
    and 1 page with 4 tokens; the window list frees the first page."""
    sl, f, s = C.csr_to_tables([0, 3, 4], [7, 2, 9, 5], [-1, 11, 12, 13], [2, 4], 4, 5)
    assert sl.tolist() == [10, 4]
    assert f.tolist() == [[7, 2, 9, -1, -1], [5, -1, -1, -1, -1]]
    assert s.tolist() == [[-1, 11, 12, -1, -1], [13, -1, -1, -1, -1]]


def _run_lag(block, lag, n_tok=3000):
    p = np.arange(n_tok)
    B = p.size
    width = -(-n_tok // block) + 1
    bt_full = np.tile(np.arange(width, dtype=np.int32) + 10_000, (B, 1))
    bt_swa = np.tile(np.arange(width, dtype=np.int32) + 50_000, (B, 1))
    ctl = C.attention_control(p + 1, np.ones(B, np.uint8), bt_full, bt_swa, block, W,
                              anchor_lag=lag)
    return p, bt_swa, ctl


@pytest.mark.parametrize("block", [16, 32, 128])
def test_lagged_anchor_keeps_the_oldest_block_one_step_longer(block):
    """"DI wiring (NIXL)": with the frame anchored one token back (both nodes
    at N - 1) the oldest block is not dropped at the printed boundary
    N % block_size == block_size - 1 but one step later, and the frame of
    step p is exactly the frame the unlagged setup gives step p - 1."""
    g = json.load(open(os.path.join(GOLD, "swa_eviction_boundary.json")))
    assert g["window"] == W and block in g["block_sizes"]
    p, bt_swa, lag = _run_lag(block, 1)
    _, _, ref = _run_lag(block, 0)
    assert C.trimmed_width(W, block, 1) == C.trimmed_width(W, block) == lag["bt_swa_trim"].shape[1]
    first = lag["bt_swa_trim"][:, 0]
    for b in range(1, p.size):
        pb = int(p[b])
        advanced = first[b] != first[b - 1]
        assert advanced == (pb % block == 0 and pb >= W + block), pb
        if pb % block == block - 1 and pb >= W:
            # the printed boundary: the unlagged frame just dropped a block,
            # the lagged one still holds it (the block of token p - W)
            assert ref["bt_swa_trim"][b, 0] != ref["bt_swa_trim"][b - 1, 0]
            assert first[b] == ref["bt_swa_trim"][b - 1, 0] == bt_swa[b, (pb - W) // block]
        # frame of p with the lag == frame of p - 1 without it
        origin_lag = pb - int(lag["pos_swa"][b])
        origin_ref = (pb - 1) - int(ref["pos_swa"][b - 1])
        assert origin_lag == origin_ref
        # the window's keys are all still in the lagged frame, and the
        # write index is the same slot
        trim = lag["bt_swa_trim"][b]
        for t in range(max(0, pb - W + 1), pb + 1):
            assert trim[(t - origin_lag) // block] == bt_swa[b, t // block]
        assert lag["upd_swa"][b] == ref["upd_swa"][b]
        assert lag["pos_full"][b] == ref["pos_full"][b] and lag["upd_full"][b] == ref["upd_full"][b]


def test_lagged_trimmed_width_grows_only_when_needed():
    # a window of 17 keys at block 16 spans 2 blocks, plus one lagged token 3
    assert C.trimmed_width(17, 16, 0) == 2 and C.trimmed_width(17, 16, 1) == 3
    assert [C.trimmed_width(W, b, 1) for b in (16, 32, 128)] == [9, 5, 2]
    with pytest.raises(ValueError):
        C.attention_control([5], [1], np.zeros((1, 1), np.int32), np.zeros((1, 1), np.int32),
                            16, W, anchor_lag=2)


@pytest.mark.parametrize("block", [16, 32])
def test_lagged_frame_attends_the_same_keys(block):
    """Window attention through the lagged frame equals attention through the
    unlagged one exactly (same keys, same order), at every offset around two
    eviction boundaries."""
    from oracle import attention as OA
    from paged_build import bf16_values, random_codes
    rng = np.random.default_rng(block)
    H, D = 1, 64
    lens = np.arange(W + block - 3, W + 2 * block + 3)      # p across two boundaries
    B = lens.size
    width = -(-int(lens.max()) // block)
    nb = width * B + 4
    perm = rng.permutation(nb)
    bt_swa = perm[:B * width].reshape(B, width).astype(np.int32)
    bt_full = np.full_like(bt_swa, -1)
    half = nb * H * block * D
    kh = random_codes(rng, (half,))
    vh = random_codes(rng, (half,))
    q = bf16_values(rng, (B, 2, D))
    outs = []
    for lag in (0, 1):
        ctl = C.attention_control(lens, np.ones(B, np.uint8), bt_swa, bt_swa, block, W,
                                  anchor_lag=lag)
        outs.append(OA.paged_decode_attention(q, kh, vh, ctl["bt_swa_trim"], ctl["pos_swa"], W,
                                              block, H, 0.125, 0.0625, 0.125))
    assert np.array_equal(outs[0], outs[1])
