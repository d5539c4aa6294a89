"""Pins of the oracle's paged decode attention (CPU only)."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import control as C
from paged_build import bf16_values, build_halves, random_codes, torch_decode


def _case(rng, B, Hq, H, Bk, D, lens, packed=True, nb_extra=5):
    nblk = [-(-L // Bk) for L in lens]
    nb = sum(nblk) + nb_extra
    perm = rng.permutation(nb)
    width = max(nblk)
    table = np.full((B, width), -1, dtype=np.int32)
    at = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[at:at + nblk[b]]
        at += nblk[b]
    k_log = [random_codes(rng, (L, H, D)) for L in lens]
    v_log = [random_codes(rng, (L, H, D), 1.0 / 16) for L in lens]
    kh, vh = build_halves(k_log, v_log, [table[b] for b in range(B)], nb, H, Bk, D, packed)
    q = bf16_values(rng, (B, Hq, D))
    return dict(nb=nb, table=table, k_log=k_log, v_log=v_log, kh=kh, vh=vh, q=q)


def _dense(case, b, g, G, lo, hi, ks, vs, sm):
    h = g // G
    K = torch_decode(case["k_log"][b][lo:hi + 1, h]) * ks
    V = torch_decode(case["v_log"][b][lo:hi + 1, h]) * vs
    return A.dense_attention(list(case["q"][b, g]), K.tolist(), V.tolist(), sm)


@pytest.mark.parametrize("packed", [True, False])
def test_matches_fsum_bruteforce(packed):
    rng = np.random.default_rng(0)
    B, Hq, H, Bk, D = 3, 4, 2, 4, 8
    lens = [1, 7, 13]
    c = _case(rng, B, Hq, H, Bk, D, lens, packed)
    ks, vs, sm = 0.125, 0.0625, 1 / math.sqrt(D)
    out = A.paged_decode_attention(c["q"], c["kh"], c["vh"], c["table"],
                                   np.array(lens) - 1, 0, Bk, H, ks, vs, sm, packed)
    for b in range(B):
        for g in range(Hq):
            ref = _dense(c, b, g, Hq // H, 0, lens[b] - 1, ks, vs, sm)
            assert np.allclose(out[b, g], ref, rtol=0, atol=1e-13)


def test_matches_torch_sdpa_gqa():
    rng = np.random.default_rng(1)
    B, Hq, H, Bk, D = 4, 16, 2, 16, 64
    lens = [300, 17, 129, 64]
    c = _case(rng, B, Hq, H, Bk, D, lens)
    ks, vs, sm = 0.125, 0.0625, 0.125
    out = A.paged_decode_attention(c["q"], c["kh"], c["vh"], c["table"],
                                   np.array(lens) - 1, 0, Bk, H, ks, vs, sm)
    G = Hq // H
    for b in range(B):
        K = torch.from_numpy(torch_decode(c["k_log"][b]) * ks).permute(1, 0, 2)  # [H, L, D]
        V = torch.from_numpy(torch_decode(c["v_log"][b]) * vs).permute(1, 0, 2)
        K = K.repeat_interleave(G, dim=0)
        V = V.repeat_interleave(G, dim=0)
        Q = torch.from_numpy(c["q"][b]).unsqueeze(1)                              # [Hq, 1, D]
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=sm).squeeze(1)
        assert np.allclose(out[b], ref.numpy(), rtol=0, atol=1e-12)


@pytest.mark.parametrize("Bk", [16, 32])
def test_window_equals_dense_over_last_128(Bk):
    rng = np.random.default_rng(2)
    B, Hq, H, D, W = 3, 8, 1, 64, 128
    lens = [300, 129, 160]
    c = _case(rng, B, Hq, H, Bk, D, lens)
    ctl = C.attention_control(np.array(lens), np.ones(B, np.uint8), c["table"], c["table"], Bk, W)
    out = A.paged_decode_attention(c["q"], c["kh"], c["vh"], ctl["bt_swa_trim"], ctl["pos_swa"],
                                   W, Bk, H, 0.125, 0.0625, 0.125)
    for b in range(B):
        for g in range(Hq):
            ref = _dense(c, b, g, Hq, lens[b] - W, lens[b] - 1, 0.125, 0.0625, 0.125)
            assert np.allclose(out[b, g], ref, rtol=0, atol=1e-13)


@pytest.mark.parametrize("Bk,W,lens", [(16, 1, [5, 1, 40]), (16, 33, [100, 33, 34]),
                                        (32, 256, [600, 257, 300]), (64, 1000, [1300, 1001, 1100])])
def test_window_equals_dense_over_the_last_w_keys(Bk, W, lens):
    """Windows other than 128: the oracle attends exactly the last W keys."""
    rng = np.random.default_rng(5)
    B, Hq, H, D = 3, 4, 1, 64
    c = _case(rng, B, Hq, H, Bk, D, lens)
    ctl = C.attention_control(np.array(lens), np.ones(B, np.uint8), c["table"], c["table"], Bk, W)
    out = A.paged_decode_attention(c["q"], c["kh"], c["vh"], ctl["bt_swa_trim"], ctl["pos_swa"],
                                   W, Bk, H, 0.125, 0.0625, 0.125)
    for b in range(B):
        for g in range(Hq):
            ref = _dense(c, b, g, Hq, max(0, lens[b] - W), lens[b] - 1, 0.125, 0.0625, 0.125)
            assert np.allclose(out[b, g], ref, rtol=0, atol=1e-13)


def test_window_equals_full_when_context_fits():
    rng = np.random.default_rng(3)
    B, Hq, H, Bk, D, W = 4, 8, 2, 16, 64, 128
    lens = [1, 40, 127, 128]
    c = _case(rng, B, Hq, H, Bk, D, lens)
    ctl = C.attention_control(np.array(lens), np.ones(B, np.uint8), c["table"], c["table"], Bk, W)
    full = A.paged_decode_attention(c["q"], c["kh"], c["vh"], c["table"], ctl["pos_full"],
                                    0, Bk, H, 0.125, 0.0625, 0.125)
    swa = A.paged_decode_attention(c["q"], c["kh"], c["vh"], ctl["bt_swa_trim"], ctl["pos_swa"],
                                   W, Bk, H, 0.125, 0.0625, 0.125)
    assert np.array_equal(full, swa)


def test_single_token_returns_its_value():
    rng = np.random.default_rng(4)
    c = _case(rng, 1, 8, 1, 16, 64, [1])
    out = A.paged_decode_attention(c["q"], c["kh"], c["vh"], c["table"], [0], 0, 16, 1,
                                   0.125, 0.0625, 0.125)
    v0 = torch_decode(c["v_log"][0][0, 0]) * 0.0625
    assert np.array_equal(out[0], np.tile(v0, (8, 1)))


def test_equal_keys_give_mean_of_values():
    rng = np.random.default_rng(5)
    c = _case(rng, 1, 8, 1, 16, 64, [50])
    c["k_log"][0][:] = c["k_log"][0][0]
    kh, vh = build_halves(c["k_log"], c["v_log"], [c["table"][0]], c["nb"], 1, 16, 64)
    out = A.paged_decode_attention(c["q"], kh, vh, c["table"], [49], 0, 16, 1, 0.125, 0.0625, 0.125)
    mean = (torch_decode(c["v_log"][0][:, 0]) * 0.0625).mean(axis=0)
    assert np.allclose(out[0], np.tile(mean, (8, 1)), rtol=0, atol=1e-15)


def test_block_relabelling_is_invisible():
    rng = np.random.default_rng(6)
    B, Hq, H, Bk, D = 2, 8, 2, 16, 64
    lens = [200, 77]
    c = _case(rng, B, Hq, H, Bk, D, lens)
    relabel = rng.permutation(c["nb"])
    t2 = np.where(c["table"] >= 0, relabel[np.maximum(c["table"], 0)], -1).astype(np.int32)
    kh2, vh2 = build_halves(c["k_log"], c["v_log"], [t2[b] for b in range(B)], c["nb"], H, Bk, D)
    a = A.paged_decode_attention(c["q"], c["kh"], c["vh"], c["table"], np.array(lens) - 1,
                                 0, Bk, H, 0.125, 0.0625, 0.125)
    b = A.paged_decode_attention(c["q"], kh2, vh2, t2, np.array(lens) - 1, 0, Bk, H,
                                 0.125, 0.0625, 0.125)
    assert np.array_equal(a, b)


def test_scale_linearity_head_map_and_inactive():
    rng = np.random.default_rng(7)
    B, Hq, H, Bk, D = 3, 8, 2, 16, 64
    lens = [33, 90, 5]
    c = _case(rng, B, Hq, H, Bk, D, lens)
    c["q"][:, 1] = c["q"][:, 0]
    pos = np.array(lens) - 1
    pos[2] = -1
    o1 = A.paged_decode_attention(c["q"], c["kh"], c["vh"], c["table"], pos, 0, Bk, H,
                                  0.125, 0.0625, 0.125)
    o2 = A.paged_decode_attention(c["q"], c["kh"], c["vh"], c["table"], pos, 0, Bk, H,
                                  0.125, 0.125, 0.125)
    assert np.array_equal(2 * o1, o2)
    assert np.array_equal(o1[:, 0], o1[:, 1])
    assert np.all(o1[2] == 0)
    # q heads 0..3 read KV head 0 and 4..7 read KV head 1: a head-1-only change
    v_log = [v.copy() for v in c["v_log"]]
    for v in v_log:
        v[:, 1] = 0x38      # 1.0
    kh, vh = build_halves(c["k_log"], v_log, [c["table"][b] for b in range(B)], c["nb"], H, Bk, D)
    o3 = A.paged_decode_attention(c["q"], kh, vh, c["table"], pos, 0, Bk, H, 0.125, 0.0625, 0.125)
    assert np.array_equal(o3[:2, :4], o1[:2, :4])
    assert np.allclose(o3[:2, 4:], 0.0625, rtol=0, atol=1e-15)


def test_poison_outside_tables_never_read():
    rng = np.random.default_rng(8)
    c = _case(rng, 2, 8, 1, 16, 64, [20, 50])
    out = A.paged_decode_attention(c["q"], c["kh"], c["vh"], c["table"], [19, 49], 0, 16, 1,
                                   0.125, 0.0625, 0.125)
    assert np.all(np.isfinite(out))
