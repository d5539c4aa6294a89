"""Pins of the oracle's buffer layout (CPU only)."""
import itertools
import json
import os

import numpy as np
import torch

from oracle import layout as Lo

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_buffer_bytes_reproduce_the_120b_budget():
    g = json.load(open(os.path.join(GOLD, "kv_budget_120b.json")))
    per_buffer = Lo.buffer_bytes(g["num_blocks"], g["kv_heads"], g["block"], g["head_size"])
    total = g["group_size"] * per_buffer
    assert round(total / 2 ** 30, g["printed_digits"]) == g["kv_gib_printed"]
    assert total == 10_668_441_600


def test_packed_and_plain_halves_have_equal_size():
    for nb, H, Bk, D in [(5, 2, 16, 64), (3, 8, 32, 64), (2, 1, 128, 64)]:
        n = Lo.half_bytes(nb, H, Bk, D)
        assert n == nb * H * (Bk // 2) * D * 2


def _all_offsets(fn, nb, H, Bk, D):
    return [fn(n, h, t, j, H, Bk, D)
            for n, h, t, j in itertools.product(range(nb), range(H), range(Bk), range(D))]


def test_offsets_are_bijections():
    nb, H, Bk, D = 3, 2, 8, 5
    for fn in (Lo.plain_offset, Lo.packed_offset):
        offs = _all_offsets(fn, nb, H, Bk, D)
        assert sorted(offs) == list(range(Lo.half_bytes(nb, H, Bk, D)))


def test_offsets_agree_with_torch_views():
    """The page's shapes, taken literally through torch.view, locate the same bytes."""
    g = json.load(open(os.path.join(GOLD, "packed_k_view.json")))
    assert g["packed_k_view_tail"] == ["block//2", "d", "2"]
    nb, H, Bk, D = 3, 2, 8, 5
    n_half = Lo.half_bytes(nb, H, Bk, D)
    plain = torch.zeros(n_half, dtype=torch.int64)
    packed = torch.zeros(n_half, dtype=torch.int64)
    pv = plain.view(nb, H, Bk, D)
    kv = packed.view(nb, H, Bk // 2, D, 2)
    for n, h, t, j in itertools.product(range(nb), range(H), range(Bk), range(D)):
        tag = 1 + ((n * H + h) * Bk + t) * D + j
        plain[Lo.plain_offset(n, h, t, j, H, Bk, D)] = tag
        packed[Lo.packed_offset(n, h, t, j, H, Bk, D)] = tag
        assert pv[n, h, t, j] == tag
        assert kv[n, h, t // 2, j, t % 2] == tag
    # both halves hold every tag once: same bytes, different arrangement
    assert sorted(plain.tolist()) == sorted(packed.tolist())
    # and the packed arrangement interleaves token pairs per dimension
    assert kv[0, 0, 0, 0, 1] == plain.view(nb, H, Bk, D)[0, 0, 1, 0]


def test_rank_rule_distinguishes_packed_k():
    nb, H, Bk, D = 4, 2, 16, 64
    buf = torch.zeros(2, nb, H, Bk, D, dtype=torch.uint8)
    k = buf[0].view(nb, H, Bk // 2, D, 2)
    v = buf[1]
    assert k.dim() == v.dim() + 1
    assert k.data_ptr() == buf.data_ptr() and k.numel() == v.numel()
