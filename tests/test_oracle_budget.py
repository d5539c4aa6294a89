"""Pins of the KV-budget host policy ("determine_available_memory design").
Inputs use fractions that are exact in binary, so every expected value is a
closed form written out here; the truncation, clamp and guard cases are the
page's own edge cases."""
import json
import os

import numpy as np
import pytest

from oracle import budget as OB

GIB = 1 << 30
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_cap_binds():
    # 288 GiB device, 10 GiB resident, GMU 3/4, cap 1/4 of the 216 GiB budget
    assert OB.kv_budget(288 * GIB, 10 * GIB, 0.75, 0.25) == 54 * GIB


def test_resident_memory_binds():
    # 16 GiB * 3/4 = 12 GiB budget, 10 GiB resident -> 2 GiB (< the 3 GiB cap)
    assert OB.kv_budget(16 * GIB, 10 * GIB, 0.75, 0.25) == 2 * GIB


def test_products_are_truncated():
    # 10 * 0.55 = 5.5 -> 5; cap 5 * 0.5 = 2.5 -> 2
    assert OB.kv_budget(10, 0, 0.55, 0.5, min_kv_gib=0) == 2
    # 7 * 0.5 = 3.5 -> 3 total, 1 resident -> 2; cap 3 * 1.0 = 3
    assert OB.kv_budget(7, 1, 0.5, 1.0, min_kv_gib=0) == 2


def test_clamped_at_zero_then_guarded():
    assert OB.kv_budget(4 * GIB, 8 * GIB, 0.5, 1.0, min_kv_gib=0) == 0
    with pytest.raises(OB.BudgetTooSmall):
        OB.kv_budget(4 * GIB, 8 * GIB, 0.5, 1.0)


def test_guard_threshold_is_one_gib_inclusive():
    # total budget 4 GiB (gmu 1), cap 1/4 -> exactly 1 GiB: allowed
    assert OB.kv_budget(4 * GIB, 0, 1.0, 0.25) == GIB
    with pytest.raises(OB.BudgetTooSmall):
        OB.kv_budget(4 * GIB - 4, 0, 1.0, 0.25)      # 1 GiB - 1 byte
    assert OB.DEFAULT_CAP_FRACTION == 0.30 and OB.DEFAULT_MIN_KV_GIB == 1.0


def test_monotone_in_memory_and_resident_bytes():
    rng = np.random.default_rng(0)
    for _ in range(500):
        tot = int(rng.integers(1, 1 << 40)); used = int(rng.integers(0, 1 << 39))
        gmu = float(rng.uniform(0.05, 1.0)); cap = float(rng.uniform(0.0, 1.0))
        a = OB.kv_budget(tot, used, gmu, cap, min_kv_gib=0)
        assert a <= OB.kv_budget(tot + int(rng.integers(0, 1 << 30)), used, gmu, cap, min_kv_gib=0)
        assert a >= OB.kv_budget(tot, used + int(rng.integers(0, 1 << 30)), gmu, cap, min_kv_gib=0)
        assert 0 <= a <= int(tot * gmu)


def test_blocks_for_the_printed_120b_budget():
    """"GPT-OSS-120B giga-kernel decode", "KV budget (no cap)": 36,175 blocks of
    the 120B shapes over 18 buffers; any budget in [36175, 36176) block-bytes
    yields exactly that count."""
    g = json.load(open(os.path.join(GOLD, "kv_budget_120b.json")))
    per = g["group_size"] * 2 * g["kv_heads"] * g["block"] * g["head_size"]
    for extra in (0, 1, per - 1):
        assert OB.num_blocks(g["num_blocks"] * per + extra, g["group_size"], g["kv_heads"],
                             g["block"], g["head_size"]) == g["num_blocks"]
    assert OB.num_blocks(g["num_blocks"] * per - 1, g["group_size"], g["kv_heads"],
                         g["block"], g["head_size"]) == g["num_blocks"] - 1
