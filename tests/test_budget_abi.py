"""The library's KV-budget calls against the oracle (host-only, no GPU)."""
import numpy as np
import pytest

import paged_fp8_kv_amd as P
from oracle import budget as OB

GIB = 1 << 30


def test_budget_matches_oracle_on_random_inputs():
    rng = np.random.default_rng(7)
    for _ in range(3000):
        tot = int(rng.integers(0, 1 << 40))
        used = int(rng.integers(0, 1 << 40)) if rng.random() < 0.5 else int(rng.integers(0, tot + 1))
        gmu = float(rng.choice([rng.uniform(0, 1), 0.9, 0.95, 1.0, 0.55, 0.3]))
        cap = float(rng.choice([rng.uniform(0, 1), 0.30, 0.25, 1.0]))
        mn = float(rng.choice([0.0, 1.0, 0.5, 4.0]))
        try:
            want = OB.kv_budget(tot, used, gmu, cap, mn)
        except OB.BudgetTooSmall:
            with pytest.raises(P.PkvError) as e:
                P.pkv_kv_budget(tot, used, gmu, cap, mn)
            assert e.value.status == P.PKV_ERR_DATA
            continue
        assert P.pkv_kv_budget(tot, used, gmu, cap, mn) == want, (tot, used, gmu, cap, mn)


def test_budget_defaults_and_errors():
    assert P.pkv_kv_budget(288 * GIB, 10 * GIB, 0.75, 0.25) == 54 * GIB
    assert P.pkv_kv_budget(288 * GIB, 10 * GIB, 0.9) == OB.kv_budget(288 * GIB, 10 * GIB, 0.9)
    for bad in ((-1, 0, 0.5), (1, -1, 0.5), (1, 0, 1.5), (1, 0, float("nan"))):
        with pytest.raises(P.PkvError) as e:
            P.pkv_kv_budget(*bad)
        assert e.value.status == P.PKV_ERR_ARG


@pytest.mark.parametrize("avail,nbuf,H,Bk,D", [(36175 * 294912, 18, 1, 128, 64),
                                               (9 * GIB + 12345, 18, 8, 32, 64), (0, 1, 1, 16, 64),
                                               (1 << 50, 1, 1, 16, 64)])
def test_num_blocks_matches_oracle(avail, nbuf, H, Bk, D):
    want = min(OB.num_blocks(avail, nbuf, H, Bk, D), 2**31 - 1)
    assert P.pkv_kv_num_blocks(avail, nbuf, H, Bk, D) == want
