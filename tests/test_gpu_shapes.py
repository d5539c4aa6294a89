"""Parity against the oracle across the supported shapes that the benchmark
configurations leave out: query/KV group sizes 1, 2, 4 and 8, blocks of 16,
64 and 128 tokens, batches on both sides of the 64-sequence register prefix
up to the largest supported batch, contexts of one token, contexts that end
mid-block or just past the window, contexts of up to 131,072 tokens (items
cut into hundreds of pieces), tiny items split between two waves, inactive
rows and an all-inactive batch.
Each case runs the alternating window/full layer pair through the layer entry
point; the written cache is compared byte for byte, the outputs within the
attention tolerance."""
import numpy as np
import pytest

import workloads as W
from gpu_harness import assert_close, gpu_step, oracle_step, poison_stale
from workloads import Config

pytestmark = pytest.mark.gpu

PAIR = ("swa", "full")
CASES = [
    # name,                  hq, hkv, block, batch, contexts,      inactive, seed
    ("g1_bk16_b3_L1-300", 4, 4, 16, 3, ("uniform", 1, 300), 0, 11),
    ("g2_bk64_b70_L1-700", 8, 4, 64, 70, ("uniform", 1, 700), 5, 12),
    ("g4_bk128_b5_L100-1500", 8, 2, 128, 5, ("uniform", 100, 1500), 0, 13),
    ("g8_bk64_b2_L129", 16, 2, 64, 2, ("fixed", 129), 0, 14),
    ("g8_bk16_b8192_L1-40", 8, 1, 16, 8192, ("uniform", 1, 40), 100, 15),
    # items of 1-3 sub-tiles split between two waves: a 1-sub-tile item's second
    # share holds only padding, a 2-sub-tile item has padding on both sides,
    # a 3-sub-tile item splits 2 + 1 (register prefix, then LDS prefix)
    ("g8_bk16_b40_L1-70_halves", 16, 2, 16, 40, ("uniform", 1, 70), 3, 16),
    ("g4_bk16_b100_L1-70_halves", 16, 4, 16, 100, ("uniform", 1, 70), 7, 17),
    # the same short contexts behind tables 1024 tokens wide: the full layer
    # can no longer bound its items by the table, so it runs the stream-K
    # kernel (its two-waves-per-item mode and, at 8192 sequences, its LDS
    # prefix) instead of the direct one
    ("g8_bk16_b40_L1-70_halves_wide", 16, 2, 16, 40, ("uniform", 1, 70), 3, 16, 1024),
    ("g4_bk16_b100_L1-70_halves_wide", 16, 4, 16, 100, ("uniform", 1, 70), 7, 17, 1024),
    ("g8_bk16_b8192_L1-40_wide", 8, 1, 16, 8192, ("uniform", 1, 40), 100, 15, 1024),
    # 128K-token contexts: one item of 4,096 sub-tiles cut between ~340 waves
    # and merged in rounds of eight; two and six sequences whose items are
    # cut into tens of pieces each
    ("g8_bk16_b1_L131072", 8, 1, 16, 1, ("fixed", 131072), 0, 18),
    ("g8_bk32_b2_L100k-128k", 64, 8, 32, 2, ("uniform", 100000, 131072), 0, 19),
    ("g8_bk32_b6_L16-128k_log", 64, 8, 32, 6, ("loguniform", 16, 131072), 1, 35),
]


def _run(cfg, gpu):
    wl = W.make_workload(cfg)
    host = W.make_buffers(wl, "cpu")
    poison_stale(host, wl)
    snaps = [h.numpy().copy() for h in host]
    bufs = [h.to(gpu) for h in host]
    print(f"[shapes] {cfg.name}: nb={wl.nb}", flush=True)
    outs, _ = gpu_step(wl, bufs, gpu)
    ref, _ = oracle_step(wl, snaps)  # brings `snaps` to the post-step cache
    for j, b in enumerate(bufs):
        got = b.cpu().numpy()
        assert np.array_equal(got, snaps[j]), \
            f"{cfg.name} buffer {j}: {int((got != snaps[j]).sum())} bytes differ"
    return wl, outs, ref


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_shapes_match_oracle(case, gpu):
    name, hq, hkv, block, batch, ctx, inactive, seed = case[:8]
    cfg = Config(name, PAIR, batch, hq, hkv, 64, block, ctx, seed=seed, n_inactive=inactive,
                 max_ctx=case[8] if len(case) > 8 else ctx[-1])
    wl, outs, ref = _run(cfg, gpu)
    for i in range(cfg.layers):
        assert_close(outs[i], ref[i], f"{name} layer {i}")


def test_all_inactive_batch(gpu):
    """No sequence has work: every output row is +0 and the cache is untouched."""
    cfg = Config("inactive_b4", PAIR, 4, 8, 1, 64, 32, ("uniform", 1, 100), seed=7,
                 n_inactive=4, max_ctx=100)
    wl, outs, ref = _run(cfg, gpu)
    for i in range(cfg.layers):
        o = outs[i].float().cpu().numpy()
        assert np.array_equal(o, np.zeros_like(o)) and not np.signbit(o).any(), f"layer {i}"
        assert np.array_equal(ref[i], np.zeros_like(ref[i]))


def test_many_piece_merge_is_repeatable(gpu):
    """One 131,072-token item cut between ~340 waves: five steps on the same
    cache (each rewrites the same new token) give bitwise the same outputs
    and the same cache, as every piece is cut at a fixed point and the pieces
    merge in a fixed order whichever wave arrives last."""
    import torch
    cfg = Config("g8_bk16_b1_L131072_repeat", PAIR, 1, 8, 1, 64, 16, ("fixed", 131072), seed=18,
                 max_ctx=131072)
    wl = W.make_workload(cfg)
    bufs = [h.to(gpu) for h in W.make_buffers(wl, "cpu")]
    first, _ = gpu_step(wl, bufs, gpu)
    after = [b.clone() for b in bufs]
    for r in range(4):
        outs, _ = gpu_step(wl, bufs, gpu)
        for i in range(cfg.layers):
            assert torch.equal(outs[i].view(torch.int16), first[i].view(torch.int16)), (r, i)
        for j, b in enumerate(bufs):
            assert torch.equal(b, after[j]), (r, j)
