"""Sliding windows other than 128 keys, on the GPU against the oracle.

The pages' model uses a 128-key window ("GPT-OSS-120B giga-kernel decode",
"Kernel contract"), but the setup and the attention entry points take the
window as an argument.  A window of up to 224 keys spans at most 8 32-token
sub-tiles, so its items run the direct kernel like the 128-key window; longer
windows give items of up to 33+ sub-tiles, which run the stream-K kernel's
windowed instantiation with items cut between waves and merged through the
workspace, or the direct kernel with one wave per item when the items alone
fill the GPU.  Each case runs the window/full layer pair through the layer
entry point (one case through the separate update + attention calls); the
written cache is compared byte for byte, the outputs within the attention
tolerance and its tighter guards.

Which kernel a case takes on a 256-CU MI355X is noted beside it; the
comparison does not depend on it."""
import numpy as np
import pytest

import workloads as W
from gpu_harness import assert_close, gpu_step, oracle_step, poison_stale
from workloads import Config

pytestmark = pytest.mark.gpu

PAIR = ("swa", "full")
# name, window, hq, hkv, block, batch, contexts, inactive, seed, extra options
CASES = [
    # only the new token attends to itself; direct, one wave per item
    ("w1_g8_bk16_b16", 1, 8, 1, 16, 16, ("uniform", 1, 300), 2, 21, {}),
    # 33 keys over 16-token blocks: 2 sub-tiles, direct, two waves per item
    ("w33_g8_bk16_b9", 33, 16, 2, 16, 9, ("uniform", 1, 500), 0, 22, {}),
    # the longest direct window item (8 sub-tiles), four waves per item
    ("w224_g8_bk32_b12", 224, 64, 8, 32, 12, ("uniform", 100, 1200), 1, 23, {}),
    # 9 sub-tiles and few items: stream-K, items cut between waves
    ("w256_g8_bk32_b10", 256, 64, 8, 32, 10, ("uniform", 200, 2000), 0, 24, {}),
    # 33 sub-tiles, lagged anchor, 64-token blocks: stream-K
    ("w1000_g4_bk64_b24_lag1", 1000, 16, 4, 64, 24, ("uniform", 300, 3000), 3, 25,
     dict(anchor_lag=1)),
    # long windows: one item spread over many waves, multi-round merges
    ("w4096_g8_bk32_b6", 4096, 64, 8, 32, 6, ("uniform", 2000, 9000), 0, 26, {}),
    # 2,400 items of up to 11 sub-tiles fill the GPU: direct, one wave each
    ("w300_g1_bk16_b300", 300, 8, 8, 16, 300, ("uniform", 1, 800), 30, 27, {}),
    # token-major K rows through the windowed stream-K kernel
    ("w500_g8_bk16_b8_unpacked", 500, 64, 8, 16, 8, ("uniform", 100, 1500), 0, 28,
     dict(k_packed=False)),
    # 129 keys at 128-token blocks, far absolute positions: direct
    ("w129_g8_bk128_b5_offset", 129, 16, 2, 128, 5, ("uniform", 100, 1500), 0, 29,
     dict(pos_offset_max=100000)),
    # rotary embedding on the windowed stream-K kernel, separate calls
    ("w700_g8_bk32_b8_rope_calls", 700, 64, 8, 32, 8, ("uniform", 500, 3000), 1, 30,
     dict(rope=True, use_layer_api=False)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_window_matches_oracle(case, gpu):
    name, window, hq, hkv, block, batch, ctx, inactive, seed, opt = case
    cfg = Config(name, PAIR, batch, hq, hkv, 64, block, ctx, seed=seed, window=window,
                 n_inactive=inactive, pos_offset_max=opt.get("pos_offset_max", 0),
                 max_ctx=ctx[-1])
    k_packed = opt.get("k_packed", True)
    lag = opt.get("anchor_lag", 0)
    wl = W.make_workload(cfg)
    host = W.make_buffers(wl, "cpu")
    poison_stale(host, wl, k_packed=k_packed)
    snaps = [h.numpy().copy() for h in host]
    bufs = [h.to(gpu) for h in host]
    rope = W.rope_tables(wl) if opt.get("rope") else None
    print(f"[window] {name}: nb={wl.nb}", flush=True)
    outs, _ = gpu_step(wl, bufs, gpu, use_layer_api=opt.get("use_layer_api", True),
                       k_packed=k_packed, rope=rope, anchor_lag=lag)
    ref, _ = oracle_step(wl, snaps, k_packed=k_packed, rope=rope, anchor_lag=lag)
    for j, b in enumerate(bufs):
        got = b.cpu().numpy()
        assert np.array_equal(got, snaps[j]), \
            f"{name} buffer {j}: {int((got != snaps[j]).sum())} bytes differ"
    for i in range(cfg.layers):
        assert_close(outs[i], ref[i], f"{name} layer {i}")
