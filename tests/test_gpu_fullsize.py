"""Parity at the full workload sizes, in the configuration the benchmark times
(the layer entry point with its default split and workspace): the whole step
runs on the GPU; the oracle recomputes a sample of sequences from a copy of
the blocks they reference, taken before the step."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_harness import (assert_close, gather_blocks, gpu_step, mini_workload, oracle_step,
                         sampled_blocks)

pytestmark = pytest.mark.gpu


def _run(name, rows_fn, layers, gpu):
    cfg = W.CONFIGS[name]
    hbm = torch.cuda.mem_get_info(gpu)[1]
    wl = W.make_workload(cfg, hbm_bytes=hbm)
    rows = rows_fn(wl)
    print(f"[fullsize] {name}: nb={wl.nb} rows={rows.tolist()} layers={layers}", flush=True)
    bufs = []
    for j in range(cfg.n_buffers):
        t = torch.empty(2 * wl.half_bytes, dtype=torch.uint8, device=gpu)
        W.fill_buffer(t, wl, j)
        bufs.append(t)
    blocks = sampled_blocks(wl, rows)
    before = [gather_blocks(b, wl, blocks) for b in bufs]
    outs, _ = gpu_step(wl, bufs, gpu)
    after = [gather_blocks(b, wl, blocks) for b in bufs]
    mini = mini_workload(wl, rows, blocks)
    ref, _ = oracle_step(mini, before, layers=set(layers))   # updates `before` in place
    worst = 0.0
    for i in layers:
        got = outs[i][torch.from_numpy(rows).to(gpu)]
        worst = max(worst, assert_close(got, ref[i][rows], f"{name} layer {i} rows {rows.tolist()}"))
    # every byte of the sampled blocks (the new tokens' slots included)
    for j in range(cfg.n_buffers):
        assert np.array_equal(after[j], before[j]), \
            f"{name} buffer {j}: {int((after[j] != before[j]).sum())} bytes differ"
    print(f"[fullsize] {name}: max abs err {worst:.2e}", flush=True)
    # hand the pool back now: the driver's clean-up of tens of GB of freed
    # device memory slows later bandwidth-bound work for some seconds, so let
    # it overlap the rest of the session rather than what runs after it
    del bufs, outs
    torch.cuda.empty_cache()


def test_fullsize_36_layer_batch64(gpu):
    """36 alternating layers, batch 64, 8192-token contexts: two sequences,
    the first and the last pair of layers."""
    _run("cfg3", lambda wl: np.array([5, 63]), [0, 1, 34, 35], gpu)


def test_fullsize_ragged_batch128_large_pool(gpu):
    """Batch 128, log-uniform 128..32768 contexts, pool at 30% of HBM: the
    longest, the shortest and a middle sequence."""
    def rows(wl):
        o = np.argsort(wl.seq_lens, kind="stable")
        return np.array(sorted({int(o[-1]), int(o[0]), int(o[len(o) // 2])}))
    _run("cfg4", rows, [0], gpu)
