"""Wide score ranges, on the GPU against the oracle.

With N(0,1) queries the scores of the benchmark workloads span a few units,
so the online softmax rarely meets a new running maximum far above the old
one and the weights stay spread over many keys.  Scaling the queries by 8,
32 and 128 (still exact in bf16) widens the scores to tens and hundreds of
units: the running maximum jumps often and by far more than the lazy-rescale
slack, the weights of most keys underflow to zero, and the output approaches
the value rows of the best few keys.  Each case runs the window/full layer
pair through the layer entry point; the cache is compared byte for byte and
the outputs within the benchmark spec's tolerance and the tight element-wise
guard with an absolute part derived for this case.  The kernel feeds the
softmax weights to the PV product in fp16: a weight p (at most 2^8 under the
lazy rescale; the sum l is at least 1) is off by at most 2^-11 p when
normal, and by at most 2^-25 when it falls into or below the fp16
subnormals.  Divided by l, the first term is at most 2^-11 times the exact
weighted mean of |V| (from the oracle), and the second at most 2^-25 *
sum_t |v_t|, below 2^-11 for these contexts (at most 4096 keys whose |v|
average about 0.8, so the sum stays under 2^14 with room to spare).  So
the floor is 2^-11 * (mean |V| + 1): with weights on a few keys the mean is
the size of those keys' values, and weights far below the best one are
dropped by the fp16 underflow."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as W
from gpu_harness import assert_close, gpu_step, oracle_step, poison_stale, value_magnitude

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("mult", [8, 32, 128])
@pytest.mark.parametrize("name", ["cfg2", "cfg5"])
def test_wide_score_ranges_match_oracle(name, mult, gpu):
    wl = W.make_workload(W.CONFIGS[name])
    wl = dataclasses.replace(wl, q=(wl.q.float() * mult).to(torch.bfloat16))
    host = W.make_buffers(wl, "cpu")
    poison_stale(host, wl)
    snaps = [h.numpy().copy() for h in host]
    mag = value_magnitude(wl, snaps)
    bufs = [h.to(gpu) for h in host]
    print(f"[numerics] {name} q x{mult}", flush=True)
    outs, _ = gpu_step(wl, bufs, gpu)
    ref, _ = oracle_step(wl, snaps)
    for j, b in enumerate(bufs):
        got = b.cpu().numpy()
        assert np.array_equal(got, snaps[j]), f"buffer {j}"
    for i in range(wl.cfg.layers):
        assert_close(outs[i], ref[i], f"{name} q x{mult} layer {i}",
                     floor=2.0 ** -11 * (mag[i] + 1.0))
