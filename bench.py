"""Benchmark: one decode step of paged attention over the packed-FP8 KV cache.

A step is the whole path: the layer-invariant control setup, then for each of
36 layers (alternating sliding-window 128 / full, 18 shared buffers) the
quantising KV write and the paged decode attention, all through libpkv on one
stream.  Workload: batch 64, 64 query / 8 KV heads, head_dim 64, block 32,
every context 8192 tokens, random block tables, synthetic N(0,1) data.

Prints one JSON line.  `value` is the step's algorithmic KV bytes (K + V FP8
of every attended key of every layer) divided by the measured step time,
in GB/s; tokens/s is batch / step time.  The step is replayed as a HIP graph
(inputs resident in HBM); a second, eager phase issues a step's full-layer
launches back to back between two events on their stream to get the dominant
kernel's average launch duration for the roofline (window layers likewise).  `cpu_baseline` times the CPU
oracle on a bounded sample of the same workload (before the GPU timing).  `hbm_ceiling` is the best rate
of the read probes of libpkv_probe on a 4 GiB buffer: one stream, and whole
tiles of the kernel's tile size (block x head_dim bytes) in a scrambled order,
over a few launch sizes with plain and non-temporal loads.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config cfgN]
    python bench.py --calibrate-copy      # plain device copy, for counter scaling

The all-core CPU baseline starts worker processes; under a profiler that
preloads a GPU library into child processes, pass --no-cpu-baseline.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# what decides the dominant kernel's code: its sources and the build flags
KERNEL_SOURCES = ["paged_fp8_kv_amd/csrc/decode_attn.hip", "paged_fp8_kv_amd/csrc/pkv_device.hpp",
                  "paged_fp8_kv_amd/build.py"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_attn_full_cfg3_traffic.json")


def kernel_sha():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kv_bytes_per_layer(wl, kind):
    c = wl.cfg
    n = wl.seq_lens.astype(np.int64)
    if kind == "swa":
        n = np.minimum(n, c.window)
    n = np.where(wl.active > 0, n, 0)
    return int(n.sum()) * c.hkv * 2 * c.head_dim


def calibrate_copy(steps):
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "launches": steps}), flush=True)


def hbm_ceiling(dev, tile_bytes, reps=10, nbytes=1 << 32):
    """Best read rates (GB/s) of the stream and tile probes, each launch timed
    with events on torch's current stream, the one the probes launch on."""
    import torch
    from paged_fp8_kv_amd import probe as Q
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(0x5A)
    sink = torch.zeros(4096, dtype=torch.int32, device=dev)
    best = {}
    for kind in ("stream", "tiles"):
        for nt in (0, 1):
            for grid in (256, 512, 1024, 2048, 4096):
                if kind == "stream":
                    def run():
                        return Q.pkv_probe_stream_read(buf, grid, nt, sink)
                else:
                    def run():
                        return Q.pkv_probe_tile_read(buf, tile_bytes, grid, nt, sink)
                for _ in range(2):
                    n = run()
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record()
                for _ in range(reps):
                    run()
                b.record()
                torch.cuda.synchronize()
                gbs = n * reps / (a.elapsed_time(b) * 1e-3) / 1e9
                if gbs > best.get(kind, (0.0,))[0]:
                    best[kind] = (gbs, grid, nt)
    del buf
    torch.cuda.empty_cache()
    return {"stream_read_GBps": round(best["stream"][0], 1),
            "tile_read_GBps": round(best["tiles"][0], 1), "tile_bytes": tile_bytes,
            "probe_bytes": nbytes,
            "best_launch": {k: {"grid": v[1], "nontemporal": bool(v[2])} for k, v in best.items()}}


def _oracle_rows(task):
    """Worker of the all-core CPU baseline: the oracle's paged attention for
    one sequence of one full-attention layer, reading the layer's referenced
    blocks from a memory-mapped file.  Returns the KV bytes attended."""
    from threadpoolctl import threadpool_limits

    from oracle import attention as OA
    path, half, q, table, pos, block, hkv, ks, vs, sm, nbytes = task
    buf = np.memmap(path, dtype=np.uint8, mode="r")
    with threadpool_limits(1):
        OA.paged_decode_attention(q, buf[:half], buf[half:], table, pos, 0, block, hkv, ks, vs,
                                  sm, True)
    return nbytes


def _host_blocks(buf, wl):
    """Host copy of the blocks the full table references (both halves, in
    the order of their ids) and the full table relabelled onto them."""
    import torch
    c = wl.cfg
    ids = np.unique(wl.bt_full[wl.bt_full >= 0]).astype(np.int64)
    per = c.hkv * c.block * c.head_dim
    sel = buf.view(2, wl.nb, per).index_select(1, torch.from_numpy(ids).to(buf.device))
    remap = np.full(wl.nb, -1, np.int64)
    remap[ids] = np.arange(ids.size)
    table = np.where(wl.bt_full >= 0, remap[np.maximum(wl.bt_full, 0)], -1).astype(np.int32)
    return sel.cpu().numpy().reshape(-1), ids.size * per, table


def cpu_baseline(wl, bufs_dev, seconds, workers):
    """Time the oracle's paged attention over the full-attention layers of the
    step (float64 numpy, never tuned for speed), reported as KV GB/s attended.

    One core: sequence after sequence, layer after layer, for `seconds`.
    All cores: a pool of `workers` processes (spawned, CPU only) over the
    (layer, sequence) pairs of the first full layers of the step, each
    worker with one BLAS thread and the layers' referenced blocks
    memory-mapped from files; the sample is sized to about `seconds` of
    one-core work per worker.  Both run before any GPU timing."""
    import multiprocessing as mp
    import tempfile

    from threadpoolctl import threadpool_limits

    from oracle import attention as OA
    c = wl.cfg
    full_layers = [i for i, k in enumerate(c.kinds) if k == "full"]
    pos = (wl.seq_lens - 1).astype(np.int64)
    sm = 1.0 / np.sqrt(c.head_dim)
    active = [b for b in range(c.batch) if wl.active[b]]
    kv = lambda b: int(wl.seq_lens[b]) * c.hkv * 2 * c.head_dim
    # ---- one core
    done_bytes, rows, layers, dt = 0, 0, 0, 0.0
    with threadpool_limits(1):
        for layer in full_layers:
            host, half, table = _host_blocks(bufs_dev[layer // 2], wl)
            q = wl.q[layer].float().numpy().astype(np.float64)
            layers += 1
            t0 = time.perf_counter()
            for b in active:
                OA.paged_decode_attention(q, host[:half], host[half:], table, pos, 0, c.block,
                                          c.hkv, wl.k_scale[layer], wl.v_scale[layer], sm, True,
                                          rows=[b])
                done_bytes += kv(b)
                rows += 1
                if dt + time.perf_counter() - t0 >= seconds:
                    break
            dt += time.perf_counter() - t0
            del host
            if dt >= seconds:
                break
    one = {"value": round(done_bytes / dt / 1e9, 6), "unit": "GB/s", "cores": 1,
           "sample": f"{rows} sequence-layers over {layers} full-attention layers "
                     f"({done_bytes / 1e6:.1f} MB of KV) in {dt:.1f} s"}
    # ---- all cores: enough (layer, sequence) pairs for ~`seconds` per worker
    target = done_bytes / dt * seconds * workers
    tasks, staged, total = [], [], 0
    tmpdir = tempfile.mkdtemp(prefix="pkv_cpu_")
    try:
        for layer in full_layers:
            if total >= target:
                break
            host, half, table = _host_blocks(bufs_dev[layer // 2], wl)
            path = os.path.join(tmpdir, f"layer{layer}.bin")
            host.tofile(path)
            staged.append(path)
            del host
            q = wl.q[layer].float().numpy().astype(np.float64)
            for b in active:
                tasks.append((path, half, q[b:b + 1], table[b:b + 1], pos[b:b + 1], c.block,
                              c.hkv, wl.k_scale[layer], wl.v_scale[layer], sm, kv(b)))
                total += kv(b)
                if total >= target:
                    break
        with mp.get_context("spawn").Pool(workers) as pool:
            pool.map(_oracle_rows, tasks[:workers], chunksize=1)   # start the workers
            t0 = time.perf_counter()
            got = sum(pool.map(_oracle_rows, tasks, chunksize=1))
            wall = time.perf_counter() - t0
    finally:
        for pth in staged:
            os.remove(pth)
        os.rmdir(tmpdir)
    return {"value": round(got / wall / 1e9, 6), "unit": "GB/s", "cores": workers,
            "kind": "oracle",
            "sample": f"{len(tasks)} sequence-layers over {len(staged)} full-attention layers "
                      f"({got / 1e6:.1f} MB of KV) in {wall:.1f} s on {workers} worker processes "
                      f"(numpy float64, 1 BLAS thread each; the host reports {os.cpu_count()} "
                      f"CPUs)",
            "one_core": one}


def full_kernel_name(cfg, wl, args):
    """Which attention kernel the library launches for this workload's full
    layers (for the label only; the library decides on the same shapes):
    the direct kernel when no item can exceed 8 sub-tiles of 32 keys, or 32
    when the items alone fill half of the GPU's resident waves (256 CUs x 8),
    else the stream-K kernel."""
    import math
    longest = math.ceil(wl.bt_full.shape[1] * cfg.block / 32)
    items = cfg.batch * cfg.hkv
    direct = longest <= 8 or (longest <= 32 and 2 * items >= 256 * 8)
    name = "decode_attn_direct_kernel" if direct else "decode_attn_kernel"
    return (f"{name}<{cfg.block}, false, {str(args.k_layout == 'packed').lower()}, "
            f"{str(args.rope).lower()}> (full layers)")


def identity_tables(wl):
    """The control run's tables: sequence b's full-table blocks are the pool's
    ids b*W .. b*W + n - 1 (W = table width) and its window blocks follow all
    of those, so every sequence streams one contiguous region."""
    import dataclasses
    c = wl.cfg
    B, Wd = c.batch, wl.bt_full.shape[1]
    full = np.full_like(wl.bt_full, -1)
    swa = np.full_like(wl.bt_swa, -1)
    keep = int((wl.bt_swa >= 0).sum(axis=1).max()) if (wl.bt_swa >= 0).any() else 0
    if B * (Wd + keep) > wl.nb:
        raise SystemExit(f"identity tables need {B * (Wd + keep)} blocks, the pool has {wl.nb}")
    for b in range(B):
        n = int((wl.bt_full[b] >= 0).sum())
        full[b, :n] = b * Wd + np.arange(n)
        cols = np.nonzero(wl.bt_swa[b] >= 0)[0]
        swa[b, cols] = B * Wd + b * keep + np.arange(len(cols))
    ref = np.unique(np.concatenate([full[full >= 0], swa[swa >= 0]])).astype(np.int64)
    return dataclasses.replace(wl, bt_full=full.astype(np.int32), bt_swa=swa.astype(np.int32),
                               referenced=ref)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="cfg3")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="seconds of oracle work per core (one-core run, and per worker)")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="worker processes of the all-core oracle timing (default: the CPUs "
                         "this process may use, at most 16)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the HBM read probes (stream and scrambled tiles)")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--tables", choices=["padded", "csr"], default="padded",
                    help="block tables as padded rows (default) or compressed page lists")
    ap.add_argument("--k-layout", choices=["packed", "unpacked"], default="packed",
                    help="K half arrangement: packed token pairs (default) or token-major rows")
    ap.add_argument("--rope", action="store_true",
                    help="turn the queries and new keys by per-sequence rotary cos/sin")
    ap.add_argument("--control", choices=["random", "identity"], default="random",
                    help="identity: every sequence's blocks consecutive in the pool (isolates "
                         "the cost of the gather)")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="steps timed one by one after evicting the 256 MB Infinity Cache: this "
                         "many after writing and reading back 1 GiB (cold_step_ms_median) "
                         "and as many after only writing it (cold_dirty_step_ms_median); "
                         "0 = none")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the decode step is data-parallel over sequences and KV heads: each GPU would "
              f"run this step on its own share)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        calibrate_copy(max(args.steps, 1))
        return

    import paged_fp8_kv_amd as P
    import workloads as W

    dev = torch.device("cuda:0")
    cfg = W.CONFIGS[args.config]
    hbm = torch.cuda.mem_get_info(dev)[1]
    wl = W.make_workload(cfg, hbm_bytes=hbm)
    if args.control == "identity":
        wl = identity_tables(wl)
    log(f"workload {cfg.name}: nb={wl.nb}, {cfg.n_buffers} buffers of "
        f"{2 * wl.half_bytes / 1e9:.2f} GB")
    bufs = []
    for j in range(cfg.n_buffers):
        t = torch.empty(2 * wl.half_bytes, dtype=torch.uint8, device=dev)
        W.fill_buffer(t, wl, j)
        bufs.append(t)
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    seq_lens, active = to(wl.seq_lens.astype(np.int32)), to(wl.active)
    positions = to(wl.positions.astype(np.int64))
    bt_full, bt_swa = to(wl.bt_full), to(wl.bt_swa)
    q, k_new, v_new = wl.q.to(dev), wl.k_new.to(dev), wl.v_new.to(dev)
    has_swa = "swa" in cfg.kinds
    win = cfg.window if has_swa else 0
    rkw = {}
    if args.rope:
        rc, rs = W.rope_tables(wl)
        rkw = dict(rope_cos=to(rc), rope_sin=to(rs))
    if args.tables == "csr":
        # the same tables as compressed page lists; the setup writes the padded
        # full table the layers read
        Bk = cfg.block
        n_pages = -(-wl.seq_lens.astype(np.int64) // Bk)
        indptr = np.concatenate([[0], np.cumsum(n_pages)]).astype(np.int32)
        full_idx = np.concatenate([wl.bt_full[b, :n_pages[b]] for b in range(cfg.batch)]).astype(np.int32)
        swa_idx = np.concatenate([wl.bt_swa[b, :n_pages[b]] for b in range(cfg.batch)]).astype(np.int32)
        last = (wl.seq_lens - (n_pages - 1) * Bk).astype(np.int32)
        csr = (to(indptr), to(full_idx), to(swa_idx), to(last))
        ctl = P.pkv_setup_attn_control_csr(*csr, active, cfg.block, win, wl.bt_full.shape[1],
                                           positions=positions)
        bt_full = ctl["bt_full"]
    else:
        csr = None
        ctl = P.pkv_setup_attn_control(seq_lens, active, bt_full, bt_swa, cfg.block, win,
                                       positions=positions)

    def setup():
        if csr is not None:
            P.pkv_setup_attn_control_csr(*csr, active, cfg.block, win, wl.bt_full.shape[1],
                                         positions=positions, out=ctl)
        else:
            P.pkv_setup_attn_control(seq_lens, active, bt_full, bt_swa, cfg.block, win,
                                     positions=positions, out=ctl)
    tw = ctl["bt_swa_trim"].shape[1]
    ws_full = P.new_workspace(cfg.batch, cfg.hq, cfg.hkv, cfg.head_dim, cfg.block,
                              wl.bt_full.shape[1], 0, dev)
    ws_swa = P.new_workspace(cfg.batch, cfg.hq, cfg.hkv, cfg.head_dim, cfg.block, tw, win,
                             dev) if has_swa else None
    outs = [torch.empty_like(q[i]) for i in range(cfg.layers)]
    sm = 1.0 / float(np.sqrt(cfg.head_dim))
    # the layer entry point runs window layers at even and full layers at odd
    # indices (layer i on buffer i // 2): an alternating schedule maps onto it
    # as is, a lone full layer as layer 1 (the full layer of buffer 0)
    alternating = all(k == ("swa" if i % 2 == 0 else "full") for i, k in enumerate(cfg.kinds))
    lone_full = tuple(cfg.kinds) == ("full",)
    layer_id = (lambda i: i) if alternating else (lambda i: 1)
    kp = args.k_layout == "packed"
    step_desc = P.make_step(bufs, ctl, bt_full, cfg.batch, cfg.hq, cfg.hkv, cfg.head_dim,
                            cfg.block, cfg.window, wl.nb, k_packed=kp,
                            **rkw) if (alternating or lone_full) else None

    def attn(i):
        swa = cfg.kinds[i] == "swa"
        buf = bufs[i // 2]
        if swa:
            P.pkv_paged_decode_attn(q[i], buf, ctl["bt_swa_trim"], ctl["pos_swa"], cfg.block,
                                    wl.nb, cfg.window, wl.k_scale[i], wl.v_scale[i], sm, cfg.hkv,
                                    out=outs[i], workspace=ws_swa, k_packed=kp, **rkw)
        else:
            P.pkv_paged_decode_attn(q[i], buf, bt_full, ctl["pos_full"], cfg.block, wl.nb, 0,
                                    wl.k_scale[i], wl.v_scale[i], sm, cfg.hkv, out=outs[i],
                                    workspace=ws_full, k_packed=kp, **rkw)

    def update(i):
        swa = cfg.kinds[i] == "swa"
        P.pkv_kv_cache_update(bufs[i // 2], k_new[i], v_new[i],
                              ctl["upd_swa"] if swa else ctl["upd_full"], cfg.block, wl.nb,
                              wl.k_scale[i], wl.v_scale[i], k_packed=kp, **rkw)

    def layer(i):
        if step_desc is not None:
            li = layer_id(i)
            P.pkv_decode_layer(step_desc, li, q[i], k_new[i], v_new[i], wl.k_scale[i],
                               wl.v_scale[i], sm, outs[i], ws_swa if li % 2 == 0 else ws_full)
        else:
            update(i)
            attn(i)

    def step():
        setup()
        for i in range(cfg.layers):
            layer(i)

    # The CPU baseline runs before any GPU timing: besides being cheap to place
    # here, its seconds of host work let the device settle after whatever ran
    # before this process (another process freeing ~100 GB of device memory
    # was measured to slow this step by ~4% for about 20 s).
    cpu = None
    if not args.no_cpu_baseline:
        workers = args.cpu_workers or min(16, len(os.sched_getaffinity(0)))
        cpu = cpu_baseline(wl, bufs, args.cpu_seconds, workers)

    # eager warm-up; after the first step the cache holds this step's tokens,
    # so every later step recomputes identical outputs
    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]

    use_graph = not args.no_graph
    g = None
    if use_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for r in range(3):
            for o in outs:
                o.zero_()
            g.replay()
            torch.cuda.synchronize()
            if not all(torch.equal(a, b) for a, b in zip(outs, ref)):
                log("graph replay differs from the eager step; timing eagerly")
                use_graph = False
                break
        for _ in range(args.warmup):
            g.replay() if use_graph else step()
        torch.cuda.synchronize()

    # ---- timed region: whole steps (an event before each step for percentiles)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        marks[k].record()
        g.replay() if use_graph else step()
    marks[-1].record()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms = dt * 1e3 / args.steps
    per_step = np.array([marks[k].elapsed_time(marks[k + 1]) for k in range(args.steps)])

    # ---- cold steps: each after evicting the 256 MB Infinity Cache with 1 GiB of
    # other data.  `cold`: the 1 GiB is written and then read back, so that the
    # caches hold clean unrelated lines when the step starts (as after the
    # weight reads of a model's other layers).  `cold_dirty`: written only; the
    # step then also pays for writing back the dirty lines it evicts (≈ 40 us
    # more at config 3)
    cold, cold_dirty = [], []
    if args.cold_steps > 0:
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        for k in range(2 * args.cold_steps):
            clean = k % 2 == 0
            scratch.fill_(k & 0xff)
            if clean:
                scratch.view(torch.int64).sum()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay() if use_graph else step()
            b.record()
            torch.cuda.synchronize()
            (cold if clean else cold_dirty).append(a.elapsed_time(b))
        del scratch

    # ---- dominant kernel: the full-layer launches of a step, made exactly as the
    # step makes them but back to back between two events on their stream (the
    # layers of a step are independent), so the average is the launch duration
    # plus the gap between consecutive launches; the same for the window layers,
    # issued right behind the full ones so that the device is still busy when
    # they are queued.  The host needs about 7 us to issue a launch: a group of
    # launches shorter than that would be timed with the host's gaps, so short
    # groups are issued 16 times over between their events.  Long launches are
    # not repeated: after a few milliseconds of back-to-back full layers the
    # same launch was measured up to 25% slower (the device's clocks drop
    # under sustained load).  When a step has fewer than 4 full layers, a
    # first timed pass decides whether they are short, and each timed group is
    # preceded by an untimed pass so that the host's first launch is queued
    # while the device is busy.
    full_layers = [i for i, k in enumerate(cfg.kinds) if k == "full"]
    swa_layers = [i for i, k in enumerate(cfg.kinds) if k == "swa"]
    ev = {"full": [], "swa": []}

    def timed(group, reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            for i in group:
                layer(i)
        b.record()
        return a, b

    torch.cuda.synchronize()
    reps_full = 1
    if 0 < len(full_layers) < 4:
        setup()
        for i in full_layers:  # untimed lead, as below
            layer(i)
        la, lb = timed(full_layers, 1)
        lb.synchronize()
        if la.elapsed_time(lb) * 1e3 / len(full_layers) < 60.0:
            reps_full = -(-16 // len(full_layers))
    for _ in range(max(1, min(args.steps, 5))):
        setup()
        if 0 < len(full_layers) < 4:
            for i in full_layers:  # untimed: the queue stays ahead of the device
                layer(i)
        if full_layers:
            a, b = timed(full_layers, reps_full)
            ev["full"].append((a, b, reps_full * len(full_layers)))
        if swa_layers:
            reps = -(-16 // len(swa_layers))
            a, b = timed(swa_layers, reps)
            ev["swa"].append((a, b, reps * len(swa_layers)))
    torch.cuda.synchronize()
    full_us = float(np.mean([a.elapsed_time(b) / n for a, b, n in ev["full"]])) * 1e3
    swa_us = float(np.mean([a.elapsed_time(b) / n for a, b, n in ev["swa"]])) * 1e3 if ev["swa"] else None
    for a, b in zip(outs, ref):
        assert torch.equal(a, b), "outputs changed between steps"

    step_bytes = sum(kv_bytes_per_layer(wl, k) for k in cfg.kinds)
    full_bytes = kv_bytes_per_layer(wl, "full")
    achieved = full_bytes / (full_us * 1e-6) / 1e9
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        tr = json.load(open(TRAFFIC_FILE))
        if (tr.get("kernel_sha") == kernel_sha() and tr.get("config") == args.config
                and args.k_layout == "packed" and args.tables == "padded" and not args.rope
                and args.control == "random"):
            traffic = tr.get("bytes_per_launch")
    value = step_bytes / (ms * 1e-3) / 1e9
    result = {
        "metric": "decode-attention KV GB/s (% of HBM peak) and tokens/s/GPU at batch 64",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3-kv/bf16-q/fp32-acc",
        "data": "synthetic (seeded N(0,1) activations, FP8 history, random block tables)",
        "config": {"workload": cfg.name, "layers": cfg.layers, "batch": cfg.batch,
                   "q_heads": cfg.hq, "kv_heads": cfg.hkv, "head_dim": cfg.head_dim,
                   "block": cfg.block, "context": str(cfg.ctx[1]) if cfg.ctx[0] == "fixed" else str(cfg.ctx),
                   "window": cfg.window, "num_blocks": wl.nb, "k_layout": args.k_layout, "tables": args.tables,
                   "rope": args.rope, "control": args.control, "graph": use_graph},
        "tokens_per_s": round(cfg.batch / (ms * 1e-3), 1),
        "step_ms_p10_p50_p90": [round(float(np.percentile(per_step, p)), 4) for p in (10, 50, 90)],
        "cold_step_ms_median": round(float(np.median(cold)), 4) if cold else None,
        "cold_dirty_step_ms_median": round(float(np.median(cold_dirty)), 4) if cold_dirty else None,
        "hbm_frac_step": round(value / HBM_PEAK_GBS, 4),
        "kv_bytes_per_step": step_bytes,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": full_kernel_name(cfg, wl, args),
                     "bytes_per_launch": full_bytes, "avg_launch_us": round(full_us, 2),
                     "swa_avg_launch_us": round(swa_us, 2) if swa_us else None},
        "hbm_ceiling": None,
        "cpu_baseline": None,
    }
    if not args.no_ceiling:
        ceil = hbm_ceiling(dev, cfg.block * cfg.head_dim)
        ceil["full_layer_frac_of_stream"] = round(achieved / ceil["stream_read_GBps"], 4)
        ceil["full_layer_frac_of_tiles"] = round(achieved / ceil["tile_read_GBps"], 4)
        result["hbm_ceiling"] = ceil
    result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
