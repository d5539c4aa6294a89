"""Parity of the HIP path (through the C ABI) against the CPU oracle."""
import numpy as np
import pytest
import torch

import paged_fp8_kv_amd as P
import workloads as W
from gpu_harness import (alternating, assert_close, device_inputs, gpu_step, oracle_step,
                         packed_to_unpacked, poison_stale)
from oracle import control as OC
from oracle import fp8_e4m3 as OF
from oracle import update as OU

pytestmark = pytest.mark.gpu


def _small_case(name, gpu):
    wl = W.make_workload(W.CONFIGS[name])
    host = W.make_buffers(wl, "cpu")
    poison_stale(host, wl)
    snaps = [h.numpy().copy() for h in host]
    bufs = [h.to(gpu) for h in host]
    return wl, bufs, snaps


@pytest.mark.parametrize("name", ["cfg1", "cfg2", "cfg5"])
def test_step_matches_oracle(name, gpu):
    print(f"[parity] {name}", flush=True)
    wl, bufs, snaps = _small_case(name, gpu)
    outs, ctl = gpu_step(wl, bufs, gpu)
    ref, ref_ctl = oracle_step(wl, snaps)
    for i in range(wl.cfg.layers):
        assert_close(outs[i], ref[i], f"{name} layer {i}")
    # the KV writes and everything else in every buffer: bit-exact
    for j, b in enumerate(bufs):
        got = b.cpu().numpy()
        assert np.array_equal(got, snaps[j]), f"{name} buffer {j}: {int((got != snaps[j]).sum())} bytes differ"
    # the control itself
    for key in ("pos_full", "upd_full", "pos_abs"):
        assert np.array_equal(ctl[key].cpu().numpy(), ref_ctl[key] if key != "pos_abs" else
                              OC.attention_control(wl.seq_lens, wl.active, wl.bt_full, wl.bt_swa,
                                                   wl.cfg.block, wl.cfg.window,
                                                   positions=wl.positions)["pos_abs"]), key
    if "swa" in wl.cfg.kinds:
        for key in ("pos_swa", "upd_swa", "bt_swa_trim"):
            assert np.array_equal(ctl[key].cpu().numpy(), ref_ctl[key]), key


def test_step_direct_calls_equal_layer_api(gpu):
    """The per-call path and the layer-schedule entry point give identical bytes."""
    wl, bufs, snaps = _small_case("cfg2", gpu)
    bufs2 = [b.clone() for b in bufs]
    a, _ = gpu_step(wl, bufs, gpu, use_layer_api=True)
    b, _ = gpu_step(wl, bufs2, gpu, use_layer_api=False)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    for x, y in zip(bufs, bufs2):
        assert torch.equal(x, y)


def test_repeat_runs_are_bitwise_identical(gpu):
    wl, bufs, _ = _small_case("cfg5", gpu)
    bufs2 = [b.clone() for b in bufs]
    a, _ = gpu_step(wl, bufs, gpu)
    b, _ = gpu_step(wl, bufs2, gpu)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("scale", [1.0, 0.0173])
def test_kv_write_every_bf16_pattern(scale, gpu):
    """All 65536 bf16 bit patterns through the device quantiser, bit-exact."""
    B, H, D, Bk, nb = 128, 8, 64, 16, 130
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    k_new = bits.reshape(B, H, D)
    v_new = bits.flip(0).reshape(B, H, D)
    slots = (torch.arange(B, dtype=torch.int64) * Bk + (torch.arange(B) % Bk))
    half, total = P.pkv_kv_buffer_bytes(nb, H, Bk, D)
    host = torch.full((total,), 0x5A, dtype=torch.uint8)
    buf = host.to(gpu)
    P.pkv_kv_cache_update(buf, k_new.to(gpu), v_new.to(gpu), slots.to(gpu), Bk, nb, scale, scale)
    torch.cuda.synchronize()
    ref = host.numpy().copy()
    OU.kv_cache_update(ref[:half], ref[half:], k_new.float().numpy(), v_new.float().numpy(),
                       slots.numpy(), Bk, scale, scale, True)
    got = buf.cpu().numpy()
    assert np.array_equal(got, ref), f"{int((got != ref).sum())} bytes differ"


def test_device_dequant_covers_all_codes(gpu):
    """Single-token sequences return their V row: every E4M3 code read back exactly."""
    B, H, Hq, D, Bk, nb = 4, 1, 8, 64, 16, 8
    half, total = P.pkv_kv_buffer_bytes(nb, H, Bk, D)
    buf = torch.zeros(total, dtype=torch.uint8)
    codes = torch.arange(256, dtype=torch.uint8).reshape(B, D)
    table = torch.arange(B, dtype=torch.int32).reshape(B, 1) * 2
    for b in range(B):
        blk = int(table[b, 0])
        buf[half + blk * Bk * D: half + blk * Bk * D + D] = codes[b]
    q = torch.randn(B, Hq, D).to(torch.bfloat16)
    pos = torch.zeros(B, dtype=torch.int32)
    out = P.pkv_paged_decode_attn(q.to(gpu), buf.to(gpu), table.to(gpu), pos.to(gpu), Bk, nb, 0,
                                  1.0, 1.0, 0.125, H)
    torch.cuda.synchronize()
    ref = OF.decode(codes.numpy())
    got = out.float().cpu().numpy()
    for g in range(Hq):
        gg = got[:, g, :]
        assert np.array_equal(np.isnan(gg), np.isnan(ref))
        fin = ~np.isnan(ref)
        assert np.array_equal(gg[fin], ref[fin])


def test_window_equals_full_when_contexts_fit(gpu):
    """Bitwise: with every context <= 128 keys, the window and full paths agree."""
    rng = np.random.default_rng(11)
    B, Hq, H, D, Bk = 16, 64, 8, 64, 32
    L = rng.integers(1, 129, size=B).astype(np.int32)
    nb = 64
    perm = rng.permutation(nb)[: B * 4].reshape(B, 4).astype(np.int32)
    half, total = P.pkv_kv_buffer_bytes(nb, H, Bk, D)
    buf = torch.from_numpy(rng.integers(0, 0x7F, size=total, dtype=np.uint8)).to(gpu)
    q = torch.randn(B, Hq, D).to(torch.bfloat16).to(gpu)
    d = dict(seq_lens=torch.from_numpy(L).to(gpu), active=torch.ones(B, dtype=torch.uint8, device=gpu),
             bt=torch.from_numpy(perm).to(gpu))
    ctl = P.pkv_setup_attn_control(d["seq_lens"], d["active"], d["bt"], d["bt"], Bk, 128)
    full = P.pkv_paged_decode_attn(q, buf, d["bt"], ctl["pos_full"], Bk, nb, 0, 0.125, 0.0625, 0.125, H)
    swa = P.pkv_paged_decode_attn(q, buf, ctl["bt_swa_trim"], ctl["pos_swa"], Bk, nb, 128, 0.125,
                                  0.0625, 0.125, H)
    torch.cuda.synchronize()
    assert torch.equal(full, swa)


def test_block_relabelling_is_bitwise_invisible(gpu):
    wl = W.make_workload(W.CONFIGS["cfg2"])
    c = wl.cfg
    host = W.make_buffers(wl, "cpu")[0]
    rng = np.random.default_rng(3)
    relabel = rng.permutation(wl.nb)
    per = c.hkv * c.block * c.head_dim
    halves = host.view(2, wl.nb, per)
    moved = torch.empty_like(halves)
    moved[:, torch.from_numpy(relabel)] = halves
    t2 = np.where(wl.bt_full >= 0, relabel[np.maximum(wl.bt_full, 0)], -1).astype(np.int32)
    pos = torch.from_numpy(wl.seq_lens - 1).to(gpu)
    q = wl.q[1].to(gpu)
    a = P.pkv_paged_decode_attn(q, host.to(gpu), torch.from_numpy(wl.bt_full).to(gpu), pos,
                                c.block, wl.nb, 0, 0.125, 0.0625, 0.125, c.hkv)
    b = P.pkv_paged_decode_attn(q, moved.reshape(-1).to(gpu), torch.from_numpy(t2).to(gpu), pos,
                                c.block, wl.nb, 0, 0.125, 0.0625, 0.125, c.hkv)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_bad_ids_and_positions_give_nan_not_faults(gpu):
    rng = np.random.default_rng(5)
    B, Hq, H, D, Bk, nb = 4, 8, 1, 64, 16, 16
    half, total = P.pkv_kv_buffer_bytes(nb, H, Bk, D)
    buf = torch.from_numpy(rng.integers(0, 0x7F, size=total, dtype=np.uint8)).to(gpu)
    table = torch.tensor([[0, 1], [2, 99], [4, -3], [6, 7]], dtype=torch.int32, device=gpu)
    pos = torch.tensor([20, 20, 20, 40], dtype=torch.int32, device=gpu)   # row 3 beyond the table
    q = torch.randn(B, Hq, D).to(torch.bfloat16).to(gpu)
    out = P.pkv_paged_decode_attn(q, buf, table, pos, Bk, nb, 0, 0.125, 0.0625, 0.125, H)
    torch.cuda.synchronize()
    o = out.float().cpu()
    assert torch.isfinite(o[0]).all()
    assert torch.isnan(o[1]).all() and torch.isnan(o[2]).all() and torch.isnan(o[3]).all()


def test_workspace_too_small_is_rejected(gpu):
    wl = W.make_workload(W.CONFIGS["cfg1"])
    buf = W.make_buffers(wl, "cpu")[0].to(gpu)
    q = wl.q[0].to(gpu)
    pos = torch.from_numpy(wl.seq_lens - 1).to(gpu)
    ws = torch.zeros(256, dtype=torch.uint8, device=gpu)
    with pytest.raises(P.PkvError) as e:
        P.pkv_paged_decode_attn(q, buf, torch.from_numpy(wl.bt_full).to(gpu), pos, 16, wl.nb, 0,
                                0.125, 0.125, 0.125, 1, workspace=ws)
    assert e.value.status == P.PKV_ERR_WORKSPACE


def test_validate_attn_control(gpu):
    wl = W.make_workload(W.CONFIGS["cfg5"])
    d = device_inputs(wl, gpu)
    P.pkv_validate_attn_control(d["seq_lens"], d["active"], d["bt_full"], d["bt_swa"],
                                wl.cfg.block, wl.cfg.window, wl.nb)
    bad = wl.bt_swa.copy()
    b = int(np.flatnonzero(wl.active)[0])
    c = (int(wl.seq_lens[b]) - 1) // wl.cfg.block
    bad[b, c] = wl.bt_full[b, 0]
    with pytest.raises(P.PkvError) as e:
        P.pkv_validate_attn_control(d["seq_lens"], d["active"], d["bt_full"],
                                    torch.from_numpy(bad).to(gpu), wl.cfg.block, wl.cfg.window, wl.nb)
    assert e.value.status == P.PKV_ERR_DATA


def _small_case_unpacked(name, gpu):
    wl = W.make_workload(W.CONFIGS[name])
    host = W.make_buffers(wl, "cpu")
    poison_stale(host, wl, k_packed=False)
    snaps = [h.numpy().copy() for h in host]
    return wl, [h.to(gpu) for h in host], snaps


@pytest.mark.parametrize("name", ["cfg1", "cfg2", "cfg5"])
def test_step_matches_oracle_unpacked_k(name, gpu):
    """Token-major K rows (the unpacked arrangement): the same step against
    the oracle reading K through the plain offsets."""
    print(f"[parity unpacked K] {name}", flush=True)
    wl, bufs, snaps = _small_case_unpacked(name, gpu)
    outs, _ = gpu_step(wl, bufs, gpu, k_packed=False)
    ref, _ = oracle_step(wl, snaps, k_packed=False)
    for i in range(wl.cfg.layers):
        assert_close(outs[i], ref[i], f"{name} unpacked layer {i}")
    for j, b in enumerate(bufs):
        got = b.cpu().numpy()
        assert np.array_equal(got, snaps[j]), f"{name} buffer {j}: {int((got != snaps[j]).sum())} bytes differ"


@pytest.mark.parametrize("name", ["cfg2", "cfg5"])
def test_packed_and_unpacked_k_agree_bitwise(name, gpu):
    """One cache in both K arrangements: identical outputs bit for bit, and
    the written caches are the same bytes up to the arrangement."""
    wl, bufs, _ = _small_case(name, gpu)
    unp = [packed_to_unpacked(b, wl) for b in bufs]
    a, _ = gpu_step(wl, bufs, gpu)
    b, _ = gpu_step(wl, unp, gpu, k_packed=False)
    for x, y in zip(a, b):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    for x, y in zip(bufs, unp):
        assert torch.equal(packed_to_unpacked(x, wl), y)


@pytest.mark.parametrize("name", ["cfg1", "cfg2", "cfg5"])
def test_step_matches_oracle_at_non_power_of_two_scales(name, gpu):
    """k_scale 0.0173 and v_scale 0.0411 (not powers of two, so the
    quantising division rounds and the scales do not factor out exactly)."""
    import dataclasses
    print(f"[parity scales] {name}", flush=True)
    wl, bufs, snaps = _small_case(name, gpu)
    n = wl.cfg.layers
    wl = dataclasses.replace(wl, k_scale=[0.0173] * n, v_scale=[0.0411] * n)
    outs, _ = gpu_step(wl, bufs, gpu)
    ref, _ = oracle_step(wl, snaps)
    for i in range(n):
        assert_close(outs[i], ref[i], f"{name} scales layer {i}")
    for j, b in enumerate(bufs):
        got = b.cpu().numpy()
        assert np.array_equal(got, snaps[j]), f"{name} buffer {j}: {int((got != snaps[j]).sum())} bytes differ"
