"""Pins of the oracle's layer schedule (CPU only).

"GPT-OSS-120B giga-kernel decode", section "Kernel contract": even layers are
sliding-window (128) and odd layers full; a layer picks its block table and
write index by ``i % 2`` and its buffer by ``i // 2``.  The step below is
built so that every way of getting that wrong changes a result: the window
blocks and the full blocks of a sequence hold *different* histories, contexts
exceed the window, the two buffers hold different histories, and every layer
has its own new token.  Expected values are written from the definition with
torch views of the printed layout (``paged_build``) and ``math.fsum``
(``oracle.attention.dense_attention``), not through the oracle's gather.
"""
import numpy as np
import pytest
import torch

from oracle import attention as OA
from oracle import step as OS
from paged_build import bf16_values, build_halves, random_codes, torch_decode

NB, H, G, BK, D, W = 64, 1, 2, 16, 64, 128
HQ = H * G
LENS = np.array([300, 150])          # both beyond the window; 150 ends mid-block
K_SCALE, V_SCALE = [0.125, 0.25, 0.0625, 0.125], [0.0625, 0.125, 0.25, 0.0625]
SM = 0.125


def _tables():
    """Full blocks 0.., window blocks 40.. (disjoint); the window table only
    holds the last blocks of each sequence (older ones were freed)."""
    B = LENS.size
    width = -(-int(LENS.max()) // BK)
    bt_full = np.full((B, width), -1, np.int32)
    bt_swa = np.full((B, width), -1, np.int32)
    nxt_f, nxt_s = 0, 40
    for b, L in enumerate(LENS):
        n = -(-int(L) // BK)
        bt_full[b, :n] = np.arange(nxt_f, nxt_f + n)
        nxt_f += n
        keep = -(-(W + BK) // BK)
        first = max(0, n - keep)
        bt_swa[b, first:n] = np.arange(nxt_s, nxt_s + n - first)
        nxt_s += n - first
    assert nxt_f <= 40 and nxt_s <= NB
    return bt_full, bt_swa


def _make():
    rng = np.random.default_rng(11)
    bt_full, bt_swa = _tables()
    # per buffer: a full-table history and a different window-table history
    hist = []
    bufs = []
    for j in range(2):
        kf = [random_codes(rng, (int(L), H, D), 1 / 8) for L in LENS]
        vf = [random_codes(rng, (int(L), H, D), 1 / 8) for L in LENS]
        ks = [random_codes(rng, (int(L), H, D), 1 / 8) for L in LENS]
        vs = [random_codes(rng, (int(L), H, D), 1 / 8) for L in LENS]
        kh, vh = build_halves(kf, vf, [bt_full[b] for b in range(LENS.size)], NB, H, BK, D)
        # window blocks: laid over the same halves (disjoint block ids);
        # only the logical blocks the window table keeps are written
        kt = torch.from_numpy(kh).view(NB, H, BK // 2, D, 2)
        vt = torch.from_numpy(vh).view(NB, H, BK, D)
        for b in range(LENS.size):
            for t in range(int(LENS[b])):
                blk = int(bt_swa[b, t // BK])
                if blk < 0:
                    continue
                s = t % BK
                kt[blk, :, s // 2, :, s % 2] = torch.from_numpy(ks[b][t])
                vt[blk, :, s, :] = torch.from_numpy(vs[b][t])
        bufs.append((kh, vh))
        hist.append(dict(full=(kf, vf), swa=(ks, vs)))
    q = [bf16_values(rng, (LENS.size, HQ, D)) for _ in range(4)]
    kn = [bf16_values(rng, (LENS.size, H, D)) for _ in range(4)]
    vn = [bf16_values(rng, (LENS.size, H, D)) for _ in range(4)]
    return bt_full, bt_swa, bufs, hist, q, kn, vn


def _cast(x, scale):
    t = torch.from_numpy(np.asarray(x, np.float32)) / torch.tensor(scale, dtype=torch.float32)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _expected(layer, b, g, hist, q, kn, vn):
    """Dense attention of layer `layer`, sequence b, query head g, written out
    from the schedule the page states."""
    window = layer % 2 == 0
    kc, vc = hist[layer // 2]["swa" if window else "full"]
    p = int(LENS[b]) - 1
    lo = max(0, p - W + 1) if window else 0
    h = g // G
    krows = [torch_decode(kc[b][t, h]) * K_SCALE[layer] for t in range(lo, p)]
    vrows = [torch_decode(vc[b][t, h]) * V_SCALE[layer] for t in range(lo, p)]
    krows.append(torch_decode(_cast(kn[layer][b, h], K_SCALE[layer])) * K_SCALE[layer])
    vrows.append(torch_decode(_cast(vn[layer][b, h], V_SCALE[layer])) * V_SCALE[layer])
    return np.array(OA.dense_attention(list(q[layer][b, g]), [list(r) for r in krows],
                                       [list(r) for r in vrows], SM))


def _run(n_layers, bufs, bt_full, bt_swa, q, kn, vn):
    work = [(k.copy(), v.copy()) for k, v in bufs]
    outs, ctl = OS.decode_step(work, q[:n_layers], kn[:n_layers], vn[:n_layers], LENS,
                               np.ones(LENS.size, np.uint8), bt_full, bt_swa, BK, H, W,
                               K_SCALE[:n_layers], V_SCALE[:n_layers], SM)
    return outs, ctl, work


def test_each_layer_attends_its_own_table_window_and_buffer():
    bt_full, bt_swa, bufs, hist, q, kn, vn = _make()
    outs, _, _ = _run(4, bufs, bt_full, bt_swa, q, kn, vn)
    assert sorted(outs) == [0, 1, 2, 3]
    for layer in range(4):
        for b in range(LENS.size):
            for g in range(HQ):
                want = _expected(layer, b, g, hist, q, kn, vn)
                got = outs[layer][b, g]
                assert np.allclose(got, want, rtol=1e-12, atol=1e-12), (layer, b, g)


def test_each_layer_writes_exactly_its_own_slot():
    """Run the step one more layer at a time: layer i changes only buffer
    i // 2, and only the new token's slot in the window table (i even) or the
    full table (i odd), with the codes of its own new K/V."""
    bt_full, bt_swa, bufs, hist, q, kn, vn = _make()
    prev = [(k.copy(), v.copy()) for k, v in bufs]
    for n in range(1, 5):
        _, _, now = _run(n, bufs, bt_full, bt_swa, q, kn, vn)
        i = n - 1
        table = bt_swa if i % 2 == 0 else bt_full
        for j in range(2):
            for half in range(2):
                changed = np.flatnonzero(now[j][half] != prev[j][half])
                if j != i // 2:
                    assert changed.size == 0, (i, j, half)
        kt = torch.from_numpy(now[i // 2][0]).view(NB, H, BK // 2, D, 2)
        vt = torch.from_numpy(now[i // 2][1]).view(NB, H, BK, D)
        expect_k = np.array(prev[i // 2][0])
        expect_v = np.array(prev[i // 2][1])
        ek = torch.from_numpy(expect_k).view(NB, H, BK // 2, D, 2)
        ev = torch.from_numpy(expect_v).view(NB, H, BK, D)
        for b in range(LENS.size):
            p = int(LENS[b]) - 1
            blk, s = int(table[b, p // BK]), p % BK
            ek[blk, :, s // 2, :, s % 2] = torch.from_numpy(_cast(kn[i][b], K_SCALE[i]))
            ev[blk, :, s, :] = torch.from_numpy(_cast(vn[i][b], V_SCALE[i]))
        assert torch.equal(kt, ek) and torch.equal(vt, ev), i
        prev = now


def test_explicit_kinds_equal_the_default_schedule():
    bt_full, bt_swa, bufs, hist, q, kn, vn = _make()
    a, _, wa = _run(4, bufs, bt_full, bt_swa, q, kn, vn)
    work = [(k.copy(), v.copy()) for k, v in bufs]
    b_, _ = OS.decode_step(work, q, kn, vn, LENS, np.ones(LENS.size, np.uint8), bt_full, bt_swa,
                           BK, H, W, K_SCALE, V_SCALE, SM, kinds=["swa", "full", "swa", "full"])
    for i in range(4):
        assert np.array_equal(a[i], b_[i])
    for (k1, v1), (k2, v2) in zip(wa, work):
        assert np.array_equal(k1, k2) and np.array_equal(v1, v2)


@pytest.mark.parametrize("mistake", ["swap_parity", "full_table_for_window", "pos_full_for_window",
                                     "buffer_by_layer"])
def test_planted_schedule_mistakes_are_caught(mistake, monkeypatch):
    """A copy of the schedule with one planted mistake (in the oracle, on the
    CPU) must fail the dense comparison above."""
    bt_full, bt_swa, bufs, hist, q, kn, vn = _make()
    from oracle import attention, control, update

    def bad_step(buffers, q_, k_new, v_new, seq_lens, active, bt_f, bt_s, block, kv_heads, window,
                 k_scale, v_scale, sm_scale, k_packed=True, layers=None, kinds=None,
                 rope_cos=None, rope_sin=None):
        ctl = control.attention_control(seq_lens, active, bt_f, bt_s, block, window)
        outs = {}
        for i in range(len(q_)):
            j = min(i, len(buffers) - 1) if mistake == "buffer_by_layer" else i // 2
            k_half, v_half = buffers[j]
            swa = (i % 2 == 1) if mistake == "swap_parity" else (i % 2 == 0)
            slots = ctl["upd_swa"] if swa else ctl["upd_full"]
            update.kv_cache_update(k_half, v_half, np.asarray(k_new[i]), np.asarray(v_new[i]),
                                   slots, block, k_scale[i], v_scale[i], k_packed)
            table = ctl["bt_swa_trim"] if swa and mistake != "full_table_for_window" else bt_f
            pos = ctl["pos_swa"] if swa and mistake != "pos_full_for_window" else ctl["pos_full"]
            if swa and mistake == "full_table_for_window":
                pos = ctl["pos_full"]
            outs[i] = attention.paged_decode_attention(q_[i], k_half, v_half, table, pos,
                                                       window if swa else 0, block, kv_heads,
                                                       k_scale[i], v_scale[i], sm_scale, k_packed)
        return outs, ctl

    monkeypatch.setattr(OS, "decode_step", bad_step)
    with np.errstate(all="ignore"):
        try:
            outs, _, _ = _run(4, bufs, bt_full, bt_swa, q, kn, vn)
        except (ValueError, IndexError):
            return  # the mistake reads a missing block: caught
    mism = 0
    for layer in range(4):
        for b in range(LENS.size):
            for g in range(HQ):
                want = _expected(layer, b, g, hist, q, kn, vn)
                if not np.allclose(outs[layer][b, g], want, rtol=1e-12, atol=1e-12):
                    mism += 1
    assert mism > 0, mistake
