"""Test plumbing shared by the GPU parity tests: build a workload, poison the
slots no key may read, run one decode step through libpkv and the same step
through the oracle on a pre-step snapshot, and compare.

Nothing here computes any part of the method: the HIP path runs through the
C ABI, the expected values come from ``oracle``."""
import numpy as np
import torch

import paged_fp8_kv_amd as P
import workloads as W
from oracle import attention as OA
from oracle import control as OC
from oracle import layout as OL
from oracle import step as OS
from oracle import update as OU

ATOL, RTOL = 2e-3, 1e-2


def alternating(cfg):
    return all(k == ("swa" if i % 2 == 0 else "full") for i, k in enumerate(cfg.kinds))


def stale_offsets(wl, per_blk_tokens, k_packed=True):
    """Byte offsets (K half, V half) of every slot of a referenced block that no
    key of this step reads: slots from the new token onward in the last block
    of each table, and window-table slots outside [p - W + 1, p].  The new
    token's own slot is included (it is written before it is read)."""
    cfg = wl.cfg
    Bk, H, D = cfg.block, cfg.hkv, cfg.head_dim
    blks, toks = [], []
    for b in range(cfg.batch):
        L = int(wl.seq_lens[b])
        p = L - 1
        for c in range(-(-L // Bk)):
            blk = int(wl.bt_full[b, c])
            for t in range(Bk):
                if c * Bk + t >= p:
                    blks.append(blk); toks.append(t)
            if "swa" in cfg.kinds and wl.bt_swa[b, c] >= 0:
                blk = int(wl.bt_swa[b, c])
                for t in range(Bk):
                    tok = c * Bk + t
                    if tok >= p or tok < p - cfg.window + 1:
                        blks.append(blk); toks.append(t)
    blks = np.array(blks, dtype=np.int64)[:, None, None]
    toks = np.array(toks, dtype=np.int64)[:, None, None]
    hh = np.arange(H)[None, :, None]
    jj = np.arange(D)[None, None, :]
    ko = OL.k_offset(blks, hh, toks, jj, H, Bk, D, k_packed).ravel()
    vo = OL.v_offset(blks, hh, toks, jj, H, Bk, D).ravel()
    return ko, vo


def poison_stale(bufs, wl, k_packed=True):
    ko, vo = stale_offsets(wl, None, k_packed)
    half = wl.half_bytes
    for buf in bufs:
        k = buf[:half]
        v = buf[half:]
        k[torch.from_numpy(ko).to(buf.device)] = W.POISON
        v[torch.from_numpy(vo).to(buf.device)] = W.POISON


def device_inputs(wl, dev):
    c = wl.cfg
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return dict(seq_lens=t(wl.seq_lens.astype(np.int32)), active=t(wl.active),
                positions=t(wl.positions.astype(np.int64)), bt_full=t(wl.bt_full),
                bt_swa=t(wl.bt_swa), q=wl.q.to(dev), k_new=wl.k_new.to(dev),
                v_new=wl.v_new.to(dev))


def gpu_step(wl, bufs, dev, use_layer_api=True, workspaces=None, k_packed=True, rope=None):
    """Run setup + every layer on the GPU; returns (outputs list, control dict).
    rope: optional (cos, sin) float32 numpy [B, D/2] rotation of the step."""
    c = wl.cfg
    d = device_inputs(wl, dev)
    rc, rs = (None, None) if rope is None else (torch.from_numpy(rope[0]).to(dev),
                                                 torch.from_numpy(rope[1]).to(dev))
    win = c.window if "swa" in c.kinds else 0
    ctl = P.pkv_setup_attn_control(d["seq_lens"], d["active"], d["bt_full"], d["bt_swa"],
                                   c.block, win, positions=d["positions"])
    sm = 1.0 / np.sqrt(c.head_dim)
    tw = ctl["bt_swa_trim"].shape[1]
    ws_full = P.new_workspace(c.batch, c.hq, c.hkv, c.head_dim, c.block, wl.bt_full.shape[1], 0, dev)
    ws_swa = P.new_workspace(c.batch, c.hq, c.hkv, c.head_dim, c.block, tw, win, dev) if win else None
    outs = []
    if use_layer_api and alternating(c):
        step = P.make_step(bufs, ctl, d["bt_full"], c.batch, c.hq, c.hkv, c.head_dim, c.block,
                           c.window, wl.nb, k_packed=k_packed, rope_cos=rc, rope_sin=rs)
        for i in range(c.layers):
            out = torch.empty_like(d["q"][i])
            ws = ws_swa if i % 2 == 0 else ws_full
            P.pkv_decode_layer(step, i, d["q"][i], d["k_new"][i], d["v_new"][i], wl.k_scale[i],
                               wl.v_scale[i], sm, out, ws)
            outs.append(out)
    else:
        for i, kind in enumerate(c.kinds):
            buf = bufs[i // 2]
            swa = kind == "swa"
            P.pkv_kv_cache_update(buf, d["k_new"][i], d["v_new"][i],
                                  ctl["upd_swa"] if swa else ctl["upd_full"], c.block, wl.nb,
                                  wl.k_scale[i], wl.v_scale[i], k_packed=k_packed,
                                  rope_cos=rc, rope_sin=rs)
            if swa:
                out = P.pkv_paged_decode_attn(d["q"][i], buf, ctl["bt_swa_trim"], ctl["pos_swa"],
                                              c.block, wl.nb, c.window, wl.k_scale[i],
                                              wl.v_scale[i], sm, c.hkv, workspace=ws_swa,
                                              k_packed=k_packed, rope_cos=rc, rope_sin=rs)
            else:
                out = P.pkv_paged_decode_attn(d["q"][i], buf, d["bt_full"], ctl["pos_full"],
                                              c.block, wl.nb, 0, wl.k_scale[i], wl.v_scale[i],
                                              sm, c.hkv, workspace=ws_full, k_packed=k_packed,
                                              rope_cos=rc, rope_sin=rs)
            outs.append(out)
    torch.cuda.synchronize()
    return outs, ctl


def oracle_step(wl, snaps, layers=None, k_packed=True, rope=None):
    """snaps: list of host uint8 arrays (whole buffers, pre-step).  Updated in place."""
    c = wl.cfg
    half = wl.half_bytes
    bufs = [(s[:half], s[half:]) for s in snaps]
    q = [wl.q[i].float().numpy().astype(np.float64) for i in range(c.layers)]
    kn = [wl.k_new[i].float().numpy() for i in range(c.layers)]
    vn = [wl.v_new[i].float().numpy() for i in range(c.layers)]
    return OS.decode_step(bufs, q, kn, vn, wl.seq_lens, wl.active, wl.bt_full, wl.bt_swa,
                          c.block, c.hkv, c.window, wl.k_scale, wl.v_scale,
                          1.0 / np.sqrt(c.head_dim), k_packed, layers=layers, kinds=list(c.kinds),
                          rope_cos=None if rope is None else rope[0],
                          rope_sin=None if rope is None else rope[1])


def assert_close(got_bf16, ref, what=""):
    g = got_bf16.float().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    bad = ~(np.abs(g - ref) <= ATOL + RTOL * np.abs(ref))
    if bad.any():
        idx = np.argwhere(bad)[:5]
        err = np.abs(g - ref)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; "
                             f"max abs err {err[np.isfinite(err)].max() if np.isfinite(err).any() else 'nan'}; "
                             f"first {idx.tolist()} got {[g[tuple(i)] for i in idx]} "
                             f"ref {[ref[tuple(i)] for i in idx]}")
    return float(np.max(np.abs(g - ref))) if g.size else 0.0


def sampled_blocks(wl, rows):
    """Sorted ids of every block the given sequences reference (either table)."""
    ids = np.concatenate([wl.bt_full[rows].ravel(), wl.bt_swa[rows].ravel()])
    return np.unique(ids[ids >= 0]).astype(np.int64)


def gather_blocks(buf, wl, blocks):
    """Host copy (flat uint8, both halves) of the given blocks of one device
    buffer, in the order given: block blocks[i] becomes block i."""
    c = wl.cfg
    per = c.hkv * c.block * c.head_dim
    halves = buf.view(2, wl.nb, per)
    idx = torch.from_numpy(blocks).to(buf.device)
    return halves.index_select(1, idx).cpu().numpy().reshape(-1)


def mini_workload(wl, rows, blocks):
    """The workload restricted to ``rows`` over a pool holding only ``blocks``
    (relabelled 0..n-1): other sequences are inactive and have empty tables.
    The oracle run on it computes exactly the sampled rows of the full one."""
    import dataclasses
    remap = np.full(wl.nb, -1, dtype=np.int64)
    remap[blocks] = np.arange(blocks.size)
    def relabel(t):
        out = np.full_like(t, -1)
        sub = t[rows]
        out[rows] = np.where(sub >= 0, remap[np.maximum(sub, 0)], -1).astype(t.dtype)
        return out
    active = np.zeros_like(wl.active)
    active[rows] = wl.active[rows]
    return dataclasses.replace(wl, nb=int(blocks.size), active=active,
                               bt_full=relabel(wl.bt_full), bt_swa=relabel(wl.bt_swa),
                               referenced=None)


def packed_to_unpacked(buf, wl):
    """The same cache with its K half rearranged from the packed view
    [nb, H, Bk/2, D, 2] to token-major rows [nb, H, Bk, D] (a pure
    permutation of bytes; the V half is unchanged)."""
    c = wl.cfg
    halves = buf.view(2, wl.nb, c.hkv, c.block // 2, c.head_dim, 2)
    out = buf.clone().view(2, wl.nb, c.hkv, c.block, c.head_dim)
    out[0] = halves[0].permute(0, 1, 2, 4, 3).reshape(wl.nb, c.hkv, c.block, c.head_dim)
    return out.view(-1)
