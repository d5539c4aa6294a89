"""The layer entry point writes each new token inside the attention launch;
its buffers and outputs must equal the separate cache update followed by the
attention, byte for byte, at every block size, every offset of the new token
in its sub-tile, every bf16 input pattern and the degenerate rows."""
import numpy as np
import pytest
import torch

import paged_fp8_kv_amd as P

pytestmark = pytest.mark.gpu


def _case(block, seed):
    rng = np.random.default_rng(seed)
    B, Hq, H, D, W = 128, 64, 8, 64, 128
    L = 1 + (np.arange(B) * 37 + rng.integers(0, 5, B)) % 700          # every offset mod 32
    L[:3] = [1, 2, block]
    width = -(-int(L.max()) // block)
    n_full = -(-L // block)
    keep = -(-(W + block) // block)
    swa_first = np.maximum(0, n_full - keep)
    need = int(n_full.sum() + (n_full - swa_first).sum())
    nb = need + 17
    perm = rng.permutation(nb).astype(np.int32)
    bt_full = np.full((B, width), -1, np.int32)
    bt_swa = np.full((B, width), -1, np.int32)
    at = 0
    for b in range(B):
        bt_full[b, :n_full[b]] = perm[at:at + n_full[b]]; at += n_full[b]
    for b in range(B):
        k = n_full[b] - swa_first[b]
        bt_swa[b, swa_first[b]:n_full[b]] = perm[at:at + k]; at += k
    active = np.ones(B, np.uint8)
    active[[7, 50]] = 0
    # the new token's block outside the pool (full table) / missing (window table)
    bt_full[9, (L[9] - 1) // block] = nb + 5
    bt_swa[11, (L[11] - 1) // block] = -1
    return B, Hq, H, D, W, nb, L.astype(np.int32), active, bt_full, bt_swa


@pytest.mark.parametrize("block", [16, 32, 64, 128])
def test_fused_write_matches_separate_update(block, gpu):
    B, Hq, H, D, W, nb, L, active, bt_full, bt_swa = _case(block, 100 + block)
    print(f"[fused] block {block} nb {nb}", flush=True)
    half, total = P.pkv_kv_buffer_bytes(nb, H, block, D)
    rng = np.random.default_rng(block)
    buf_a = torch.from_numpy(rng.integers(0, 0x7F, size=total, dtype=np.uint8)).to(gpu)
    buf_b = buf_a.clone()
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(gpu)
    sl, act, btf, bts = t(L), t(active), t(bt_full), t(bt_swa)
    ctl = P.pkv_setup_attn_control(sl, act, btf, bts, block, W)
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    k_new = [bits.reshape(B, H, D).to(gpu), bits.flip(0).reshape(B, H, D).to(gpu)]
    v_new = [bits.flip(0).reshape(B, H, D).to(gpu), bits.reshape(B, H, D).to(gpu)]
    q = [torch.randn(B, Hq, D).to(torch.bfloat16).to(gpu) for _ in range(2)]
    ks, vs, sm = 0.0173, 0.0411, 0.125
    step = P.make_step([buf_a], ctl, btf, B, Hq, H, D, block, W, nb)
    ws = [P.new_workspace(B, Hq, H, D, block, ctl["bt_swa_trim"].shape[1], W, gpu),
          P.new_workspace(B, Hq, H, D, block, bt_full.shape[1], 0, gpu)]
    out_a = [torch.empty_like(q[i]) for i in range(2)]
    for i in range(2):
        P.pkv_decode_layer(step, i, q[i], k_new[i], v_new[i], ks, vs, sm, out_a[i], ws[i])
    out_b = []
    for i, swa in enumerate((True, False)):
        P.pkv_kv_cache_update(buf_b, k_new[i], v_new[i], ctl["upd_swa"] if swa else ctl["upd_full"],
                              block, nb, ks, vs)
        if swa:
            out_b.append(P.pkv_paged_decode_attn(q[i], buf_b, ctl["bt_swa_trim"], ctl["pos_swa"],
                                                 block, nb, W, ks, vs, sm, H, workspace=ws[i]))
        else:
            out_b.append(P.pkv_paged_decode_attn(q[i], buf_b, btf, ctl["pos_full"], block, nb, 0,
                                                 ks, vs, sm, H, workspace=ws[i]))
    torch.cuda.synchronize()
    ga, gb = buf_a.cpu().numpy(), buf_b.cpu().numpy()
    assert np.array_equal(ga, gb), f"{int((ga != gb).sum())} buffer bytes differ"
    for i in range(2):
        a16, b16 = out_a[i].view(torch.int16).cpu(), out_b[i].view(torch.int16).cpu()
        assert torch.equal(a16, b16), f"layer {i}: {int((a16 != b16).sum())} output bits differ"
    # the degenerate rows behave as the separate path says: no write, NaN rows
    o = out_a[1].float().cpu()
    assert torch.isnan(o[9]).all() and (o[7] == 0).all()
