"""Test helper: lay out a logical (unpaged) KV sequence into paged halves using
torch views of the shapes the pages print -- independent of oracle.layout."""
import numpy as np
import torch

POISON = 0x7F


def build_halves(k_log, v_log, table_row_list, nb, H, Bk, D, packed=True, fill=POISON):
    """k_log, v_log: lists (one per sequence) of uint8 [n_tok, H, D] codes.
    table_row_list: per sequence, an int array of block ids for logical blocks.
    Returns flat numpy uint8 halves (K, V)."""
    kh = torch.full((nb * H * Bk * D,), fill, dtype=torch.uint8)
    vh = torch.full((nb * H * Bk * D,), fill, dtype=torch.uint8)
    kview = kh.view(nb, H, Bk // 2, D, 2) if packed else kh.view(nb, H, Bk, D)
    vview = vh.view(nb, H, Bk, D)
    for kl, vl, row in zip(k_log, v_log, table_row_list):
        kl = torch.from_numpy(np.asarray(kl, dtype=np.uint8))
        vl = torch.from_numpy(np.asarray(vl, dtype=np.uint8))
        for t in range(kl.shape[0]):
            blk, s = int(row[t // Bk]), t % Bk
            if packed:
                kview[blk, :, s // 2, :, s % 2] = kl[t]
            else:
                kview[blk, :, s, :] = kl[t]
            vview[blk, :, s, :] = vl[t]
    return kh.numpy(), vh.numpy()


def torch_decode(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()


def random_codes(rng, shape, scale=1.0 / 8):
    x = rng.standard_normal(shape).astype(np.float32) / np.float32(scale)
    return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def bf16_values(rng, shape):
    x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32))
    return x.to(torch.bfloat16).to(torch.float64).numpy()
