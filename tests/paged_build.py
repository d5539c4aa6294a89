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


# 1.0625 + 2^-24 = 1.5 * C_TIE exactly: halfway between two fp32 neighbours,
# and 1.0625 itself is halfway between the E4M3 values 1.0 and 1.125.
C_TIE = 5941931 * 2.0 ** -23
TINY = 2.0 ** -40


def rope_fma_trap():
    """Rotation inputs where fusing a product into the sum changes the FP8 code.

    Returns (x float32 [2, 64] of bf16 values, cos, sin float32 [2, 32],
    traps).  At each trap (row, dim) the exact rotated value is
    1.0625 + 2^-24 + 2^-40: one product is exactly the fp32 tie 1.0625 + 2^-24
    (rounded to even: 1.0625), the other is 2^-40.  Rounding each product and
    then the sum gives 1.0625 (E4M3 code 0x38 at scale 1: a tie, to even);
    a fused multiply-add over the tied product gives 1.0625 + 2^-23 (0x39).
    The four traps put the tied product in each of the four product positions
    (x_lo*cos, x_hi*sin, x_hi*cos, x_lo*sin).  Other dimensions: random bf16
    values and a random rotation.
    """
    rng = np.random.default_rng(77)
    x = bf16_values(rng, (2, 64)).astype(np.float32)
    th = rng.uniform(-np.pi, np.pi, (2, 32))
    c, s = np.cos(th).astype(np.float32), np.sin(th).astype(np.float32)
    # row 0, dim 0: lo = 1.5*C_TIE - 1*(-TINY)          (tie in x_lo*cos)
    x[0, 0], x[0, 32], c[0, 0], s[0, 0] = 1.5, 1.0, C_TIE, -TINY
    # row 1, dim 0: lo = 1*TINY - 1.5*(-C_TIE)          (tie in x_hi*sin)
    x[1, 0], x[1, 32], c[1, 0], s[1, 0] = 1.0, 1.5, TINY, -C_TIE
    # row 0, dim 33: hi = 1.5*C_TIE + 1*TINY            (tie in x_hi*cos)
    x[0, 1], x[0, 33], c[0, 1], s[0, 1] = 1.0, 1.5, C_TIE, TINY
    # row 1, dim 33: hi = 1*TINY + 1.5*C_TIE            (tie in x_lo*sin)
    x[1, 1], x[1, 33], c[1, 1], s[1, 1] = 1.5, 1.0, TINY, C_TIE
    return x, c, s, [(0, 0), (1, 0), (0, 33), (1, 33)]
