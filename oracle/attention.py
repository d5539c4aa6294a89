"""Paged decode attention over the FP8 cache, in float64.

What is computed (one layer, one step) -- the plain definition of decode
attention, read through the paged layout of "GPT-OSS-120B giga-kernel decode"
("Kernel contract" for the block tables / positions / window parity,
"KV-cache layout" for the packed-K and plain-V bytes):

  for each active sequence b (frame position ``hi = frame_pos[b] >= 0``) and
  query head ``g`` (KV head ``h = g // (Hq / Hkv)``):
      keys are frame positions t in [lo, hi], lo = 0 for full attention and
      lo = max(0, hi - W + 1) for a window of W;
      token t lives in block ``table[b, t // Bk]`` at slot ``t % Bk``;
      K^ = decode(K code) * k_scale,  V^ = decode(V code) * v_scale;
      s_t = sm_scale * sum_j q_j K^_tj;   w_t = exp(s_t - max_t s_t);
      out = sum_t w_t V^_t / sum_t w_t.
  inactive sequences (frame position < 0) produce zeros.

Everything is float64; the decoded FP8 values times a float32 scale are exact
in float64.  ``dense_attention`` is the brute-force twin over a logical
(unpaged) sequence used to pin this function.
"""
import math

import numpy as np

from . import fp8_e4m3, layout, rope


def gather_kv(k_half, v_half, table_row, lo: int, hi: int, head: int,
              kv_heads: int, block: int, head_dim: int, k_packed: bool = True):
    """Codes of keys lo..hi of one (sequence, KV head): two uint8 [n, D] arrays."""
    t = np.arange(lo, hi + 1, dtype=np.int64)
    blk = np.asarray(table_row, dtype=np.int64)[t // block]
    if np.any(blk < 0):
        raise ValueError("block table entry -1 inside the attended range")
    tok = t % block
    dims = np.arange(head_dim, dtype=np.int64)
    B_, J_ = np.meshgrid(np.arange(t.size), dims, indexing="ij")
    k_off = layout.k_offset(blk[B_], head, tok[B_], J_, kv_heads, block, head_dim, k_packed)
    v_off = layout.v_offset(blk[B_], head, tok[B_], J_, kv_heads, block, head_dim)
    return np.asarray(k_half)[k_off], np.asarray(v_half)[v_off]


def key_range(frame_pos: int, window: int):
    hi = int(frame_pos)
    lo = 0 if window == 0 else max(0, hi - window + 1)
    return lo, hi


def paged_decode_attention(q, k_half, v_half, block_table, frame_pos, window: int,
                           block: int, kv_heads: int, k_scale: float, v_scale: float,
                           sm_scale: float, k_packed: bool = True, rows=None,
                           rope_cos=None, rope_sin=None):
    """Return out float64 [B, Hq, D].

    q          : [B, Hq, D] values (bf16 values held exactly in any float dtype)
    k_half/v_half : flat uint8 halves of one shared buffer
    block_table: int [B, width] (full table, or the trimmed window table)
    frame_pos  : int [B], -1 for inactive
    rows       : optional iterable of sequence indices to compute (others stay 0)
    rope_cos, rope_sin : optional [B, D/2] per-sequence rotation applied to
                 every query head first (``rope.rotate``, float64)
    """
    q = np.asarray(q, dtype=np.float64)
    if rope_cos is not None:
        q = rope.rotate(q, np.asarray(rope_cos)[:, None, :], np.asarray(rope_sin)[:, None, :])
    B, Hq, D = q.shape
    G = Hq // kv_heads
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in (range(B) if rows is None else rows):
        if int(frame_pos[b]) < 0:
            continue
        lo, hi = key_range(frame_pos[b], window)
        for h in range(kv_heads):
            kc, vc = gather_kv(k_half, v_half, block_table[b], lo, hi, h,
                               kv_heads, block, D, k_packed)
            K = fp8_e4m3.decode(kc) * float(k_scale)
            V = fp8_e4m3.decode(vc) * float(v_scale)
            for g in range(G):
                s = (K @ q[b, h * G + g]) * float(sm_scale)
                w = np.exp(s - s.max())
                out[b, h * G + g] = (w @ V) / w.sum()
    return out


def dense_attention(q_vec, k_rows, v_rows, sm_scale: float):
    """Brute force over explicit lists: exact sums with math.fsum.

    q_vec: D floats; k_rows, v_rows: lists of D-float rows (already dequantised).
    """
    s = [sm_scale * math.fsum(a * b for a, b in zip(q_vec, k)) for k in k_rows]
    m = max(s)
    w = [math.exp(x - m) for x in s]
    z = math.fsum(w)
    D = len(v_rows[0])
    return [math.fsum(w[t] * v_rows[t][j] for t in range(len(w))) / z for j in range(D)]
