"""Write of the new token's K and V into the FP8 cache (one layer).

"GPT-OSS-120B giga-kernel decode", section "Kernel contract": each step writes
the new token's K/V through an update index -- layer ``i`` uses the
sliding-window index when ``i`` is even and the full index when odd -- into
the buffer ``i // 2`` shared by layers ``2j`` and ``2j + 1``; section
"KV-cache layout": K goes through the packed view, V is plain.

The stored code is ``E4M3(fp32(x) / fp32(scale))`` with ``scale`` the
per-tensor dequantisation multiplier.  With rotary cos/sin given (the
attention control of "Kernel contract"), K is first rotated in fp32 as
``rope.rotate_f32`` states and the rotated value is quantised.
"""
import numpy as np

from . import fp8_e4m3, layout, rope


def kv_cache_update(k_half, v_half, k_new, v_new, slot_idx, block: int,
                    k_scale: float, v_scale: float, k_packed: bool = True,
                    rope_cos=None, rope_sin=None):
    """Write in place.  k_half / v_half: flat uint8 arrays of one half each.

    k_new, v_new : float arrays [B, H, D] holding the bf16 values exactly.
    slot_idx     : int64 [B]; -1 means the sequence is inactive (no write).
    rope_cos, rope_sin : optional float32 [B, D/2] per-sequence rotation of K.
    """
    B, H, D = k_new.shape
    if rope_cos is not None:
        k_new = rope.rotate_f32(k_new, np.asarray(rope_cos)[:, None, :],
                                np.asarray(rope_sin)[:, None, :])
    k_codes = fp8_e4m3.quantize(k_new, k_scale)
    v_codes = fp8_e4m3.quantize(v_new, v_scale)
    for b in range(B):
        slot = int(slot_idx[b])
        if slot < 0:
            continue
        blk, tok = divmod(slot, block)
        for h in range(H):
            for j in range(D):
                k_half[layout.k_offset(blk, h, tok, j, H, block, D, k_packed)] = k_codes[b, h, j]
                v_half[layout.v_offset(blk, h, tok, j, H, block, D)] = v_codes[b, h, j]
    return k_codes, v_codes
