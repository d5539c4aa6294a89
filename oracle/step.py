"""The layer schedule of one decode step over shared buffers.

"GPT-OSS-120B giga-kernel decode", section "Kernel contract": layer ``i`` is
sliding-window (window 128) when ``i`` is even and full attention when odd; it
picks its block table and write index by ``i % 2`` and its KV buffer by
``i // 2`` (layers ``2j`` and ``2j + 1`` share buffer ``j``).  Section
"KV-cache layout": one full table and one sliding-window table serve every
layer.  Each layer first writes its new token's K/V, then attends (the new
token is read back from the cache, i.e. after quantisation).
"""
import numpy as np

from . import attention, control, update


def decode_step(buffers, q, k_new, v_new, seq_lens, active, bt_full, bt_swa,
                block: int, kv_heads: int, window: int, k_scale, v_scale,
                sm_scale: float, k_packed: bool = True, layers=None, kinds=None,
                rope_cos=None, rope_sin=None, anchor_lag: int = 0):
    """Run ``len(q)`` layers in place on ``buffers``.

    buffers : list of (k_half, v_half) flat uint8 arrays, one pair per buffer.
    q, k_new, v_new : per-layer arrays [L][B, H*, D].
    k_scale, v_scale : per-layer sequences of floats.
    layers  : optional subset of layer indices whose attention is computed
              (writes are always done for every layer, in order).
    kinds   : optional per-layer list of "swa" / "full"; default is the
              alternating schedule (even layers sliding-window).
    rope_cos, rope_sin : optional float32 [B, D/2]; the one rotation of this
              step's queries and new keys, shared by every layer.
    anchor_lag : window-frame anchor lag of the control (``control``, the
              N - 1 reading of "DI wiring (NIXL)"); the attended keys are the
              same either way.
    Returns (outputs dict layer -> [B, Hq, D] float64, control dict).
    """
    ctl = control.attention_control(seq_lens, active, bt_full, bt_swa, block, window,
                                    anchor_lag=anchor_lag)
    outs = {}
    for i in range(len(q)):
        k_half, v_half = buffers[i // 2]
        swa = (i % 2 == 0) if kinds is None else (kinds[i] == "swa")
        slots = ctl["upd_swa"] if swa else ctl["upd_full"]
        update.kv_cache_update(k_half, v_half, np.asarray(k_new[i]), np.asarray(v_new[i]),
                               slots, block, k_scale[i], v_scale[i], k_packed,
                               rope_cos, rope_sin)
        if layers is not None and i not in layers:
            continue
        table = ctl["bt_swa_trim"] if swa else bt_full
        pos = ctl["pos_swa"] if swa else ctl["pos_full"]
        outs[i] = attention.paged_decode_attention(
            q[i], k_half, v_half, table, pos, window if swa else 0, block, kv_heads,
            k_scale[i], v_scale[i], sm_scale, k_packed, rope_cos=rope_cos, rope_sin=rope_sin)
    return outs, ctl
