"""Layer-invariant attention control for one decode step.

"GPT-OSS-120B giga-kernel decode", section "Kernel contract": per step the
kernel consumes, built once from the per-layer metadata, a full block table and
a trimmed sliding-window block table, an active mask, absolute and
window-frame positions, and two KV-update indices (one for the full table, one
for the trimmed sliding-window table).  Even layers use a window of 128 keys.

Readings (design notes):
  * ``seq_lens[b]`` counts the sequence's tokens including the new one; the
    new token's index is ``p = seq_lens[b] - 1`` and the cache is indexed by
    that token index, never by the absolute position.
  * the window holds the ``W`` most recent tokens including the new one:
    token indices ``[p - W + 1, p]``.  This is the only width for which the
    early-eviction boundary described in "DI wiring (NIXL)" falls at
    ``N % block_size == block_size - 1``.
  * the trimmed table lists the sliding-window table's block ids for logical
    blocks ``f .. p // Bk`` where ``f = max(0, p - W + 1) // Bk``, padded with
    -1 to width ``ceil((W - 1) / Bk) + 1``; the window-frame position is
    ``p - f * Bk``.
  * an update index is the cache slot ``block_id * Bk + offset`` (int64);
    inactive sequences get -1 everywhere (no write, no read, zero output), and
    so does an update index whose table entry is negative (no block).
  * "DI wiring (NIXL)" (sliding-window DI truncation): a decode node that
    admits a prompt of N tokens but recomputes its last token would evict the
    window's oldest block one step early at ``N % block_size ==
    block_size - 1``; the fix makes both nodes operate at N - 1.  Reading
    taken for the setup: an optional lag of one token in the window frame's
    anchor.  With ``anchor_lag = 1`` the frame's first block is the one the
    step at ``p - 1`` would use, ``f = max(0, p - 1 - W + 1) // Bk``, so the
    oldest block stays in the trimmed table one step longer (it leaves at
    ``p % Bk == 0`` instead of ``p % Bk == Bk - 1``).  The attended keys stay
    ``[p - W + 1, p]``; the trimmed table is
    ``ceil((W - 1 + anchor_lag) / Bk) + 1`` wide.
"""
import numpy as np


def trimmed_width(window: int, block: int, anchor_lag: int = 0) -> int:
    """Most logical blocks a frame of ``window + anchor_lag`` tokens can touch."""
    return -(-(window - 1 + anchor_lag) // block) + 1


def attention_control(seq_lens, active, bt_full, bt_swa, block: int, window: int,
                      positions=None, anchor_lag: int = 0):
    """Return the per-step control as a dict of numpy arrays.

    bt_full, bt_swa : int32 [B, width] tables indexed by logical block.
    Keys: ``pos_full`` (int32 [B], p), ``pos_swa`` (int32 [B], window-frame
    position), ``bt_swa_trim`` (int32 [B, n_swa]), ``upd_full`` and
    ``upd_swa`` (int64 [B] cache slots), ``pos_abs`` (int64 [B], the absolute
    positions carried for the rotary stage; -1 when not given or inactive).
    anchor_lag : 0, or 1 for the N - 1 reading of "DI wiring (NIXL)" above.
    """
    if anchor_lag not in (0, 1):
        raise ValueError("anchor_lag must be 0 or 1")
    seq_lens = np.asarray(seq_lens)
    B = seq_lens.shape[0]
    n_swa = trimmed_width(window, block, anchor_lag)
    pos_full = np.full(B, -1, dtype=np.int32)
    pos_swa = np.full(B, -1, dtype=np.int32)
    trim = np.full((B, n_swa), -1, dtype=np.int32)
    upd_full = np.full(B, -1, dtype=np.int64)
    upd_swa = np.full(B, -1, dtype=np.int64)
    pos_abs = np.full(B, -1, dtype=np.int64)
    for b in range(B):
        if not active[b]:
            continue
        p = int(seq_lens[b]) - 1
        pos_full[b] = p
        blk_full = int(bt_full[b, p // block])
        upd_full[b] = blk_full * block + p % block if blk_full >= 0 else -1
        first = max(0, p - anchor_lag - window + 1) // block
        for c in range(first, p // block + 1):
            trim[b, c - first] = bt_swa[b, c]
        wf = p - first * block
        pos_swa[b] = wf
        blk_swa = int(trim[b, wf // block])
        upd_swa[b] = blk_swa * block + wf % block if blk_swa >= 0 else -1
        if positions is not None:
            pos_abs[b] = int(positions[b])
    return dict(pos_full=pos_full, pos_swa=pos_swa, bt_swa_trim=trim,
                upd_full=upd_full, upd_swa=upd_swa, pos_abs=pos_abs)


def csr_to_tables(kv_indptr, full_indices, swa_indices, last_page_len, block: int, width: int):
    """Padded per-sequence inputs from compressed page lists.

    "MPK Internals: Compilation-to-Runtime Pipeline", "Phase 4: Runtime
    Initialization", names the per-step page meta-tensors (`qo_indptr`,
    `paged_kv_indptr`, `paged_kv_indices`, `paged_kv_last_page_len`) without
    defining them.  Reading: sequence b's pages are
    ``full_indices[kv_indptr[b]:kv_indptr[b+1]]`` in logical order; its token
    count is ``(pages - 1) * block + last_page_len[b]`` (0 pages: no tokens);
    the sliding-window page list shares ``kv_indptr`` and holds -1 where the
    window's blocks were freed; a decode step has one query per sequence, so
    ``qo_indptr`` is the identity and is not needed.

    Returns (seq_lens int32 [B], bt_full int32 [B, width], bt_swa int32
    [B, width]), -1 beyond each sequence's pages (pages past `width` dropped).
    """
    kv_indptr = np.asarray(kv_indptr, dtype=np.int64)
    B = kv_indptr.size - 1
    seq_lens = np.zeros(B, dtype=np.int32)
    bt_full = np.full((B, width), -1, dtype=np.int32)
    bt_swa = np.full((B, width), -1, dtype=np.int32)
    for b in range(B):
        lo, hi = int(kv_indptr[b]), int(kv_indptr[b + 1])
        n = hi - lo
        if n > 0:
            seq_lens[b] = (n - 1) * block + int(last_page_len[b])
        for c in range(min(n, width)):
            bt_full[b, c] = full_indices[lo + c]
            if swa_indices is not None:
                bt_swa[b, c] = swa_indices[lo + c]
    return seq_lens, bt_full, bt_swa
