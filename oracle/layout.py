"""Byte layout of one shared KV buffer.

"GPT-OSS-120B giga-kernel decode", section "KV-cache layout (per-buffer,
HMA-preserving)": each group buffer is one allocation of shape
``[2, num_blocks, kv_heads, block, head_dim]`` (K half first, then V half),
one byte per FP8 element; paired layers share a buffer.  K may be stored
packed: a trailing view ``[..., block // 2, head_dim, 2]`` over the same bytes
and the same number of blocks, while V is never packed.

Reading of the packed view (design notes): element ``[pair, j, e]`` of the
view is token ``2 * pair + e`` at dimension ``j`` -- two consecutive tokens of
a block interleave per dimension.  The plain layout is token-major
``[block, head_dim]``.

All offsets are byte offsets inside one half (K half or V half); the V half
starts ``half_bytes`` after the K half.
"""


def half_bytes(num_blocks: int, kv_heads: int, block: int, head_dim: int) -> int:
    """Bytes of one half (K or V) of a shared buffer (1 byte per element)."""
    return num_blocks * kv_heads * block * head_dim


def buffer_bytes(num_blocks: int, kv_heads: int, block: int, head_dim: int) -> int:
    """Bytes of one shared buffer: the K half plus the V half."""
    return 2 * half_bytes(num_blocks, kv_heads, block, head_dim)


def plain_offset(blk: int, head: int, tok: int, dim: int,
                 kv_heads: int, block: int, head_dim: int) -> int:
    """Offset of (block, head, token-in-block, dim) in a ``[nb, H, Bk, D]`` half."""
    return ((blk * kv_heads + head) * block + tok) * head_dim + dim


def packed_offset(blk: int, head: int, tok: int, dim: int,
                  kv_heads: int, block: int, head_dim: int) -> int:
    """Offset of (block, head, token-in-block, dim) in a packed K half,
    i.e. of view element ``[blk, head, tok // 2, dim, tok % 2]`` of
    ``[nb, H, Bk // 2, D, 2]``."""
    pair, parity = divmod(tok, 2)
    return (((blk * kv_heads + head) * (block // 2) + pair) * head_dim + dim) * 2 + parity


def k_offset(blk, head, tok, dim, kv_heads, block, head_dim, packed: bool) -> int:
    if packed:
        return packed_offset(blk, head, tok, dim, kv_heads, block, head_dim)
    return plain_offset(blk, head, tok, dim, kv_heads, block, head_dim)


def v_offset(blk, head, tok, dim, kv_heads, block, head_dim) -> int:
    return plain_offset(blk, head, tok, dim, kv_heads, block, head_dim)
