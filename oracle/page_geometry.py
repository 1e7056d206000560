"""Page-size facts printed by the pages (test infrastructure only).

Page-alignment post (luanjiahao.me), §2: the access unit is 64 tokens; 784
splits into 12 full 64-token groups plus a 16-token tail, 832 into 13 full
groups; 832 is the smallest multiple of 64 that is at least 784, adding about
6.1% capacity where 1024 adds about 30.6%.  §4: one K (or V) page holds
BLOCK_SIZE * 4 * 256 bf16 values.
"""
from __future__ import annotations

GROUP_TOKENS = 64


def groups_in_page(block_size: int, group: int = GROUP_TOKENS):
    """(number of full groups, tail tokens) of one page."""
    if block_size < 1:
        raise ValueError("block_size must be positive")
    return block_size // group, block_size % group


def page_bytes(block_size: int, num_kv_heads: int = 4, head_dim: int = 256,
               elem_bytes: int = 2) -> int:
    """Bytes of one K page (or one V page) in the [pages, B, Hkv, D] layout."""
    return block_size * num_kv_heads * head_dim * elem_bytes


def smallest_aligned_page(block_size: int, group: int = GROUP_TOKENS) -> int:
    """Smallest multiple of ``group`` that is >= block_size."""
    return -(-block_size // group) * group
