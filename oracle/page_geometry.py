"""Page-size facts printed by the pages (test infrastructure only).

Page-alignment post (luanjiahao.me), §2: the access unit is 64 tokens; 784
splits into 12 full 64-token groups plus a 16-token tail, 832 into 13 full
groups; 832 is the smallest multiple of 64 that is at least 784, adding about
6.1% capacity where 1024 adds about 30.6%.  §4: one K (or V) page holds
BLOCK_SIZE * 4 * 256 bf16 values.  §3: with prefix caching off, a hybrid
model's attention page is sized so that it holds at least one Mamba state
page, rounded up to whole groups of alignment_tokens tokens.
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


def attn_page_bytes_per_token(num_kv_heads: int = 4, head_dim: int = 256, elem_bytes: int = 2) -> int:
    """One token's K and V for one attention layer (§4: K and V pages of
    BLOCK_SIZE x heads x head_dim elements each)."""
    return 2 * num_kv_heads * head_dim * elem_bytes


def required_page_tokens(mamba_page_bytes: int, attn_bytes_per_token: int,
                         alignment_tokens: int) -> int:
    """§3: ceil(mamba_page_bytes / (alignment_tokens * attn_page_size_1_token))
    * alignment_tokens, in exact integer arithmetic (the minimum comparison
    and padding branches the page omits are omitted here too)."""
    if mamba_page_bytes <= 0 or attn_bytes_per_token <= 0 or alignment_tokens <= 0:
        raise ValueError("arguments must be positive")
    group_bytes = alignment_tokens * attn_bytes_per_token
    return -(-mamba_page_bytes // group_bytes) * alignment_tokens
