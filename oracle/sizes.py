"""Byte and block counts that the pages state.

- "KV cache: la memoria de trabajo ...", "El precio: cuanto pesa la
  mochila": KV size = 2 * n_layers * n_kv_heads * head_dim * context_len *
  bytes per element (the 2 is K and V); per token it is a constant of the
  model.
- same post, "Por que existe: el coste cuadratico sin el": without a cache,
  generating N tokens costs sum_{i=1..N} i = N(N+1)/2 attention
  computations; with it, N.
- "PagedAttention por dentro", "El modelo de bloques": a block covers 16
  tokens of one layer, so a session of n tokens in an L-layer model holds
  ceil(n/16) * L blocks; "El pool de bloques": the all-layer bytes of 16
  tokens, and blocks available = (memory left for the cache) / block bytes.
- "vLLM en Kubernetes ...", "PagedAttention: la memoria virtual del KV
  cache": a 273-token session occupies 18 blocks.
- "Como funciona realmente vLLM", "La sobre-reserva estatica": static
  worst-case reservation versus what is used.
"""
from __future__ import annotations

BLOCK_SIZE = 16


def kv_bytes_per_token(n_layers: int, n_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    return 2 * n_layers * n_kv_heads * head_dim * elem_bytes


def kv_bytes(n_layers, n_kv_heads, head_dim, context_len, elem_bytes) -> int:
    return kv_bytes_per_token(n_layers, n_kv_heads, head_dim, elem_bytes) * context_len


def attention_ops_without_cache(n: int) -> int:
    return n * (n + 1) // 2


def blocks_for(n_tokens: int) -> int:
    return -(-n_tokens // BLOCK_SIZE)


def session_blocks(n_tokens: int, n_layers: int) -> int:
    return blocks_for(n_tokens) * n_layers


def all_layer_block_bytes(n_layers, n_kv_heads, head_dim, elem_bytes, block_size=BLOCK_SIZE):
    return block_size * n_layers * 2 * n_kv_heads * head_dim * elem_bytes


def pool_blocks(available_bytes: int, block_bytes: int) -> int:
    return available_bytes // block_bytes


def paged_waste_fraction(lengths) -> float:
    """Empty slots over allocated slots, for sequences that own their blocks."""
    alloc = sum(blocks_for(n) * BLOCK_SIZE for n in lengths)
    used = sum(lengths)
    return (alloc - used) / alloc if alloc else 0.0


def static_waste_fraction(lengths, reserved_per_seq: int) -> float:
    """Reserved-but-empty slots over reserved slots for worst-case reservation."""
    reserved = reserved_per_seq * len(lengths)
    return (reserved - sum(lengths)) / reserved if reserved else 0.0
