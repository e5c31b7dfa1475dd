"""ORACLE — test infrastructure, not the product.

KV-cache size arithmetic exactly as the source pages state it, in bytes and
elements (no unit rounding). Pinned by ``tests/test_oracle_pins.py`` against
the worked numbers the pages print (``tests/golden/cache_arithmetic.json``).
"""
from __future__ import annotations


def mha_kv_elems_per_token_layer(heads: int, head_dim: int) -> int:
    """K and V of every head: 2 x h x d (MLA tutorial page, §1)."""
    return 2 * heads * head_dim


def kv_cache_bytes(layers: int, kv_heads: int, head_dim: int, seq_len: int, batch: int,
                   dtype_bytes: int) -> int:
    """2 x layers x kv_heads x head_dim x seq_len x batch x bytes (interview guide §2.1)."""
    return 2 * layers * kv_heads * head_dim * seq_len * batch * dtype_bytes


def mla_cache_bytes(layers: int, d_c: int, seq_len: int, batch: int, dtype_bytes: int,
                    d_rope: int = 0) -> int:
    """One latent row of d_c (+ the decoupled RoPE key) per token per layer
    (MLA tutorial page §5.2; linear-algebra page, "解耦 RoPE" cache row)."""
    return layers * (d_c + d_rope) * seq_len * batch * dtype_bytes


def compression_ratio(heads: int, d_k: int, d_v: int, d_c: int, d_rope: int = 0) -> float:
    """(h x d_k + h x d_v) / cached width (MLA tutorial page §2.3)."""
    return (heads * d_k + heads * d_v) / (d_c + d_rope)


def latent_fraction(d_latent: int, heads: int, head_dim: int) -> float:
    """d_latent / (2 x heads x head_dim) (MHA->MLA trade-off page, §2.3)."""
    return d_latent / (2 * heads * head_dim)
