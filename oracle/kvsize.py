"""Closed forms for KV-cache size.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

[ch15] "KV cache / batching / paged attention", section
"KVキャッシュはどれくらいメモリを食う？": the cache holds K and V (factor 2)
for every layer, KV head, head-dimension element, token and concurrent
request, at the element's byte width.  Section "KVを小さくするモデル側の工夫"
sizes an MLA cache from one latent vector plus a positional part per layer
(no K/V factor of 2).
"""


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, elt_bytes: int) -> int:
    """2 (K and V) x layers x KV heads x head_dim x bytes per element."""
    return 2 * layers * kv_heads * head_dim * elt_bytes


def kv_bytes_total(layers: int, kv_heads: int, head_dim: int, elt_bytes: int,
                   tokens: int, requests: int) -> int:
    """Per-token size x tokens x concurrent requests."""
    return kv_bytes_per_token(layers, kv_heads, head_dim, elt_bytes) * tokens * requests


def mla_bytes_per_token(layers: int, latent_dim: int, rope_dim: int, elt_bytes: int) -> int:
    """One cached latent (plus its positional part) per layer; no separate K and V."""
    return layers * (latent_dim + rope_dim) * elt_bytes


def layer_bytes_per_token(kv_heads: int, head_dim: int, elt_bytes: int) -> int:
    """The one-layer slice of the closed form: bytes one cached token adds to
    one layer's K and V caches."""
    return kv_bytes_per_token(1, kv_heads, head_dim, elt_bytes)
