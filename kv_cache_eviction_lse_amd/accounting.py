"""Host-side work and byte accounting for reports (no GPU needed).

* KV-cache size: two tensors (K and V) of layers x tokens x KV heads x head
  dim elements, as in the KVzip review's memory example ("Background -
  optional") and the KV-cache shape (2, L, H, T, D) in the background section
  of "KVzap: Fast, Adaptive, and Faithful KV Cache Pruning".
* Compression ratio: the fraction of KV pairs removed; the matching
  size-reduction factor is 1 / (1 - ratio) (the KVzap page, §4.3 Table 2).
* Algorithmic work of the scoring passes: 2 * D flops per visible
  (query head, query, key) triple.
* Algorithmic bytes of eviction: every score read once (4 B), plus for each
  kept row its index (4 B) and one read and one write of its K and V rows
  (8 * D bytes for bf16).
"""
from __future__ import annotations


def kv_cache_bytes(layers: int, tokens: int, kv_heads: int, head_dim: int, bytes_per_elem: int = 2) -> int:
    return 2 * layers * tokens * kv_heads * head_dim * bytes_per_elem


def compression_ratio(kept: int, total: int) -> float:
    return 1.0 - kept / total if total else 0.0


def compression_factor(ratio: float) -> float:
    return 1.0 / (1.0 - ratio)


def lse_pairs(n_qheads: int, n_ctx: int, n_q: int, mask: str, chunk: int = 0) -> int:
    """Visible (query head, query, key) triples of the LSE pass."""
    if mask == "causal":
        return n_qheads * n_q * (n_q + 1) // 2
    c = chunk if chunk > 0 else n_q
    full, tail = divmod(n_q, c)
    self_pairs = full * c * (c + 1) // 2 + tail * (tail + 1) // 2
    return n_qheads * (n_q * n_ctx + self_pairs)


def max_pairs(n_qheads: int, n_ctx: int, n_q: int) -> int:
    """Triples of the max-mode score pass: every repeat query sees every context key."""
    return n_qheads * n_q * n_ctx


def sum_pairs(n_qheads: int, T: int, window: int) -> int:
    """Triples of the future-mass pass: query j counts for key i when j >= i + window."""
    m = max(T - window, 0)
    return n_qheads * m * (m + 1) // 2


def flops(pairs: int, head_dim: int) -> int:
    return 2 * head_dim * pairs


def evict_bytes(n_kvheads: int, n_tok: int, kept_total: int, head_dim: int) -> int:
    return 4 * n_kvheads * n_tok + kept_total * (4 + 8 * head_dim)
