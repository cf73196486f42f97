"""Float64 CPU oracle for sparse MLA decode (DeepSeek Sparse Attention): index
scores over the cached tokens, top-k selection, and the MLA decode over the
selected positions only.  TEST INFRASTRUCTURE ONLY: imported by ``tests/``
and ``bench.py``'s CPU-baseline leg, never by the product path.

Source: [V32] "DeepSeek-V3.2-Exp unboxing", section "初步研读": once the KV
cache is written, the MLA forward scores the cached tokens with an FP8 index
kernel and keeps the highest-scoring ones for the rest of the computation;
the kernel's signature takes q [b, m, h, d] in FP8, q_s [b, m, h] in FP32
(the call passes the per-head ``weights`` there), k [b, n, d] in FP8 and
k_s [b, n] in FP32 (the per-token key scale cache) and returns o [b, m, n] in
FP32; the observed shapes are q [2, 128, 64, 128] and k [2, 128, 128]; the
selected top-k indices are shared by every GPU.

Readings (each is listed in the design doc; the pages give the signature, not the
arithmetic):

* index score of cached position n for one query:
  o[n] = sum_h q_s[h] * (sum_d q[h, d] * k[n, d]) * k_s[n], q and k as E4M3
  FN values (the FP8 format of the latent cache); no other operation is
  stated, so none is applied;
* top-k: the k positions with the largest scores; equal scores: the lower
  position first; the result in ascending position order; a sequence with
  fewer than k positions keeps all of them;
* the attention is the MLA decode restricted to the selected positions, for
  one new token per sequence (q_len = 1: every cached position is visible).

Every function here is pinned by ``tests/test_dsa_oracle.py``; none is
"parity unpinned".
"""
from __future__ import annotations

import numpy as np

from .fp8 import e4m3_decode
from .mla_oracle import decode_expanded


def index_scores(q_codes, q_w, k_codes, k_scale, block_table, seq_len: int, b: int):
    """Scores of the cached positions 0..seq_len-1 of sequence b (float64 [L]).

    q_codes  uint8 [B, Hi, D] E4M3 index queries; q_w float [B, Hi] weights
    k_codes  uint8 [num_blocks, page, D] E4M3 index keys (paged like the
             latent cache, same block table); k_scale float [num_blocks, page]
    """
    page = k_codes.shape[1]
    t = np.arange(seq_len)
    blk = block_table[b, t // page].astype(np.int64)
    k = e4m3_decode(k_codes[blk, t % page])                       # [L, D]
    ks = np.asarray(k_scale, dtype=np.float64)[blk, t % page]     # [L]
    q = e4m3_decode(q_codes[b])                                    # [Hi, D]
    w = np.asarray(q_w, dtype=np.float64)[b]                       # [Hi]
    per_head = q @ k.T                                             # [Hi, L]
    return (w[:, None] * per_head).sum(axis=0) * ks


def topk_positions(scores, k: int) -> np.ndarray:
    """The k largest scores' positions (ties: lower position first), in
    ascending position order."""
    scores = np.asarray(scores, dtype=np.float64)
    n = scores.shape[0]
    k = min(k, n)
    order = np.lexsort((np.arange(n), -scores))   # by score descending, then position
    return np.sort(order[:k])


def decode_sparse(q_bits, kv_b_bits, cache_bits, block_table, seq_lens, positions, **kw):
    """MLA decode (expanded form) of one new token per sequence over the
    selected positions only: ``positions[b]`` (ascending) are gathered into a
    compact sequence and decoded with ``decode_expanded`` (q_len 1, every
    gathered position visible).  Returns float64 [B, 1, H, 128]."""
    bsz = q_bits.shape[0]
    page = cache_bits.shape[1]
    counts = [len(p) for p in positions]
    pages = [max(1, (c + page - 1) // page) for c in counts]
    compact = np.zeros((sum(pages), page, cache_bits.shape[2]), dtype=cache_bits.dtype)
    bt = np.zeros((bsz, max(pages)), dtype=np.int64)
    base = 0
    for b in range(bsz):
        pos = np.asarray(positions[b], dtype=np.int64)
        rows = cache_bits[block_table[b, pos // page].astype(np.int64), pos % page]
        j = np.arange(len(pos))
        compact[base + j // page, j % page] = rows
        bt[b, :pages[b]] = base + np.arange(pages[b])
        base += pages[b]
    return decode_expanded(q_bits, kv_b_bits, compact, bt, np.asarray(counts), 1, **kw)


__all__ = ["index_scores", "topk_positions", "decode_sparse"]
