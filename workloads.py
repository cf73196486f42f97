"""Seeded synthetic workloads for MLA latent-KV decode + cache insert.

This module only draws random inputs and counts bytes; it contains none of the
method's arithmetic.  Both the oracle tests and the HIP path consume what it
produces, so it is the one module the two sides share.

Shapes follow the DeepSeek MLA dimensions the pages give: latent (kv_lora)
512, rope 64, qk_nope 128, v 128, cache entry 576 numbers, pages of 64
tokens.  bf16 tensors are returned as numpy ``uint16`` bit patterns.

Recipe (numpy PCG64, one generator per workload, fixed draw order):
seq_lens -> block-table permutation -> kv_b -> rms_w -> cache prefix (sequence
by sequence) -> new kv_a -> q.  float32 draws are rounded to bf16 (nearest,
ties to even).  kv_b ~ N(0, var 1/512), rms_w ~ 1 + N(0, var 0.1), cache
prefix / kv_a / q ~ N(0, 1).  Cache slots that are not part of any sequence's
prefix hold the NaN pattern ``SENTINEL`` so that a kernel touching them shows.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

LATENT, ROPE, NOPE, VDIM, PAGE = 512, 64, 128, 128, 64
ENTRY = LATENT + ROPE
SENTINEL = np.uint16(0xFFC1)  # a quiet-NaN bf16 pattern
EPS = 1e-6
ROPE_BASE = 10000.0


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (r >> np.uint32(16)).astype(np.uint16)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    q_len: int
    heads: int
    lens: str            # "fixed:N" | "uniform:A:B" | "loguniform_max:A:B" | "list:a,b,c"
    permute: bool = True
    seed: int = 0
    description: str = ""


WORKLOADS = {
    "tiny_v2lite": Workload(
        "tiny_v2lite", 1, 1, 16, "fixed:256", permute=False,
        description="V2-Lite shape, batch 1, q_len 1, 16 heads, context 256, identity table"),
    "v2lite_b32": Workload(
        "v2lite_b32", 32, 1, 16, "uniform:1024:4096",
        description="V2-Lite shape, batch 32, q_len 1, 16 heads, context U[1024,4096]"),
    "v3_b64_l8192": Workload(
        "v3_b64_l8192", 64, 1, 128, "fixed:8192",
        description="V3 shape, batch 64, q_len 1, 128 heads, context 8192"),
    "v3_longskew_b8": Workload(
        "v3_longskew_b8", 8, 1, 128, "loguniform_max:2048:32768",
        description="V3 shape, batch 8, q_len 1, 128 heads, context log-uniform "
                    "[2048,32768] with one at 32768"),
    "v3_mtp_b128": Workload(
        "v3_mtp_b128", 128, 2, 128, "uniform:1024:16384",
        description="V3 shape, batch 128, q_len 2 (causal among the new tokens), "
                    "128 heads, context U[1024,16384], insert of the 2 new tokens first"),
}
ORDER = ["tiny_v2lite", "v2lite_b32", "v3_b64_l8192", "v3_longskew_b8", "v3_mtp_b128"]
# prefill in the expanded form: many new tokens per sequence
WORKLOADS.update({
    "prefill_v3_b2_s4096": Workload(
        "prefill_v3_b2_s4096", 2, 4096, 128, "fixed:4096",
        description="V3 shape prefill: 2 prompts of 4096 new tokens (no cached prefix), "
                    "128 heads"),
    "prefill_v3_chunk_b4": Workload(
        "prefill_v3_chunk_b4", 4, 1024, 128, "uniform:2048:8192",
        description="V3 shape chunked prefill: 4 sequences, a chunk of 1024 new tokens "
                    "after a cached prefix (context U[2048,8192]), 128 heads"),
})
PREFILL = ["prefill_v3_b2_s4096", "prefill_v3_chunk_b4"]

# Sparse decode (DeepSeek Sparse Attention) workloads: a decode workload, the
# number of kept positions and the index heads (64 heads of width 128, the
# indexer shapes observed in the V3.2 run).
DSA = {
    "dsa_v3_b64_l8192_k2048": dict(base="v3_b64_l8192", top_k=2048, index_heads=64,
                                   description="the V3 decode workload (64 sequences of 8192 "
                                               "positions, 128 heads) keeping 2048 positions "
                                               "per sequence by 64 FP8 index heads"),
}


def make_dsa_workload(name: str) -> dict:
    w = DSA[name]
    d = make_workload(w["base"])
    d.update(make_index_inputs(d, index_heads=w["index_heads"], seed=1))
    d["top_k"] = w["top_k"]
    d["name"] = name
    return d


def draw_lens(rng: np.random.Generator, spec: str, batch: int) -> np.ndarray:
    kind, *args = spec.split(":")
    if kind == "fixed":
        return np.full(batch, int(args[0]), dtype=np.int64)
    if kind == "uniform":
        lo, hi = int(args[0]), int(args[1])
        return rng.integers(lo, hi + 1, size=batch).astype(np.int64)
    if kind == "loguniform_max":
        lo, hi = int(args[0]), int(args[1])
        rest = np.rint(np.exp(rng.uniform(math.log(lo), math.log(hi), size=batch - 1)))
        return np.concatenate([[hi], rest]).astype(np.int64)
    if kind == "list":
        vals = [int(v) for v in args[0].split(",")]
        assert len(vals) == batch
        return np.asarray(vals, dtype=np.int64)
    raise ValueError(spec)


def make_inputs(batch: int, q_len: int, heads: int, lens, permute: bool = True,
                seed: int = 0, spare_blocks: int = 0) -> dict:
    """Draw one workload.  ``lens`` is a spec string or an explicit sequence."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if isinstance(lens, str):
        seq_lens = draw_lens(rng, lens, batch)
    else:
        seq_lens = np.asarray(lens, dtype=np.int64)
        assert seq_lens.shape == (batch,)
    assert np.all(seq_lens >= q_len)
    nblk = (seq_lens + PAGE - 1) // PAGE
    num_blocks = int(nblk.sum()) + spare_blocks
    max_blocks = int(nblk.max()) if batch else 1
    phys = rng.permutation(num_blocks) if permute else np.arange(num_blocks)
    block_table = np.zeros((batch, max(max_blocks, 1)), dtype=np.int32)
    off = 0
    for b in range(batch):
        block_table[b, :nblk[b]] = phys[off:off + nblk[b]]
        off += int(nblk[b])
    kv_b = f32_to_bf16_bits(rng.standard_normal((heads * (NOPE + VDIM), LATENT),
                                                dtype=np.float32) * np.float32(1 / math.sqrt(512)))
    rms_w = f32_to_bf16_bits(np.float32(1.0) + rng.standard_normal(LATENT, dtype=np.float32)
                             * np.float32(math.sqrt(0.1)))
    cache = np.full((num_blocks, PAGE, ENTRY), SENTINEL, dtype=np.uint16)
    for b in range(batch):
        n_prefix = int(seq_lens[b]) - q_len
        if n_prefix <= 0:
            continue
        vals = f32_to_bf16_bits(rng.standard_normal((n_prefix, ENTRY), dtype=np.float32))
        t = np.arange(n_prefix)
        cache[block_table[b, t // PAGE], t % PAGE, :] = vals
    kv_a = f32_to_bf16_bits(rng.standard_normal((batch, q_len, ENTRY), dtype=np.float32))
    q = f32_to_bf16_bits(rng.standard_normal((batch, q_len, heads, NOPE + ROPE), dtype=np.float32))
    return dict(q=q, kv_b=kv_b, rms_w=rms_w, cache=cache, kv_a=kv_a,
                block_table=block_table, seq_lens=seq_lens.astype(np.int32),
                batch=batch, q_len=q_len, heads=heads, eps=EPS, rope_base=ROPE_BASE,
                softmax_scale=1.0 / math.sqrt(NOPE + ROPE))


def make_index_inputs(d: dict, index_heads: int = 64, dim: int = 128, seed: int = 1) -> dict:
    """Seeded inputs of the sparse-attention index for workload ``d``: FP8
    (E4M3) codes drawn uniformly over the finite codes (the two NaN codes
    0x7F / 0xFF replaced by their neighbours), one query of ``index_heads``
    heads per sequence, one key per cache slot (paged like the latent cache),
    per-head weights ~ N(0, 1), per-key scales ~ U[0.25, 1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    nb = d["cache"].shape[0]

    def codes(shape):
        c = rng.integers(0, 256, size=shape, dtype=np.int64).astype(np.uint8)
        c[c == 0x7F] = 0x7E
        c[c == 0xFF] = 0xFE
        return c

    return dict(index_q=codes((d["batch"], index_heads, dim)),
                index_w=rng.standard_normal((d["batch"], index_heads), dtype=np.float32),
                index_k=codes((nb, PAGE, dim)),
                index_k_scale=rng.uniform(0.25, 1.0, size=(nb, PAGE)).astype(np.float32),
                index_heads=index_heads, index_dim=dim)


def make_workload(name: str) -> dict:
    w = WORKLOADS[name]
    d = make_inputs(w.batch, w.q_len, w.heads, w.lens, w.permute, w.seed)
    d["name"] = name
    return d


# ---------------------------------------------------------------------------
# Work accounting (algorithmic bytes and flops of one decode call)
# ---------------------------------------------------------------------------

BYTES_PER_TOKEN = ENTRY * 2  # one cache entry in bf16


def decode_bytes(seq_lens, batch: int, q_len: int, heads: int, bt_entries: int = 0,
                 row_bytes: int = BYTES_PER_TOKEN) -> int:
    """Bytes a decode call must move at minimum: every visible cache entry
    once (``row_bytes`` each: 1152 for the bf16 cache, 656 for the FP8 rows),
    kv_b once, q in, out back, the block table."""
    total_tokens = int(np.sum(seq_lens))
    return (total_tokens * row_bytes
            + heads * (NOPE + VDIM) * LATENT * 2
            + batch * q_len * heads * (NOPE + ROPE) * 2
            + batch * q_len * heads * VDIM * 2
            + 4 * bt_entries + 4 * batch)


def visible_pairs(seq_lens, q_len: int) -> int:
    """Number of (query, cache position) pairs the causal rule lets through:
    new query i of a length-L sequence sees L - q_len + i + 1 positions."""
    s = int(np.sum(seq_lens))
    return q_len * s - len(seq_lens) * q_len * (q_len - 1) // 2


def decode_flops(seq_lens, batch: int, q_len: int, heads: int) -> int:
    """Flops of the absorbed form: scores over 576 and P*c over 512 per head and
    visible (query, position) pair, plus the two per-head projections
    (2 flops per multiply-add)."""
    return (2 * heads * visible_pairs(seq_lens, q_len) * (ENTRY + LATENT)
            + 2 * 2 * batch * q_len * heads * NOPE * LATENT)


def expanded_macs(heads: int, length: int) -> tuple[int, int]:
    """Multiply-adds of one query over ``length`` positions in the expanded
    form: (decompressing every latent into all heads' K and V,
    the attention itself over 192-wide keys and 128-wide values)."""
    return (length * LATENT * heads * (NOPE + VDIM),
            heads * length * (NOPE + ROPE + VDIM))


def prefill_flops(seq_lens, q_len: int, heads: int) -> tuple[int, int]:
    """Flops of a prefill in the expanded form: (expanding every cached latent
    of the batch into all heads' k_nope and v, the attention over 192-wide
    keys and 128-wide values for every visible (query, position) pair)."""
    return (2 * int(np.sum(seq_lens)) * LATENT * heads * (NOPE + VDIM),
            2 * heads * visible_pairs(seq_lens, q_len) * (NOPE + ROPE + VDIM))


def insert_bytes(batch: int, q_len: int) -> int:
    return batch * q_len * ENTRY * 2 * 2 + LATENT * 2 + 8 * batch


# Workloads whose cache fits in the 256 MB last-level cache (Infinity Cache)
# of the MI355X are timed cold: that cache is flushed before every step.
LLC_BYTES = 256 << 20


def fits_llc(d: dict) -> bool:
    return decode_bytes(d["seq_lens"], d["batch"], d["q_len"], d["heads"]) < LLC_BYTES


INDEX_BYTES_PER_TOKEN = 128 + 4 + 4  # E4M3 key, its fp32 scale, the fp32 score written


def index_bytes(seq_lens, batch: int, index_heads: int) -> int:
    """Bytes the index-score launch must move: every cached position's key,
    scale and score, the queries and weights once."""
    return int(np.sum(seq_lens)) * INDEX_BYTES_PER_TOKEN + batch * index_heads * (128 + 4)


def gather_bytes(kept: int) -> int:
    """Bytes the gather launch moves: each kept row read and written once."""
    return kept * BYTES_PER_TOKEN * 2
