"""Pins for the sparse-attention oracle (oracle/dsa.py; no GPU).

Source: "DeepSeek-V3.2-Exp unboxing", 初步研读 (the FP8 index kernel's
signature: per-head weights, per-key scale; top-k selection of the cached
tokens before the attention).  The index score is checked against values
worked out by hand from E4M3 codes; the selection against a plain sort with
the tie rule; the sparse decode against the dense decode where they must
agree (all positions kept; a kept prefix; one kept position).
"""
import numpy as np

import workloads as wl
from oracle import bf16_bits_to_f64, cache_insert, decode_expanded
from oracle import dsa


def _filled(d):
    return cache_insert(d["cache"], d["kv_a"], d["rms_w"], d["block_table"], d["seq_lens"],
                        d["q_len"], float(np.float32(wl.EPS)), wl.ROPE_BASE, wl.LATENT)


def test_index_score_worked_by_hand():
    # 2 heads; head 0's query is 1.0 (0x38) in dim 3, head 1's is 0.5 (0x30)
    # in dim 5; keys: dim 3 = 2.0 (0x40), dim 5 = -4.0 (0xC8); weights 3, -1
    nb, page, dim = 2, 64, 128
    q = np.zeros((1, 2, dim), dtype=np.uint8)
    q[0, 0, 3] = 0x38
    q[0, 1, 5] = 0x30
    w = np.array([[3.0, -1.0]], dtype=np.float32)
    k = np.zeros((nb, page, dim), dtype=np.uint8)
    k[:, :, 3] = 0x40
    k[:, :, 5] = 0xC8
    k[1, 7, 3] = 0x48  # 4.0 at one slot
    ks = np.full((nb, page), 0.5, dtype=np.float32)
    bt = np.array([[1, 0]], dtype=np.int32)
    s = dsa.index_scores(q, w, k, ks, bt, 100, 0)
    # 3 * (1.0 * 2.0) - 1 * (0.5 * -4.0) = 8, times 0.5
    expect = np.full(100, 4.0)
    expect[7] = (3 * 4.0 + 2.0) * 0.5   # position 7 sits in physical block 1, slot 7
    assert np.array_equal(s, expect)


def test_index_score_is_linear_in_weights_and_key_scale():
    d = wl.make_inputs(2, 1, 16, [130, 70], permute=True, seed=61)
    ix = wl.make_index_inputs(d, index_heads=8, seed=62)
    a = dsa.index_scores(ix["index_q"], ix["index_w"], ix["index_k"], ix["index_k_scale"],
                         d["block_table"], 130, 0)
    b = dsa.index_scores(ix["index_q"], 2 * ix["index_w"], ix["index_k"],
                         4 * ix["index_k_scale"], d["block_table"], 130, 0)
    assert np.allclose(b, 8 * a, rtol=1e-12, atol=1e-9)


def test_topk_ties_and_order():
    s = np.array([3.0, 1.0, 3.0, 2.0, 3.0])
    assert dsa.topk_positions(s, 2).tolist() == [0, 2]
    assert dsa.topk_positions(s, 4).tolist() == [0, 2, 3, 4]
    assert dsa.topk_positions(s, 10).tolist() == [0, 1, 2, 3, 4]
    rng = np.random.default_rng(63)
    for _ in range(50):
        n = int(rng.integers(1, 300))
        sc = rng.integers(-5, 6, size=n).astype(np.float64)   # many ties
        k = int(rng.integers(1, n + 5))
        ref = sorted(sorted(range(n), key=lambda i: (-sc[i], i))[:k])
        assert dsa.topk_positions(sc, k).tolist() == ref


def test_sparse_decode_with_every_position_is_the_dense_decode():
    d = wl.make_inputs(3, 1, 16, [65, 200, 1], permute=True, seed=64)
    cache = _filled(d)
    pos = [np.arange(int(L)) for L in d["seq_lens"]]
    a = dsa.decode_sparse(d["q"], d["kv_b"], cache, d["block_table"], d["seq_lens"], pos)
    b = decode_expanded(d["q"], d["kv_b"], cache, d["block_table"], d["seq_lens"], 1)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


def test_sparse_decode_of_a_prefix_is_the_truncated_decode():
    d = wl.make_inputs(2, 1, 16, [300, 90], permute=True, seed=65)
    cache = _filled(d)
    keep = [130, 64]
    pos = [np.arange(c) for c in keep]
    a = dsa.decode_sparse(d["q"], d["kv_b"], cache, d["block_table"], d["seq_lens"], pos)
    b = decode_expanded(d["q"], d["kv_b"], cache, d["block_table"], np.array(keep), 1)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)


def test_sparse_decode_of_one_position_returns_its_value():
    d = wl.make_inputs(1, 1, 16, [300], permute=True, seed=66)
    cache = _filled(d)
    p = 211
    out = dsa.decode_sparse(d["q"], d["kv_b"], cache, d["block_table"], d["seq_lens"], [[p]])
    w_uv = bf16_bits_to_f64(d["kv_b"]).reshape(16, 256, 512)[:, 128:, :]
    c = bf16_bits_to_f64(cache[d["block_table"][0, p // 64], p % 64, :512])
    assert np.allclose(out[0, 0], w_uv @ c, rtol=1e-12, atol=1e-12)
