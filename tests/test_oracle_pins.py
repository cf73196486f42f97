"""Pins for the float64 CPU oracle (no GPU).

Each test checks the oracle against something other than itself: values
derived by hand from the pages' definitions, identities the pages state,
invariants, a library routine, or pure-Python brute force.  Sources:

* "深度解读DeepSeek：源码解读 DeepSeek-V3", section MLA, "(a) Naive实现" and
  "(b) 优化实现"  (expanded and absorbed forms);
* "DeepSeek-V2-Lite 模型结构详解", §四 RMSNorm (row rule, float32 rule, row
  independence) and §五 MLA (576-number entry, absorption identities,
  decode-cost figures);
* the "DeepSeek" tag page, excerpt on the 1/sqrt(d_k) scale;
* "DeepSeek-V3.2-Exp unboxing", 初步研读 (the triu(1) causal mask).
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import (bf16_bits_to_f64, cache_insert, decode_absorbed, decode_expanded,
                    f64_to_bf16_bits, rmsnorm_bf16, rope_bf16, rope_pairs_f64)
from oracle.brute import decode_brute, rmsnorm_brute
import workloads as wl

HERE = os.path.dirname(os.path.abspath(__file__))


def bits(x):
    return f64_to_bf16_bits(np.asarray(x, dtype=np.float64))


# ---------------------------------------------------------------- bf16 -----

def test_bf16_known_patterns():
    cases = {
        1.0: 0x3F80, -2.5: 0xC020, 0.0: 0x0000,
        1.0 + 2.0 ** -8: 0x3F80,            # tie -> even (down)
        1.0 + 3 * 2.0 ** -8: 0x3F82,        # tie -> even (up)
        1.0 + 2.0 ** -8 + 2.0 ** -40: 0x3F81,  # just above the tie: no double rounding
        2.0 ** -130: 0x0008,                # subnormal, quantum 2**-133
        1e39: 0x7F80,                       # overflow to +inf
        3.0e38: 0x7F62,
    }
    got = f64_to_bf16_bits(np.array(list(cases.keys())))
    assert [int(g) for g in got] == list(cases.values())
    assert bf16_bits_to_f64(np.array([0x3F80, 0xC020, 0x7F80], np.uint16)).tolist() == [1.0, -2.5, math.inf]


def test_bf16_matches_torch_on_float32_inputs():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(200_000) * np.exp(rng.uniform(-20, 20, 200_000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f64_to_bf16_bits(x.astype(np.float64)), ref)


# ------------------------------------------------------------- RMSNorm -----

def test_rmsnorm_closed_forms():
    # constant row: x / rms(x) == 1 exactly (eps = 0), so the output is the weight
    w = bits([1.5, -0.75, 2.0, 0.125])
    x = bits([2.0, 2.0, 2.0, 2.0])
    assert np.array_equal(rmsnorm_bf16(x, w, 0.0), w)
    # [3, 4]: rms = sqrt(12.5); n = [0.8485.., 1.1313..] (hand-derived)
    out = bf16_bits_to_f64(rmsnorm_bf16(bits([3.0, 4.0]), bits([1.0, 1.0]), 0.0))
    assert np.allclose(out, [3 / math.sqrt(12.5), 4 / math.sqrt(12.5)], rtol=2 ** -8)


def test_rmsnorm_row_rms_is_one_before_weight():
    rng = np.random.default_rng(2)
    x = wl.f32_to_bf16_bits(rng.standard_normal((64, 512), dtype=np.float32) * 3)
    ones = bits(np.ones(512))
    n = bf16_bits_to_f64(rmsnorm_bf16(x, ones, 1e-6))
    rms = np.sqrt(np.mean(n * n, axis=-1))
    xf = bf16_bits_to_f64(x)
    ms = np.mean(xf * xf, axis=-1)
    assert np.allclose(rms, np.sqrt(ms / (ms + 1e-6)), atol=2 ** -8)
    assert np.all(np.abs(rms - 1) < 2 ** -8)


def test_rmsnorm_rows_independent():
    rng = np.random.default_rng(3)
    x = wl.f32_to_bf16_bits(rng.standard_normal((5, 512), dtype=np.float32))
    w = wl.f32_to_bf16_bits(1 + rng.standard_normal(512, dtype=np.float32) * 0.3)
    y0 = rmsnorm_bf16(x, w, 1e-6)
    x2 = x.copy()
    x2[0] = bits(bf16_bits_to_f64(x[0]) * 100)
    y1 = rmsnorm_bf16(x2, w, 1e-6)
    assert np.array_equal(y0[1:], y1[1:])


def test_rmsnorm_vs_brute():
    rng = np.random.default_rng(4)
    x = wl.f32_to_bf16_bits(rng.standard_normal((8, 16), dtype=np.float32))
    w = wl.f32_to_bf16_bits(1 + rng.standard_normal(16, dtype=np.float32) * 0.3)
    got = bf16_bits_to_f64(rmsnorm_bf16(x, w, 1e-6))
    xf, wf = bf16_bits_to_f64(x), bf16_bits_to_f64(w)
    for r in range(8):
        ref = np.array(rmsnorm_brute(xf[r].tolist(), wf.tolist(), 1e-6))
        # two bf16 roundings: within 2**-7 relative of the exact value
        assert np.all(np.abs(got[r] - ref) <= 2 ** -7 * np.abs(ref) + 1e-30)


# ---------------------------------------------------------------- RoPE -----

def test_rope_closed_forms():
    x = np.zeros(64)
    x[0] = 1.0
    y = rope_pairs_f64(x, np.array(1.0), 10000.0)
    assert np.allclose(y[:2], [math.cos(1.0), math.sin(1.0)], atol=1e-15)
    assert np.all(y[2:] == 0)
    x = np.zeros(64)
    x[2] = 1.0  # pair j = 1 turns by pos * 10000**(-2/64)
    th = 3 * 10000.0 ** (-2.0 / 64)
    y = rope_pairs_f64(x, np.array(3.0), 10000.0)
    assert np.allclose(y[2:4], [math.cos(th), math.sin(th)], atol=1e-15)
    assert y[0] == 0 and y[1] == 0 and np.all(y[4:] == 0)


def test_rope_identity_at_zero_and_norm_and_relative():
    rng = np.random.default_rng(5)
    x = wl.f32_to_bf16_bits(rng.standard_normal((10, 64), dtype=np.float32))
    assert np.array_equal(rope_bf16(x, np.zeros(10), 10000.0), x)
    xf = bf16_bits_to_f64(x)
    pos = rng.integers(0, 40000, size=10).astype(np.float64)
    y = rope_pairs_f64(xf, pos, 10000.0)
    assert np.allclose(np.hypot(y[:, 0::2], y[:, 1::2]), np.hypot(xf[:, 0::2], xf[:, 1::2]), rtol=1e-12)
    q, k = xf[0], xf[1]
    a = rope_pairs_f64(q, np.array(700.0), 10000.0) @ rope_pairs_f64(k, np.array(300.0), 10000.0)
    b = rope_pairs_f64(q, np.array(1400.0), 10000.0) @ rope_pairs_f64(k, np.array(1000.0), 10000.0)
    assert abs(a - b) < 1e-9 * (1 + abs(a))


# -------------------------------------------------------------- insert -----

@pytest.mark.parametrize("permute", [False, True])
def test_cache_insert_indexing(permute):
    d = wl.make_inputs(3, 2, 16, [65, 2, 130], permute=permute, seed=11, spare_blocks=2)
    out = cache_insert(d["cache"], d["kv_a"], d["rms_w"], d["block_table"], d["seq_lens"],
                       2, 1e-6, 10000.0, 512)
    written = np.zeros(out.shape[:2], dtype=bool)
    for b, length in enumerate(d["seq_lens"]):
        for i in range(2):
            p = int(length) - 2 + i
            blk = int(d["block_table"][b, p // 64])
            if not permute:
                # identity table: the physical slot is the sequence's own numbering
                assert blk == sum((int(x) + 63) // 64 for x in d["seq_lens"][:b]) + p // 64
            written[blk, p % 64] = True
            lat = rmsnorm_bf16(d["kv_a"][b, i:i + 1, :512], d["rms_w"], 1e-6)[0]
            pe = rope_bf16(d["kv_a"][b, i:i + 1, 512:], np.array([p]), 10000.0)[0]
            assert np.array_equal(out[blk, p % 64, :512], lat)
            assert np.array_equal(out[blk, p % 64, 512:], pe)
    assert written.sum() == 6
    assert np.array_equal(out[~written], d["cache"][~written])


# -------------------------------------------------------------- decode -----

def tiny_inputs(rng, q_len, length, heads, latent, rope, nope, v_dim):
    f = lambda *s: wl.f32_to_bf16_bits(rng.standard_normal(s, dtype=np.float32))
    q = f(1, q_len, heads, nope + rope)
    kv_b = f(heads * (nope + v_dim), latent)
    cache = f(1, length, latent + rope)  # one page holding the whole sequence
    bt = np.zeros((1, 1), np.int32)
    return q, kv_b, cache, bt, np.array([length], np.int32)


@pytest.mark.parametrize("seed", range(6))
def test_decode_vs_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    q_len = 1 + seed % 2
    length = int(rng.integers(q_len, 6))
    dims = dict(latent=4, rope=2, nope=2, v_dim=3)
    q, kv_b, cache, bt, sl = tiny_inputs(rng, q_len, length, 2, **dims)
    got = decode_expanded(q, kv_b, cache, bt, sl, q_len, **dims)
    scale = 1 / math.sqrt(dims["nope"] + dims["rope"])
    ref = decode_brute(bf16_bits_to_f64(q[0]).tolist(), bf16_bits_to_f64(kv_b).tolist(),
                       bf16_bits_to_f64(cache[0]).tolist(), length, q_len,
                       dims["nope"], dims["rope"], dims["v_dim"], scale)
    assert np.allclose(got[0], np.array(ref), rtol=1e-12, atol=1e-14)


def test_decode_two_token_closed_form():
    # dims nope=1, rope=3 -> d_k = 4, scale exactly 1/2.  kv_b rows: W_UK = [1],
    # W_UV = [0.5].  c = [0, 1], k_pe = 0, q_nope = 2 -> scores [0, 1].
    # Softmax gives p1 = e/(1+e); output = 0.5 * p1 * c_1.
    dims = dict(latent=1, rope=3, nope=1, v_dim=1)
    q = bits([[[[2.0, 0.0, 0.0, 0.0]]]])
    kv_b = bits([[1.0], [0.5]])
    cache = bits([[[0.0, 0, 0, 0], [1.0, 0, 0, 0]]])
    bt, sl = np.zeros((1, 1), np.int32), np.array([2], np.int32)
    out = decode_expanded(q, kv_b, cache, bt, sl, 1, **dims)
    assert abs(out[0, 0, 0, 0] - 0.5 * math.e / (1 + math.e)) < 1e-15
    # q_len = 2: the first new query must not see position 1 (causal), so it
    # returns 0.5 * c_0 = 0; the second sees both.
    q2 = bits([[[[2.0, 0, 0, 0]], [[2.0, 0, 0, 0]]]])
    out2 = decode_expanded(q2, kv_b, cache, bt, sl, 2, **dims)
    assert out2[0, 0, 0, 0] == 0.0
    assert abs(out2[0, 1, 0, 0] - 0.5 * math.e / (1 + math.e)) < 1e-15


def test_decode_absorbed_equals_expanded():
    d = wl.make_inputs(3, 2, 16, [2, 70, 190], permute=True, seed=7)
    cache = cache_insert(d["cache"], d["kv_a"], d["rms_w"], d["block_table"], d["seq_lens"],
                         2, 1e-6, 10000.0, 512)
    e = decode_expanded(d["q"], d["kv_b"], cache, d["block_table"], d["seq_lens"], 2, chunk=50)
    a = decode_absorbed(d["q"], d["kv_b"], cache, d["block_table"], d["seq_lens"], 2)
    assert np.max(np.abs(e - a)) <= 1e-12 * np.max(np.abs(e))


def test_decode_softmax_rows_sum_to_one_and_mask():
    d = wl.make_inputs(2, 2, 16, [5, 100], permute=True, seed=8)
    cache = cache_insert(d["cache"], d["kv_a"], d["rms_w"], d["block_table"], d["seq_lens"],
                         2, 1e-6, 10000.0, 512)
    _, probs = decode_expanded(d["q"], d["kv_b"], cache, d["block_table"], d["seq_lens"], 2,
                               return_probs=True)
    for p, length in zip(probs, d["seq_lens"]):
        assert np.allclose(p.sum(-1), 1.0, atol=1e-12)
        assert np.all(p[0, :, length - 1] == 0)      # query 0 cannot see the last token
        assert np.all(p[1, :, length - 1] > 0)


def test_decode_single_token_returns_its_value():
    d = wl.make_inputs(1, 1, 16, [1], permute=False, seed=9)
    cache = cache_insert(d["cache"], d["kv_a"], d["rms_w"], d["block_table"], d["seq_lens"],
                         1, 1e-6, 10000.0, 512)
    out = decode_expanded(d["q"], d["kv_b"], cache, d["block_table"], d["seq_lens"], 1)
    c0 = bf16_bits_to_f64(cache[d["block_table"][0, 0], 0, :512])
    w = bf16_bits_to_f64(d["kv_b"])
    for h in range(16):
        w_uv = w[h * 256 + 128: h * 256 + 256]      # the last 128 rows of head h's block
        assert np.allclose(out[0, 0, h], w_uv @ c0, rtol=1e-12, atol=1e-14)


def test_decode_zero_query_is_uniform_average():
    d = wl.make_inputs(2, 2, 16, [3, 77], permute=True, seed=10)
    d["q"][:] = 0
    cache = cache_insert(d["cache"], d["kv_a"], d["rms_w"], d["block_table"], d["seq_lens"],
                         2, 1e-6, 10000.0, 512)
    out = decode_expanded(d["q"], d["kv_b"], cache, d["block_table"], d["seq_lens"], 2)
    w = bf16_bits_to_f64(d["kv_b"])
    for b, length in enumerate(d["seq_lens"]):
        t = np.arange(length)
        c = bf16_bits_to_f64(cache[d["block_table"][b, t // 64], t % 64, :512])
        for i in range(2):
            mean_c = c[:length - 1 + i].mean(0)
            for h in (0, 5, 15):
                ref = w[h * 256 + 128: h * 256 + 256] @ mean_c
                assert np.allclose(out[b, i, h], ref, rtol=1e-12, atol=1e-14)


def test_decode_paging_invariance_and_subsets():
    a = wl.make_inputs(2, 1, 16, [130, 64], permute=False, seed=12)
    b = wl.make_inputs(2, 1, 16, [130, 64], permute=True, seed=12)
    # same draws except the table permutation: rebuild b's cache from a's logical rows
    cache_b = np.full_like(a["cache"], wl.SENTINEL)
    for s, length in enumerate(a["seq_lens"]):
        t = np.arange(length)
        cache_b[b["block_table"][s, t // 64], t % 64] = a["cache"][a["block_table"][s, t // 64], t % 64]
    ins = lambda d, c: cache_insert(c, d["kv_a"], d["rms_w"], d["block_table"], d["seq_lens"],
                                    1, 1e-6, 10000.0, 512)
    ca, cb = ins(a, a["cache"]), ins(a | {"block_table": b["block_table"]}, cache_b)
    oa = decode_expanded(a["q"], a["kv_b"], ca, a["block_table"], a["seq_lens"], 1)
    ob = decode_expanded(a["q"], a["kv_b"], cb, b["block_table"], a["seq_lens"], 1)
    assert np.array_equal(oa, ob)
    sub = decode_expanded(a["q"], a["kv_b"], ca, a["block_table"], a["seq_lens"], 1,
                          batches=[1], heads=[3, 9])
    assert np.allclose(sub[0], oa[1][:, [3, 9]], rtol=1e-13, atol=1e-15)


# ------------------------------------------------- printed page numbers -----

def test_page_numbers_pin_accounting():
    g = json.load(open(os.path.join(HERE, "golden", "page_numbers.json")))
    assert wl.ENTRY == g["mla_cached_numbers_per_token_layer"] == g["mla_latent"] + g["mla_rope"]
    assert g["mha_k_width"] + g["mha_v_width"] == g["mha_cached_numbers_per_token_layer"]
    assert wl.BYTES_PER_TOKEN == 2 * 576
    dec, att = wl.expanded_macs(g["heads"], g["context"])
    assert f"{dec / 1e9:.1f}G" == g["decompress_macs_at_8192"]
    assert f"{att / 1e6:.1f}M" == g["attention_macs_at_8192"]
    assert 400 <= dec / att < 410


def test_rmsnorm_eps_inside_the_root():
    # rows with mean square ~ eps: the page puts eps under the square root,
    # so the normalised row has rms sqrt(ms / (ms + eps)), well below 1 here
    rng = np.random.default_rng(13)
    x = wl.f32_to_bf16_bits(rng.standard_normal((16, 512), dtype=np.float32) * 1e-3)
    n = bf16_bits_to_f64(rmsnorm_bf16(x, bits(np.ones(512)), 1e-6))
    xf = bf16_bits_to_f64(x)
    ms = np.mean(xf * xf, axis=-1)
    assert np.allclose(np.sqrt(np.mean(n * n, -1)), np.sqrt(ms / (ms + 1e-6)), rtol=2 ** -8)


def test_rmsnorm_rounding_points_match_page_listing_run_by_torch():
    # The RMSNorm listing on the V2-Lite page (§四, 精度): float32 normalise,
    # convert to the activation dtype, then weight * value.  Run it with torch
    # in float32 and compare: the oracle normalises in float64, so it may differ
    # by one ulp where float32 error crosses a rounding boundary, but only rarely.
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(14)
    x = wl.f32_to_bf16_bits(rng.standard_normal((256, 512), dtype=np.float32))
    w = wl.f32_to_bf16_bits(1 + rng.standard_normal(512, dtype=np.float32) * np.float32(0.316))
    tb = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    xt, wt = tb(x), tb(w)
    xf = xt.float()
    xf = xf * torch.rsqrt(xf.pow(2).mean(-1, keepdim=True) + 1e-6)
    ref = (wt * xf.to(torch.bfloat16)).view(torch.int16).numpy().view(np.uint16)
    got = rmsnorm_bf16(x, w, 1e-6)
    diff = np.abs(got.astype(np.int32) - ref.astype(np.int32))
    assert diff.max() <= 1
    assert np.mean(diff != 0) < 2e-3
