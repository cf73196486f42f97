"""Prefill (expanded form, many new tokens) — oracle pins and ABI checks (no GPU).

The prefill computes the function of the decode with a long q_len
("深度解读DeepSeek：源码解读 DeepSeek-V3", section MLA, "(a) Naive实现";
causal rule from "DeepSeek-V3.2-Exp unboxing", 初步研读, triu(1) moved to the
cache offset).  The oracle for it is ``decode_expanded``; these pins check
what a long q_len adds: a prompt's first row has one visible position, and
every row of a prefill equals a one-query decode of the sequence cut right
after that row's own position (the row sees exactly that prefix).
"""
import ctypes

import numpy as np
import pytest

import workloads as wl
from oracle import bf16_bits_to_f64, cache_insert, decode_expanded


def _filled(d):
    return cache_insert(d["cache"], d["kv_a"], d["rms_w"], d["block_table"], d["seq_lens"],
                        d["q_len"], float(np.float32(wl.EPS)), wl.ROPE_BASE, wl.LATENT)


def test_prompt_first_row_is_the_first_value():
    d = wl.make_inputs(2, 40, 16, [40, 40], permute=True, seed=31)  # prompts, no prefix
    cache = _filled(d)
    out = decode_expanded(d["q"], d["kv_b"], cache, d["block_table"], d["seq_lens"], 40)
    w_uv = bf16_bits_to_f64(d["kv_b"]).reshape(16, 256, 512)[:, 128:, :]
    for b in range(2):
        c0 = bf16_bits_to_f64(cache[d["block_table"][b, 0], 0, :512])
        assert np.allclose(out[b, 0], w_uv @ c0, rtol=1e-12, atol=1e-12)


def test_prefill_rows_equal_decodes_of_their_prefixes():
    d = wl.make_inputs(2, 12, 16, [12, 75], permute=True, seed=32)   # a prompt and a chunk
    cache = _filled(d)
    full = decode_expanded(d["q"], d["kv_b"], cache, d["block_table"], d["seq_lens"], 12)
    for b in range(2):
        for i in (0, 5, 11):
            length = int(d["seq_lens"][b]) - 12 + i + 1
            one = decode_expanded(d["q"][b:b + 1, i:i + 1], d["kv_b"], cache,
                                  d["block_table"][b:b + 1], np.array([length], np.int32), 1)
            assert np.allclose(full[b, i], one[0, 0], rtol=1e-12, atol=1e-12)


def test_prefill_abi_checks_without_gpu():
    from mla_latent_kv_07_amd import _lib
    lib = _lib.load()
    d = _lib.dims(16)
    FAKE = 16
    need = lib.mla_prefill_workspace_bytes(ctypes.byref(d), 2, 4096)
    assert need >= 2 * 16 * 4096 * (192 + 128) * 2
    assert lib.mla_prefill_workspace_bytes(ctypes.byref(d), 2, 0) == 0
    assert lib.mla_prefill_workspace_bytes(ctypes.byref(_lib.dims(8)), 2, 64) == 0
    call = lambda **kw: lib.mla_prefill(
        kw.get("dims", ctypes.byref(d)), FAKE, FAKE, FAKE, 10, FAKE, kw.get("bt_stride", 64),
        FAKE, 2, kw.get("q_len", 100), kw.get("max_len", 4096), kw.get("scale", 0.07), FAKE,
        kw.get("ws", FAKE), kw.get("ws_bytes", need), None)
    assert call(dims=None) == 1                       # MLA_ERR_NULL
    assert call(q_len=5000) == 2                      # q_len > max_seq_len
    assert call(bt_stride=63) == 2                    # table narrower than 4096 / 64 pages
    assert call(scale=float("nan")) == 2
    assert call(ws=None) == 4 and call(ws_bytes=need - 1) == 4
    assert call(dims=ctypes.byref(_lib.dims(24))) == 3  # heads not a multiple of 16
