"""GPU parity of the prefill path (mla_prefill: expansion of K/V through
kv_b, then causal attention with 192/128-wide heads) against the float64
expanded-form oracle, on the same seeded inputs; new tokens inserted on the
GPU first (mla_cache_insert, q_len up to the chunk length).

Bound: max-abs 2e-2 and relative RMS 5e-3 of the bf16 output, as for the
decode (bf16 operands: expanded K and V, the probabilities; fp32
accumulation and softmax statistics).
"""
import sys

import numpy as np
import pytest

import workloads as wl
from oracle import cache_insert as oracle_insert
from oracle import decode_expanded

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
REL_RMS = 5e-3
EPS32 = float(np.float32(wl.EPS))


def _torch():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def dev(a, torch):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def errors(got, ref):
    d = got - ref
    return float(np.max(np.abs(d))), float(np.sqrt(np.mean(d * d)) / np.sqrt(np.mean(ref * ref)))


def run(d, torch, cache_np=None):
    """Insert the new tokens on the GPU, then prefill; returns (out, cache)."""
    import mla_latent_kv_07_amd as mla
    cache = dev(d["cache"] if cache_np is None else cache_np, torch)
    bt, sl = dev(d["block_table"], torch), dev(d["seq_lens"], torch)
    mla.cache_insert(dev(d["kv_a"], torch), dev(d["rms_w"], torch), bt, sl, cache, eps=EPS32,
                     rope_base=wl.ROPE_BASE, heads=d["heads"])
    out = mla.prefill(dev(d["q"], torch), dev(d["kv_b"], torch), cache, bt, sl,
                      int(d["seq_lens"].max()))
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), cache


def ref_cache(d):
    return oracle_insert(d["cache"], d["kv_a"], d["rms_w"], d["block_table"], d["seq_lens"],
                         d["q_len"], EPS32, wl.ROPE_BASE, wl.LATENT)


SMALL = [  # (batch, q_len, heads, post-insert lengths, seed)
    (2, 300, 16, [300, 300], 91),        # prompts, two query blocks, ragged last key block
    (3, 64, 16, [64, 700, 1500], 92),    # a prompt and two chunks after cached prefixes
    (1, 257, 128, [1000], 93),           # 128 heads, one row into the second query block
    (2, 1, 32, [1, 77], 94),             # one new token (the decode case), one-token sequence
    (2, 8, 48, [8, 130], 95),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"B{c[0]}S{c[1]}H{c[2]}" for c in SMALL])
def test_prefill_parity_small(case):
    torch = _torch()
    bsz, q_len, heads, lens, seed = case
    say(f"[prefill small] B={bsz} S={q_len} H={heads} lens={lens}")
    d = wl.make_inputs(bsz, q_len, heads, lens, permute=True, seed=seed, spare_blocks=2)
    got, _ = run(d, torch)
    ref = decode_expanded(d["q"], d["kv_b"], ref_cache(d), d["block_table"], d["seq_lens"], q_len)
    mx, rr = errors(got, ref)
    say(f"   max-abs {mx:.3e} rel-rms {rr:.3e}")
    assert np.all(np.isfinite(got))
    assert mx <= MAX_ABS and rr <= REL_RMS


def test_prefill_agrees_with_decode_for_short_q_len():
    """Same function, two forms: mla_prefill and mla_decode on the same inputs."""
    torch = _torch()
    import mla_latent_kv_07_amd as mla
    say("[prefill] against the absorbed decode, q_len 4")
    d = wl.make_inputs(3, 4, 128, [4, 333, 2048], permute=True, seed=96)
    got, cache = run(d, torch)
    dec = mla.decode(dev(d["q"], torch), dev(d["kv_b"], torch), cache,
                     dev(d["block_table"], torch), dev(d["seq_lens"], torch),
                     int(d["seq_lens"].max())).float().cpu().numpy().astype(np.float64)
    ref = decode_expanded(d["q"], d["kv_b"], ref_cache(d), d["block_table"], d["seq_lens"], 4)
    for name, o in (("prefill", got), ("decode", dec)):
        mx, rr = errors(o, ref)
        say(f"   {name}: max-abs {mx:.3e} rel-rms {rr:.3e}")
        assert mx <= MAX_ABS and rr <= REL_RMS


def test_prefill_ignores_slots_beyond_length():
    torch = _torch()
    say("[prefill] slots beyond the sequence end")
    d = wl.make_inputs(2, 100, 16, [100, 190], permute=True, seed=97, spare_blocks=1)
    a, _ = run(d, torch)
    c2 = d["cache"].copy()
    rng = np.random.default_rng(98)
    for b, length in enumerate(d["seq_lens"]):
        for p in range(int(length), ((int(length) + 63) // 64) * 64):
            c2[d["block_table"][b, p // 64], p % 64] = rng.integers(0, 65536, 576)
    b2, _ = run(d, torch, c2)
    assert np.array_equal(a, b2)


PREFILL_SAMPLES = {  # sampled (sequence, head) pairs at full size
    "prefill_v3_b2_s4096": ([0, 1], [0, 77, 127]),
    "prefill_v3_chunk_b4": ([0, 3], [5, 100]),
}


@pytest.mark.parametrize("name", wl.PREFILL)
def test_prefill_workload(name):
    torch = _torch()
    say(f"[prefill workload] {name}")
    d = wl.make_workload(name)
    got, cache = run(d, torch)
    assert np.all(np.isfinite(got))
    bs, hs = PREFILL_SAMPLES[name]
    # the oracle reads the cache the GPU wrote (insert parity is tested on its own)
    cache_np = cache.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = decode_expanded(d["q"], d["kv_b"], cache_np, d["block_table"], d["seq_lens"],
                          d["q_len"], batches=bs, heads=hs)
    mx, rr = errors(got[bs][:, :, hs], ref)
    say(f"   max-abs {mx:.3e} rel-rms {rr:.3e}")
    assert mx <= MAX_ABS and rr <= REL_RMS


def test_prefill_wide_score_range():
    """Scores that jump by far more than the 2^8 slack partway through a row:
    the rope part of later keys is scaled by 8 (exact in bf16), in the cached
    prefix of sequence 1 (positions 300..599) and in the new tokens 150..299
    of both sequences, so each row's running reference is raised and its
    accumulators rescaled after several key blocks.  (k_pe is copied into the
    expanded keys exactly, so the larger scores add no rounding error; scaling
    the queries instead would grow the bf16 rounding of the expanded k_nope
    with the scores, beyond the bound, in either form of the method.)"""
    torch = _torch()
    say("[prefill] wide score range")
    d = wl.make_inputs(2, 300, 16, [300, 900], permute=True, seed=99, spare_blocks=1)
    up = lambda bits: wl.f32_to_bf16_bits((bits.astype(np.uint32) << 16).view(np.float32)
                                          * np.float32(8.0))
    cache = d["cache"].copy()
    t = np.arange(300, 600)
    rows = (d["block_table"][1, t // 64], t % 64)
    cache[rows[0], rows[1], 512:] = up(cache[rows[0], rows[1], 512:])
    d["cache"] = cache
    kv_a = d["kv_a"].copy()
    kv_a[:, 150:, 512:] = up(kv_a[:, 150:, 512:])
    d["kv_a"] = kv_a
    got, _ = run(d, torch)
    ref = decode_expanded(d["q"], d["kv_b"], ref_cache(d), d["block_table"], d["seq_lens"], 300)
    mx, rr = errors(got, ref)
    worst = np.unravel_index(np.argmax(np.abs(got - ref)), ref.shape)
    say(f"   max-abs {mx:.3e} rel-rms {rr:.3e}; |ref| there {abs(ref[worst]):.3f}, "
        f"max |ref| {np.max(np.abs(ref)):.3f}")
    assert np.all(np.isfinite(got))
    # Near one-hot rows return single value rows, up to |x| ~ 5 here: the bf16
    # output's own rounding is up to 2^-8 |x| (0.02 at |x| = 5), before the
    # bf16 probabilities and values add theirs, so the absolute bound grows
    # with the output: 2e-2 + 2^-7 |ref| elementwise, with the usual RMS bound.
    assert np.all(np.abs(got - ref) <= MAX_ABS + 2.0 ** -7 * np.abs(ref))
    assert rr <= REL_RMS
