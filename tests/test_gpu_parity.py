"""GPU parity: libmla (HIP, gfx950) against the float64 CPU oracle.

Decode tolerance (bf16 output of a bf16-MFMA pipeline): max-abs 2e-2 and
relative RMS 5e-3 against the float64 expanded-form oracle.  Insert: cache
indexing bit-exact (every byte outside the written entries unchanged, NaN
sentinels included), values within one bf16 ulp (expected identical).
"""
import math
import sys

import numpy as np
import pytest

import workloads as wl
from oracle import cache_insert as oracle_insert
from oracle import decode_expanded

pytestmark = pytest.mark.gpu

MAX_ABS = 2e-2
REL_RMS = 5e-3
EPS32 = float(np.float32(wl.EPS))  # the float the C ABI receives


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


def host_u16(t):
    return t.view(__import__("torch").int16).cpu().numpy().view(np.uint16)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def errors(got, ref):
    d = got - ref
    return float(np.max(np.abs(d))), float(np.sqrt(np.mean(d * d)) / np.sqrt(np.mean(ref * ref)))


def run_insert(d, torch):
    import mla_latent_kv_07_amd as mla
    cache = dev(d["cache"], torch)
    mla.cache_insert(dev(d["kv_a"], torch), dev(d["rms_w"], torch), dev(d["block_table"], torch),
                     dev(d["seq_lens"], torch), cache, eps=EPS32, rope_base=wl.ROPE_BASE,
                     heads=d["heads"])
    torch.cuda.synchronize()
    return cache


def run_decode(d, cache_dev, torch, hint=0):
    import mla_latent_kv_07_amd as mla
    out = mla.decode(dev(d["q"], torch), dev(d["kv_b"], torch), cache_dev,
                     dev(d["block_table"], torch), dev(d["seq_lens"], torch),
                     int(d["seq_lens"].max()), num_splits_hint=hint)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def ref_cache(d):
    return oracle_insert(d["cache"], d["kv_a"], d["rms_w"], d["block_table"], d["seq_lens"],
                         d["q_len"], EPS32, wl.ROPE_BASE, wl.LATENT)


def check_insert(d, got_u16, ref_u16):
    written = np.zeros(ref_u16.shape[:2], dtype=bool)
    for b, length in enumerate(d["seq_lens"]):
        for i in range(d["q_len"]):
            p = int(length) - d["q_len"] + i
            written[int(d["block_table"][b, p // 64]), p % 64] = True
    assert np.array_equal(got_u16[~written], ref_u16[~written]), "bytes outside the new entries changed"
    g = got_u16[written].astype(np.int32)
    r = ref_u16[written].astype(np.int32)
    ulps = np.abs(g - r)
    assert ulps.max() <= 1, f"insert values differ by {ulps.max()} ulp"
    assert np.mean(ulps != 0) < 1e-3


# ------------------------------------------------------------------ insert --

@pytest.mark.parametrize("name", wl.ORDER)
def test_insert_parity(name):
    torch = _torch()
    say(f"[insert] {name}")
    d = wl.make_workload(name)
    got = host_u16(run_insert(d, torch))
    check_insert(d, got, ref_cache(d))


def test_insert_edge_cases():
    torch = _torch()
    say("[insert] edge cases")
    # lengths at page boundaries, q_len 3, spare blocks, permuted table
    d = wl.make_inputs(5, 3, 16, [3, 63, 64, 65, 130], permute=True, seed=21, spare_blocks=3)
    got = host_u16(run_insert(d, torch))
    check_insert(d, got, ref_cache(d))


# ------------------------------------------------------------------ decode --

SMALL = [
    # (batch, q_len, heads, lens, seed): several 64-position pages, ragged tails
    (4, 1, 16, [1, 63, 64, 200], 31),
    (3, 2, 16, [2, 65, 330], 32),
    (3, 1, 128, [1, 129, 300], 33),
    (2, 2, 128, [2, 191], 34),
    (2, 1, 32, [100, 257], 35),
    (2, 1, 48, [77, 64], 36),
    (2, 4, 64, [4, 150], 37),
    (1, 8, 16, [70], 38),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"B{c[0]}q{c[1]}H{c[2]}" for c in SMALL])
def test_decode_parity_small(case):
    torch = _torch()
    bsz, q_len, heads, lens, seed = case
    say(f"[decode small] B={bsz} q_len={q_len} H={heads} lens={lens}")
    d = wl.make_inputs(bsz, q_len, heads, lens, permute=True, seed=seed, spare_blocks=2)
    cache = ref_cache(d)
    got = run_decode(d, dev(cache, torch), torch)
    ref = decode_expanded(d["q"], d["kv_b"], cache, d["block_table"], d["seq_lens"], q_len)
    mx, rr = errors(got, ref)
    say(f"   max-abs {mx:.3e} rel-rms {rr:.3e}")
    assert np.all(np.isfinite(got))
    assert mx <= MAX_ABS and rr <= REL_RMS


# Sequences the oracle checks at full size: every sequence (all heads, all
# query tokens) except for the 128-sequence multi-token workload, where every
# fourth sequence is checked (32 sequences spread over the whole item list, so
# over every XCD's range of work items), all 128 heads and both tokens.
FULL_BATCHES = {"v3_mtp_b128": list(range(0, 128, 4))}


@pytest.mark.parametrize("name", wl.ORDER)
def test_decode_parity_workload(name):
    """Full-size workload, chained insert -> decode on the GPU, in the launch
    configuration the benchmark times (automatic split plan); every output
    element of the checked sequences is compared with the float64 oracle."""
    torch = _torch()
    say(f"[decode workload] {name}")
    d = wl.make_workload(name)
    cache_dev = run_insert(d, torch)
    got = run_decode(d, cache_dev, torch)
    assert np.all(np.isfinite(got))
    cache = ref_cache(d)
    bs = FULL_BATCHES.get(name, list(range(d["batch"])))
    say(f"   oracle over {len(bs)} of {d['batch']} sequences, all {d['heads']} heads")
    ref = decode_expanded(d["q"], d["kv_b"], cache, d["block_table"], d["seq_lens"], d["q_len"],
                          batches=bs)
    mx, rr = errors(got[bs], ref)
    say(f"   max-abs {mx:.3e} rel-rms {rr:.3e}")
    assert mx <= MAX_ABS and rr <= REL_RMS


def test_decode_step_parity_v3_full():
    """The benchmarked path at its full size: mla_decode_step (insert of the
    new token, RoPE on q_pe, absorption, split-KV decode, combine) on the
    64 x 8192 V3 workload; every output element against the float64 oracle
    run on the oracle's insert and the oracle-rotated query."""
    torch = _torch()
    import mla_latent_kv_07_amd as mla
    from oracle import rotate_q
    say("[decode step] v3_b64_l8192 full size")
    d = wl.make_workload("v3_b64_l8192")
    cache_dev = dev(d["cache"], torch)
    out = mla.decode_step(dev(d["q"], torch), dev(d["kv_a"], torch), dev(d["rms_w"], torch),
                          dev(d["kv_b"], torch), cache_dev, dev(d["block_table"], torch),
                          dev(d["seq_lens"], torch), int(d["seq_lens"].max()), eps=EPS32)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    cache = ref_cache(d)
    check_insert(d, host_u16(cache_dev), cache)
    q_rot = rotate_q(d["q"], d["seq_lens"], 1, wl.ROPE_BASE, wl.NOPE)
    ref = decode_expanded(q_rot, d["kv_b"], cache, d["block_table"], d["seq_lens"], 1)
    mx, rr = errors(got, ref)
    say(f"   max-abs {mx:.3e} rel-rms {rr:.3e}")
    assert mx <= MAX_ABS and rr <= REL_RMS


def test_decode_split_invariance():
    torch = _torch()
    say("[decode] split invariance")
    d = wl.make_inputs(3, 2, 128, [700, 1500, 64], permute=True, seed=41)
    cache = ref_cache(d)
    cd = dev(cache, torch)
    ref = decode_expanded(d["q"], d["kv_b"], cache, d["block_table"], d["seq_lens"], 2)
    outs = {h: run_decode(d, cd, torch, hint=h) for h in (0, 1, 3, 24)}
    for h, o in outs.items():
        mx, rr = errors(o, ref)
        say(f"   hint {h}: max-abs {mx:.3e} rel-rms {rr:.3e}")
        assert mx <= MAX_ABS and rr <= REL_RMS
    # different split counts only change the fp32 merge order
    for h in (1, 3, 24):
        assert np.max(np.abs(outs[h] - outs[0])) <= 2e-2


def test_decode_one_long_sequence_many_splits():
    """One 32768-position sequence: the automatic plan cuts it into far more
    than 64 items (the merge's lane-parallel weights then take several blocks
    of 64 splits, split over the merge's wavefronts), q_len 1 and 2."""
    torch = _torch()
    for q_len in (1, 2):
        say(f"[decode] one sequence of 32768, q_len {q_len}")
        d = wl.make_inputs(1, q_len, 128, [32768], permute=True, seed=47 + q_len)
        cache = ref_cache(d)
        got = run_decode(d, dev(cache, torch), torch)
        ref = decode_expanded(d["q"], d["kv_b"], cache, d["block_table"], d["seq_lens"], q_len)
        mx, rr = errors(got, ref)
        say(f"   max-abs {mx:.3e} rel-rms {rr:.3e}")
        assert mx <= MAX_ABS and rr <= REL_RMS


def test_decode_ignores_slots_beyond_length():
    """Slots at positions >= seq_len hold NaN sentinels (and random pages hold
    other sequences' data); rewriting them must not change the output."""
    torch = _torch()
    say("[decode] slots beyond length")
    d = wl.make_inputs(2, 1, 16, [70, 129], permute=True, seed=42, spare_blocks=1)
    cache = ref_cache(d)
    a = run_decode(d, dev(cache, torch), torch)
    c2 = cache.copy()
    for b, length in enumerate(d["seq_lens"]):
        for p in range(int(length), ((int(length) + 63) // 64) * 64):
            c2[d["block_table"][b, p // 64], p % 64] = np.uint16(0x7F80)  # +inf
    b2 = run_decode(d, dev(c2, torch), torch)
    assert np.array_equal(a, b2)


def test_decode_zero_batch_and_no_history():
    torch = _torch()
    import mla_latent_kv_07_amd as mla
    say("[decode] B=0 and seq_len == q_len")
    d = wl.make_inputs(2, 2, 16, [2, 2], permute=False, seed=43)
    cache = ref_cache(d)
    got = run_decode(d, dev(cache, torch), torch)
    ref = decode_expanded(d["q"], d["kv_b"], cache, d["block_table"], d["seq_lens"], 2)
    mx, rr = errors(got, ref)
    assert mx <= MAX_ABS and rr <= REL_RMS
    e = torch.empty((0, 1, 16, 192), dtype=torch.bfloat16, device="cuda")
    out = mla.decode(e, dev(d["kv_b"], torch), dev(cache, torch),
                     torch.zeros((0, 1), dtype=torch.int32, device="cuda"),
                     torch.zeros((0,), dtype=torch.int32, device="cuda"), 1)
    assert out.shape == (0, 1, 16, 128)


def test_error_status_on_gpu():
    torch = _torch()
    import mla_latent_kv_07_amd as mla
    d = wl.make_inputs(1, 1, 16, [10], permute=False, seed=44)
    with pytest.raises(mla.MLAError) as ei:
        mla.decode(dev(d["q"], torch), dev(d["kv_b"], torch), dev(d["cache"], torch),
                   dev(d["block_table"], torch), dev(d["seq_lens"], torch), 10,
                   workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    assert ei.value.status == 4


def test_decode_restart_on_score_jump():
    """One late position scaled 20x makes some heads' scores jump far above the
    first chunk's max; the kernel must restart those items (exact-max pass)
    and still match the oracle.  Outputs are large here, so the max error is
    taken relative to the largest output."""
    torch = _torch()
    say("[decode] large late score (restart path)")
    d = wl.make_inputs(2, 1, 128, [300, 200], permute=True, seed=45)
    cache = ref_cache(d)
    for b, p in ((0, 250), (1, 70)):
        row = cache[d["block_table"][b, p // 64], p % 64]
        from oracle import bf16_bits_to_f64, f64_to_bf16_bits
        row[:] = f64_to_bf16_bits(bf16_bits_to_f64(row) * 20.0)
    got = run_decode(d, dev(cache, torch), torch)
    ref = decode_expanded(d["q"], d["kv_b"], cache, d["block_table"], d["seq_lens"], 1)
    mx, rr = errors(got, ref)
    rel_max = mx / float(np.max(np.abs(ref)))
    say(f"   max-abs/max|ref| {rel_max:.3e} rel-rms {rr:.3e}")
    assert rel_max <= MAX_ABS and rr <= REL_RMS


def test_debug_checks_reject_bad_tables():
    """With the debug checks on, a block id outside [0, num_blocks) or a
    length above max_seq_len is reported as MLA_ERR_BOUNDS before anything
    is launched (the kernels never see the bad table); valid inputs give the
    same output as with the checks off."""
    torch = _torch()
    import mla_latent_kv_07_amd as mla
    say("[decode] debug checks")
    d = wl.make_inputs(2, 1, 128, [100, 150], permute=True, seed=46, spare_blocks=1)
    cache = ref_cache(d)
    prev = mla.debug_checks(1)
    try:
        good = run_decode(d, dev(cache, torch), torch)
        mla.debug_checks(0)
        assert np.array_equal(good, run_decode(d, dev(cache, torch), torch))
        mla.debug_checks(1)
        bad = d["block_table"].copy()
        bad[1, 2] = cache.shape[0]  # one past the last block
        with pytest.raises(mla.MLAError) as ei:
            mla.decode(dev(d["q"], torch), dev(d["kv_b"], torch), dev(cache, torch),
                       dev(bad, torch), dev(d["seq_lens"], torch), 150)
        assert ei.value.status == 6
        with pytest.raises(mla.MLAError) as ei:
            mla.decode(dev(d["q"], torch), dev(d["kv_b"], torch), dev(cache, torch),
                       dev(d["block_table"], torch), dev(d["seq_lens"], torch), 120)
        assert ei.value.status == 6
        with pytest.raises(mla.MLAError) as ei:
            mla.cache_insert(dev(d["kv_a"], torch), dev(d["rms_w"], torch), dev(bad, torch),
                             dev(d["seq_lens"], torch), dev(cache, torch), eps=EPS32, heads=128)
        assert ei.value.status == 6
    finally:
        mla.debug_checks(prev)
