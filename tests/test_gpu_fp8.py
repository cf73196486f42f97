"""GPU parity of the FP8 latent cache: libmla's mla_cache_insert_fp8 and
mla_decode_fp8 against the float64 CPU oracle (oracle/fp8.py).

Insert: every byte of every row bit-exact (codes, rope, scale byte, padding),
and every byte outside the written rows unchanged.  Decode: the dequantised
values are exact in bf16, so the decode arithmetic is that of the bf16 path
and the same bound applies (max-abs 2e-2, relative RMS 5e-3) against the
float64 expanded-form oracle run on the same FP8 cache.
"""
import sys

import numpy as np
import pytest

import workloads as wl
from oracle import fp8 as ofp8

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


def garbage_cache(d, seed):
    """An FP8 cache of random bytes (the rows the insert must not touch)."""
    nb = d["cache"].shape[0]
    return np.random.default_rng(seed).integers(0, 256, (nb, 64, ofp8.FP8_ROW_BYTES),
                                                dtype=np.uint8)


def finite_bf16(c):
    """bf16 bits with every non-finite value (the NaN sentinels of slots the
    decode must not read) replaced by zero."""
    v = (np.asarray(c, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    return np.where(np.isfinite(v), c, np.uint16(0)).astype(np.uint16)


def finite_fp8_cache(d):
    """The workload's bf16 cache in FP8 form (sentinel slots as zeros)."""
    return ofp8.quantize_cache(finite_bf16(d["cache"]))


def sampled_fp8_cache(d, seed):
    """A full-size FP8 cache without quantising every row: codes drawn from
    the oracle's codes of a pool of N(0,1) values, scale 2^-6 per row (the
    scale the quantiser picks for such rows), rope from the bf16 cache."""
    rng = np.random.default_rng(seed)
    pool, _ = ofp8.quantize_latent(ofp8.f64_to_bf16_bits(rng.normal(size=(64, 512)) * 64.0))
    nb = d["cache"].shape[0]
    codes = rng.choice(pool.reshape(-1), size=(nb, 64, 512))
    scale = np.full((nb, 64), 127 - 6, dtype=np.uint8)
    return ofp8.pack_rows(codes, finite_bf16(d["cache"][..., 512:]), scale)


def run_insert(d, cache_u8, torch):
    import mla_latent_kv_07_amd as mla
    cache = dev(cache_u8, torch)
    mla.cache_insert(dev(d["kv_a"], torch), dev(d["rms_w"], torch), dev(d["block_table"], torch),
                     dev(d["seq_lens"], torch), cache, eps=EPS32, rope_base=wl.ROPE_BASE,
                     heads=d["heads"], fp8=True)
    torch.cuda.synchronize()
    return cache


def run_decode(d, cache_dev, torch, hint=0):
    import mla_latent_kv_07_amd as mla
    out = mla.decode(dev(d["q"], torch), dev(d["kv_b"], torch), cache_dev,
                     dev(d["block_table"], torch), dev(d["seq_lens"], torch),
                     int(d["seq_lens"].max()), num_splits_hint=hint, fp8=True)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def ref_insert(d, cache_u8):
    return ofp8.cache_insert_fp8(cache_u8, d["kv_a"], d["rms_w"], d["block_table"],
                                 d["seq_lens"], d["q_len"], EPS32, wl.ROPE_BASE)


# ------------------------------------------------------------------ insert --

INSERT_CASES = [
    ("small", lambda: wl.make_inputs(4, 1, 16, [1, 63, 64, 200], permute=True, seed=51,
                                     spare_blocks=2)),
    ("q_len 3, page edges", lambda: wl.make_inputs(5, 3, 16, [3, 63, 64, 65, 130], permute=True,
                                                   seed=52, spare_blocks=3)),
    ("v3_mtp_b128", lambda: wl.make_workload("v3_mtp_b128")),
]


@pytest.mark.parametrize("case", INSERT_CASES, ids=[c[0] for c in INSERT_CASES])
def test_insert_fp8_bit_exact(case):
    torch = _torch()
    name, make = case
    say(f"[insert fp8] {name}")
    d = make()
    c0 = garbage_cache(d, 7)
    got = run_insert(d, c0, torch).cpu().numpy()
    ref = ref_insert(d, c0)
    assert np.array_equal(got, ref), f"{np.sum(got != ref)} bytes differ"


# ------------------------------------------------------------------ decode --

SMALL = [
    (4, 1, 16, [1, 63, 64, 200], 61),
    (3, 2, 16, [2, 65, 330], 62),
    (3, 1, 128, [1, 129, 300], 63),
    (2, 2, 128, [2, 191], 64),
    (2, 1, 48, [77, 64], 65),
    (1, 8, 16, [70], 66),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"B{c[0]}q{c[1]}H{c[2]}" for c in SMALL])
def test_decode_fp8_parity_small(case):
    torch = _torch()
    bsz, q_len, heads, lens, seed = case
    say(f"[decode fp8 small] B={bsz} q_len={q_len} H={heads} lens={lens}")
    d = wl.make_inputs(bsz, q_len, heads, lens, permute=True, seed=seed, spare_blocks=2)
    c8 = ref_insert(d, finite_fp8_cache(d))
    got = run_decode(d, dev(c8, torch), torch)
    ref = ofp8.decode_expanded_fp8(d["q"], d["kv_b"], c8, d["block_table"], d["seq_lens"], q_len)
    mx, rr = errors(got, ref)
    say(f"   max-abs {mx:.3e} rel-rms {rr:.3e}")
    assert np.all(np.isfinite(got))
    assert mx <= MAX_ABS and rr <= REL_RMS


SAMPLES = {
    "v2lite_b32": ([0, 7, 31], [0, 5, 15]),
    "v3_b64_l8192": ([0, 33, 63], [0, 77, 127]),
    "v3_mtp_b128": ([0, 64, 127], [2, 50, 127]),
}


@pytest.mark.parametrize("name", list(SAMPLES))
def test_decode_fp8_workload_chained(name):
    """Full size: FP8 insert then FP8 decode on the GPU with the automatic
    split plan (the benchmark's launch configuration); sampled sequences and
    heads checked against the oracle on the same FP8 cache."""
    torch = _torch()
    say(f"[decode fp8 workload] {name}")
    d = wl.make_workload(name)
    c0 = sampled_fp8_cache(d, 70)
    cache_dev = run_insert(d, c0, torch)
    got = run_decode(d, cache_dev, torch)
    assert np.all(np.isfinite(got))
    c8 = cache_dev.cpu().numpy()
    bs, hs = SAMPLES[name]
    ref = ofp8.decode_expanded_fp8(d["q"], d["kv_b"], c8, d["block_table"], d["seq_lens"],
                                   d["q_len"], batches=bs, heads=hs)
    mx, rr = errors(got[bs][:, :, hs], ref)
    say(f"   max-abs {mx:.3e} rel-rms {rr:.3e}")
    assert mx <= MAX_ABS and rr <= REL_RMS


def test_decode_fp8_ignores_rows_beyond_length_and_split_count():
    torch = _torch()
    say("[decode fp8] rows beyond length, split counts")
    d = wl.make_inputs(3, 2, 128, [700, 1500, 65], permute=True, seed=67, spare_blocks=1)
    c8 = ref_insert(d, finite_fp8_cache(d))
    ref = ofp8.decode_expanded_fp8(d["q"], d["kv_b"], c8, d["block_table"], d["seq_lens"], 2)
    a = run_decode(d, dev(c8, torch), torch)
    c2 = c8.copy()
    rng = np.random.default_rng(68)
    for b, length in enumerate(d["seq_lens"]):
        for p in range(int(length), ((int(length) + 63) // 64) * 64):
            c2[d["block_table"][b, p // 64], p % 64] = rng.integers(0, 256, ofp8.FP8_ROW_BYTES)
    b2 = run_decode(d, dev(c2, torch), torch)
    assert np.array_equal(a, b2)
    for h in (0, 1, 5):
        o = run_decode(d, dev(c8, torch), torch, hint=h)
        mx, rr = errors(o, ref)
        say(f"   hint {h}: max-abs {mx:.3e} rel-rms {rr:.3e}")
        assert mx <= MAX_ABS and rr <= REL_RMS


# The FP8 format's cost against the bf16 cache, derived from E4M3's 3-bit
# mantissa (tests/test_fp8_oracle.py, FP8_OUT_BUDGET: 2^-4 sqrt(0.541 / 3)
# sqrt(1 + 2/3) = 0.0343 relative RMS at these workloads' score statistics),
# plus the bf16 pipeline error of the two GPU decodes (about 3.5e-3 each,
# measured against the oracle) in quadrature.
FP8_GPU_BUDGET = float(np.hypot(2.0 ** -4 * np.sqrt(0.541 / 3) * np.sqrt(5.0 / 3.0),
                                2 * 3.5e-3))


def test_fp8_cache_error_against_bf16_cache():
    """What the format costs (a property of the method, not a parity claim):
    the same tokens inserted into a bf16 and an FP8 cache, decoded on the
    GPU, within the budget derived from the format."""
    torch = _torch()
    import mla_latent_kv_07_amd as mla
    say("[decode fp8] quantisation error against the bf16 cache")
    d = wl.make_inputs(2, 1, 128, [2048, 777], permute=True, seed=69)
    cbf = dev(d["cache"], torch)
    mla.cache_insert(dev(d["kv_a"], torch), dev(d["rms_w"], torch), dev(d["block_table"], torch),
                     dev(d["seq_lens"], torch), cbf, eps=EPS32, rope_base=wl.ROPE_BASE,
                     heads=128)
    torch.cuda.synchronize()
    # the bf16 cache the GPU just wrote, and the same rows in FP8 form
    bf_host = finite_bf16(cbf.view(torch.int16).cpu().numpy().view(np.uint16))
    c8 = dev(ofp8.quantize_cache(bf_host), torch)
    a = run_decode(d, c8, torch)
    b = mla.decode(dev(d["q"], torch), dev(d["kv_b"], torch), dev(bf_host, torch),
                   dev(d["block_table"], torch), dev(d["seq_lens"], torch),
                   int(d["seq_lens"].max())).float().cpu().numpy().astype(np.float64)
    mx, rr = errors(a, b)
    say(f"   FP8 vs bf16 cache: max-abs {mx:.3e} rel-rms {rr:.3e} (budget {FP8_GPU_BUDGET:.3e})")
    assert rr <= FP8_GPU_BUDGET


def test_decode_fp8_restart_on_score_jump():
    """The FP8 cache's restart path: one late position of each sequence scaled
    20x (before quantisation; its scale byte absorbs it) makes some heads'
    scores jump far above the first chunk's max, so those items restart (an
    exact-max pass, then a pass with that reference, each chunk expanded
    again from its FP8 rows).  Outputs are large here, so the max error is
    taken relative to the largest output, as for the bf16 cache."""
    torch = _torch()
    from oracle import bf16_bits_to_f64, f64_to_bf16_bits
    say("[decode fp8] large late score (restart path)")
    d = wl.make_inputs(2, 1, 128, [300, 200], permute=True, seed=45)
    cbf = finite_bf16(ref_insert_bf16(d))
    for b, p in ((0, 250), (1, 70)):
        row = cbf[d["block_table"][b, p // 64], p % 64]
        row[:] = f64_to_bf16_bits(bf16_bits_to_f64(row) * 20.0)
    c8 = ofp8.quantize_cache(cbf)
    got = run_decode(d, dev(c8, torch), torch)
    ref = ofp8.decode_expanded_fp8(d["q"], d["kv_b"], c8, d["block_table"], d["seq_lens"], 1)
    mx, rr = errors(got, ref)
    rel_max = mx / float(np.max(np.abs(ref)))
    say(f"   max-abs/max|ref| {rel_max:.3e} rel-rms {rr:.3e}")
    assert np.all(np.isfinite(got))
    assert rel_max <= MAX_ABS and rr <= REL_RMS


def ref_insert_bf16(d):
    from oracle import cache_insert
    return cache_insert(d["cache"], d["kv_a"], d["rms_w"], d["block_table"], d["seq_lens"],
                        d["q_len"], EPS32, wl.ROPE_BASE, wl.LATENT)
