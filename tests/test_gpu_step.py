"""GPU parity of the fused decoding step (mla_decode_step / _fp8: cache
insert, RoPE on q_pe and the query absorption in one launch, then decode).

Three checks per case, on the same seeded inputs:
* the cache the step leaves is bit-identical to the oracle's insert (bf16 or
  FP8 rows; every byte, written or not);
* the step's output and cache are bit-identical to the separate calls
  (mla_cache_insert then mla_decode on q with q_pe rotated by the oracle):
  the fused rotation rounds exactly as the oracle's;
* the output is within the decode bound (max-abs 2e-2, relative RMS 5e-3) of
  the float64 expanded-form oracle run on the oracle-rotated query.
"""
import sys

import numpy as np
import pytest

import workloads as wl
from oracle import cache_insert as oracle_insert
from oracle import decode_expanded, rotate_q
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


def host(t, fp8):
    import torch
    return t.cpu().numpy() if fp8 else t.view(torch.int16).cpu().numpy().view(np.uint16)


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def errors(got, ref):
    d = got - ref
    return float(np.max(np.abs(d))), float(np.sqrt(np.mean(d * d)) / np.sqrt(np.mean(ref * ref)))


def finite_bf16(c):
    v = (np.asarray(c, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    return np.where(np.isfinite(v), c, np.uint16(0)).astype(np.uint16)


def initial_cache(d, fp8, seed):
    """bf16: the workload's cache (NaN sentinels in unused slots).  FP8: rows
    quantised from it (small cases) or sampled codes (full size)."""
    if not fp8:
        return d["cache"]
    if d["cache"].shape[0] * 64 <= 64 * 4096:
        return ofp8.quantize_cache(finite_bf16(d["cache"]))
    rng = np.random.default_rng(seed)
    pool, _ = ofp8.quantize_latent(ofp8.f64_to_bf16_bits(rng.normal(size=(64, 512)) * 64.0))
    nb = d["cache"].shape[0]
    codes = rng.choice(pool.reshape(-1), size=(nb, 64, 512))
    return ofp8.pack_rows(codes, finite_bf16(d["cache"][..., 512:]),
                          np.full((nb, 64), 127 - 6, dtype=np.uint8))


def oracle_cache(d, c0, fp8):
    if fp8:
        return ofp8.cache_insert_fp8(c0, d["kv_a"], d["rms_w"], d["block_table"], d["seq_lens"],
                                     d["q_len"], EPS32, wl.ROPE_BASE)
    return oracle_insert(c0, d["kv_a"], d["rms_w"], d["block_table"], d["seq_lens"], d["q_len"],
                         EPS32, wl.ROPE_BASE, wl.LATENT)


def run_step(d, c0, fp8, torch):
    import mla_latent_kv_07_amd as mla
    cache = dev(c0, torch)
    out = mla.decode_step(dev(d["q"], torch), dev(d["kv_a"], torch), dev(d["rms_w"], torch),
                          dev(d["kv_b"], torch), cache, dev(d["block_table"], torch),
                          dev(d["seq_lens"], torch), int(d["seq_lens"].max()), eps=EPS32,
                          rope_base=wl.ROPE_BASE, fp8=fp8)
    torch.cuda.synchronize()
    return out, cache


def run_separate(d, c0, q_rot, fp8, torch):
    import mla_latent_kv_07_amd as mla
    cache = dev(c0, torch)
    mla.cache_insert(dev(d["kv_a"], torch), dev(d["rms_w"], torch), dev(d["block_table"], torch),
                     dev(d["seq_lens"], torch), cache, eps=EPS32, rope_base=wl.ROPE_BASE,
                     heads=d["heads"], fp8=fp8)
    out = mla.decode(dev(q_rot, torch), dev(d["kv_b"], torch), cache,
                     dev(d["block_table"], torch), dev(d["seq_lens"], torch),
                     int(d["seq_lens"].max()), fp8=fp8)
    torch.cuda.synchronize()
    return out, cache


def decode_ref(d, q_rot, cache_ref, fp8, **kw):
    if fp8:
        return ofp8.decode_expanded_fp8(q_rot, d["kv_b"], cache_ref, d["block_table"],
                                        d["seq_lens"], d["q_len"], **kw)
    return decode_expanded(q_rot, d["kv_b"], cache_ref, d["block_table"], d["seq_lens"],
                           d["q_len"], **kw)


SMALL = [
    ("B4q1H16", lambda: wl.make_inputs(4, 1, 16, [1, 63, 64, 200], permute=True, seed=81,
                                       spare_blocks=2)),
    ("B5q3H16", lambda: wl.make_inputs(5, 3, 16, [3, 63, 64, 65, 130], permute=True, seed=82,
                                       spare_blocks=3)),
    ("B3q2H128", lambda: wl.make_inputs(3, 2, 128, [2, 700, 1500], permute=True, seed=83,
                                        spare_blocks=1)),
]


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_step_small(case, fp8):
    torch = _torch()
    name, make = case
    say(f"[step small] {name} fp8={fp8}")
    d = make()
    c0 = initial_cache(d, fp8, 84)
    q_rot = rotate_q(d["q"], d["seq_lens"], d["q_len"], wl.ROPE_BASE, wl.NOPE)
    out_f, cache_f = run_step(d, c0, fp8, torch)
    out_s, cache_s = run_separate(d, c0, q_rot, fp8, torch)
    cf = host(cache_f, fp8)
    ref_c = oracle_cache(d, c0, fp8)
    assert np.array_equal(cf, ref_c), "cache differs from the oracle's insert"
    assert np.array_equal(cf, host(cache_s, fp8))
    assert np.array_equal(host(out_f, False), host(out_s, False)), "fused != separate calls"
    got = out_f.float().cpu().numpy().astype(np.float64)
    ref = decode_ref(d, q_rot, ref_c, fp8)
    mx, rr = errors(got, ref)
    say(f"   max-abs {mx:.3e} rel-rms {rr:.3e}")
    assert np.all(np.isfinite(got)) and mx <= MAX_ABS and rr <= REL_RMS


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_step_v3_mtp_b128(fp8):
    """The multi-token workload (B=128, q_len 2, H=128, contexts 1024..16384)
    in the benchmark's launch configuration: fused == separate bit for bit,
    the written rows equal the oracle's, sampled outputs within the bound."""
    torch = _torch()
    say(f"[step workload] v3_mtp_b128 fp8={fp8}")
    d = wl.make_workload("v3_mtp_b128")
    c0 = initial_cache(d, fp8, 85)
    q_rot = rotate_q(d["q"], d["seq_lens"], d["q_len"], wl.ROPE_BASE, wl.NOPE)
    out_f, cache_f = run_step(d, c0, fp8, torch)
    out_s, cache_s = run_separate(d, c0, q_rot, fp8, torch)
    bits = (lambda t: t) if fp8 else (lambda t: t.view(torch.int16))  # NaN sentinels
    assert torch.equal(bits(cache_f), bits(cache_s))
    assert torch.equal(out_f.view(torch.int16), out_s.view(torch.int16))
    cf = host(cache_f, fp8)
    bs, hs = [0, 64, 127], [2, 50, 127]
    # written rows against the oracle's insert (every new token)
    ref_c = oracle_cache(d, c0, fp8)
    for b, length in enumerate(d["seq_lens"]):
        for i in range(d["q_len"]):
            p = int(length) - d["q_len"] + i
            blk, slot = int(d["block_table"][b, p // 64]), p % 64
            assert np.array_equal(cf[blk, slot], ref_c[blk, slot])
    got = out_f.float().cpu().numpy().astype(np.float64)
    ref = decode_ref(d, q_rot, cf, fp8, batches=bs, heads=hs)
    mx, rr = errors(got[bs][:, :, hs], ref)
    say(f"   max-abs {mx:.3e} rel-rms {rr:.3e}")
    assert mx <= MAX_ABS and rr <= REL_RMS
