"""Pins for the FP8 latent-cache oracle (no GPU).

The element format is checked against torch's own float8_e4m3fn conversion
(an independent implementation) over every bf16 input and every code, and
against values derived by hand from the format's fields; the scale rule, the
error bound, the row layout and the insert/decode wrappers are checked against
properties the format fixes and against the bf16 oracle.  Sources: "DeepSeek-
V3.2-Exp unboxing", 初步研读 (FP8 KV cache, per-token key scales); the vLLM
DeepSeek-V4 notes, section 一 (KV quant in the insert, UE8M0 scales);
"DeepSeek-V2-Lite 模型结构详解" §五 (latent then rope).
"""
import numpy as np
import pytest
import torch

from oracle import cache_insert, decode_expanded, f64_to_bf16_bits, bf16_bits_to_f64
from oracle import fp8
import workloads as wl


def all_bf16_values():
    with np.errstate(invalid="ignore"):
        return (np.arange(65536, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


# ------------------------------------------------------------ element format

def test_e4m3_encode_matches_torch_on_every_bf16_input():
    x = all_bf16_values()
    fin = np.isfinite(x) & (np.abs(x) <= 464.0)
    ref = torch.tensor(x[fin].astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.e4m3_encode(x[fin]), ref)
    beyond = np.isfinite(x) & (np.abs(x) > 464.0)
    codes = fp8.e4m3_encode(x[beyond])
    assert set((codes & 0x7F).tolist()) == {0x7F}          # NaN


def test_e4m3_decode_matches_torch_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.tensor(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = fp8.e4m3_decode(codes)
    assert np.all((got == ref) | (np.isnan(got) & np.isnan(ref)))


def test_e4m3_hand_values_from_the_format_fields():
    enc = lambda v: int(fp8.e4m3_encode(np.array([v]))[0])
    assert enc(448.0) == 0x7E            # S.1111.110: (1 + 6/8) * 2**8
    assert enc(1.0) == 0x38              # E = 7
    assert enc(2.0 ** -6) == 0x08        # smallest normal
    assert enc(2.0 ** -9) == 0x01        # smallest subnormal
    assert enc(-0.0) == 0x80
    assert enc(1.0 + 1 / 16) == 0x38     # tie -> even mantissa (down)
    assert enc(1.0 + 3 / 16) == 0x3A     # tie -> even mantissa (up)
    assert enc(2.0 ** -10) == 0x00       # tie between 0 and 2**-9 -> 0
    assert enc(3 * 2.0 ** -10) == 0x02   # tie between 2**-9 and 2**-8 -> even
    assert enc(464.0) == 0x7E            # tie between 448 and (NaN) 480 -> 448
    assert np.isnan(fp8.e4m3_decode(np.array([0x7F], dtype=np.uint8))[0])
    assert fp8.e4m3_decode(np.array([0x7E], dtype=np.uint8))[0] == 448.0


def test_e4m3_round_trip_and_order_of_finite_codes():
    pos = np.arange(0x7F, dtype=np.uint8)                     # 0x00 .. 0x7E
    vals = fp8.e4m3_decode(pos)
    assert np.all(np.diff(vals) > 0)                          # strictly increasing
    codes = np.concatenate([pos, pos | 0x80])
    assert np.array_equal(fp8.e4m3_encode(fp8.e4m3_decode(codes)), codes)


# --------------------------------------------------------- scale and quantise

def test_scale_exponent_is_the_smallest_valid_power_of_two():
    rng = np.random.default_rng(3)
    amax = np.exp2(rng.uniform(-60, 60, 4000))
    e = fp8.scale_exponent(amax).astype(np.float64)
    assert np.all(amax * np.exp2(-e) <= 448.0)
    assert np.all(amax * np.exp2(-(e - 1)) > 448.0)
    exact = 448.0 * np.exp2(np.arange(-20, 21))
    assert np.array_equal(fp8.scale_exponent(exact), np.arange(-20, 21))
    assert fp8.scale_exponent(np.array([0.0]))[0] == 0
    assert fp8.scale_exponent(np.array([1e300]))[0] == 127     # clamped


def test_quantisation_error_bound_on_random_rows():
    rng = np.random.default_rng(4)
    rows = f64_to_bf16_bits(rng.normal(size=(64, 512)) * np.exp2(rng.integers(-8, 8, (64, 1))))
    codes, scale = fp8.quantize_latent(rows)
    x = bf16_bits_to_f64(rows)
    y = fp8.dequantize_latent(codes, scale)
    e = scale.astype(np.float64) - 127
    u = np.abs(x) * np.exp2(-e)[:, None]                      # scaled magnitudes, <= 448
    assert np.all(u <= 448.0)
    # half a quantum of the scaled value's binade, in original units
    _, ex = np.frexp(np.where(u > 0, u, 1.0))
    half_q = np.where(u >= 2.0 ** -6, np.exp2(ex - 5.0), 2.0 ** -10) * np.exp2(e)[:, None]
    assert np.all(np.abs(x - y) <= half_q)
    assert np.max(np.abs(x) * np.exp2(-e)[:, None], axis=1).min() > 224.0  # range is used


def test_row_layout_round_trip():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 256, (3, 7, 512)).astype(np.uint8)
    rope = rng.integers(0, 65536, (3, 7, 64)).astype(np.uint16)
    scale = rng.integers(1, 255, (3, 7)).astype(np.uint8)
    rows = fp8.pack_rows(codes, rope, scale)
    assert rows.shape == (3, 7, 656)
    assert np.all(rows[..., 641:] == 0)
    assert np.array_equal(rows[..., 640], scale)
    assert np.array_equal(rows[..., 512:514].view("<u2")[..., 0], rope[..., 0])
    c2, r2, s2 = fp8.unpack_rows(rows)
    assert np.array_equal(c2, codes) and np.array_equal(r2, rope) and np.array_equal(s2, scale)


# ------------------------------------------------------------ insert / decode

def test_insert_fp8_is_the_bf16_insert_quantised():
    d = wl.make_inputs(3, 2, 16, [70, 2, 130], permute=True, seed=11)
    eps = float(np.float32(wl.EPS))
    bf = cache_insert(d["cache"], d["kv_a"], d["rms_w"], d["block_table"], d["seq_lens"], 2,
                      eps, wl.ROPE_BASE, wl.LATENT)
    c8 = fp8.quantize_cache(d["cache"])
    got = fp8.cache_insert_fp8(c8, d["kv_a"], d["rms_w"], d["block_table"], d["seq_lens"], 2,
                               eps, wl.ROPE_BASE)
    page = bf.shape[1]
    touched = np.zeros(bf.shape[:2], dtype=bool)
    for b in range(3):
        for p in range(int(d["seq_lens"][b]) - 2, int(d["seq_lens"][b])):
            touched[int(d["block_table"][b, p // page]), p % page] = True
    assert np.array_equal(got[~touched], c8[~touched])          # nothing else written
    codes, scale = fp8.quantize_latent(bf[touched][:, :512])
    assert np.array_equal(got[touched], fp8.pack_rows(codes, bf[touched][:, 512:], scale))


def test_decode_fp8_equals_bf16_decode_on_exactly_representable_cache():
    # codes and scales drawn directly; their values are exact in bf16, so a
    # bf16 cache holding them must give the same decode as the FP8 cache
    rng = np.random.default_rng(6)
    d = wl.make_inputs(2, 2, 16, [100, 64], permute=True, seed=7)
    nb, page = d["cache"].shape[:2]
    codes = rng.integers(0, 0x7F, (nb, page, 512)).astype(np.uint8)
    codes |= (rng.integers(0, 2, codes.shape) << 7).astype(np.uint8)
    codes[codes == 0x7F] = 0x7E
    codes[codes == 0xFF] = 0xFE
    scale = rng.integers(127 - 10, 127 - 6, (nb, page)).astype(np.uint8)
    rope = f64_to_bf16_bits(rng.normal(size=(nb, page, 64)))   # finite everywhere
    c8 = fp8.pack_rows(codes, rope, scale)
    lat = fp8.dequantize_latent(codes, scale)
    lat_bits = f64_to_bf16_bits(lat)
    assert np.array_equal(bf16_bits_to_f64(lat_bits), lat)      # exact in bf16
    cbf = np.concatenate([lat_bits, rope], axis=-1)
    a = fp8.decode_expanded_fp8(d["q"], d["kv_b"], c8, d["block_table"], d["seq_lens"], 2)
    b = decode_expanded(d["q"], d["kv_b"], cbf, d["block_table"], d["seq_lens"], 2)
    assert np.array_equal(a, b)


# ---- what the FP8 format costs against the bf16 cache (error budget) --------
#
# Derivation.  An E4M3 value with mantissa m in [1, 2) and exponent k sits in a
# binade whose quantum is 2^(k-3); round to nearest even leaves an error
# uniform in half a quantum, so the relative error of x = m 2^k is uniform in
# +-2^-4 / m and its mean square is (2^-4)^2 E[m^-2] / 3.  E[m^-2] is 1/2 for
# mantissas uniform in [1, 2) and 0.541 for log-uniform ones (N(0, 1) draws lie
# between), so the per-element relative RMS error is
#     eps = 2^-4 sqrt(E[m^-2] / 3)  in [0.0255, 0.0266].
# (The per-token power-of-two scale only moves exponents, it never rounds.)
# In the decode, the latent error enters the values directly (relative eps)
# and the scores through q_lat . dc (a fraction f of the score variance comes
# from the latent, the rope part stays bf16); a score error ds moves each
# weight by p ds, so for independent value rows the output's relative RMS
# error is about
#     eps sqrt(1 + f sigma_s^2)
# with sigma_s the score spread in natural-log units.  The workloads draw
# q, c ~ N(0, 1) and kv_b with variance 1/512: q_lat . c has variance 128 and
# q_pe . k_pe 64, so f = 2/3 and sigma_s = 1 after the 1/sqrt(192) scale,
# giving a budget of 0.0266 sqrt(5/3) = 0.0343 (plus the bf16 pipeline's own
# ~3e-3 when both sides run on the GPU, added in quadrature).
FP8_EPS_LO, FP8_EPS_HI = 2.0 ** -4 * np.sqrt(0.5 / 3), 2.0 ** -4 * np.sqrt(0.541 / 3)
FP8_OUT_BUDGET = FP8_EPS_HI * np.sqrt(1.0 + 2.0 / 3.0)


def _finite_bf16(c):
    v = (np.asarray(c, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    return np.where(np.isfinite(v), c, np.uint16(0)).astype(np.uint16)


@pytest.mark.parametrize("case", [(2, 128, [2048, 777], 69), (2, 16, [3000, 1500], 70),
                                  (1, 128, [300], 71)])
def test_fp8_error_budget_matches_derivation(case):
    """The oracle's FP8 decode against its bf16 decode of the same rows: the
    per-element latent error matches eps (within 5 % of the derived band) and
    the output's relative RMS error stays within the derived budget."""
    bsz, heads, lens, seed = case
    d = wl.make_inputs(bsz, 1, heads, lens, permute=True, seed=seed)
    c = _finite_bf16(cache_insert(d["cache"], d["kv_a"], d["rms_w"], d["block_table"],
                                  d["seq_lens"], 1, float(np.float32(wl.EPS)), wl.ROPE_BASE,
                                  wl.LATENT))
    deq = fp8.dequantize_cache(fp8.quantize_cache(c))
    lat = bf16_bits_to_f64(c[..., :512])
    nz = lat != 0
    eps = np.sqrt(np.mean(((deq[..., :512][nz] - lat[nz]) / lat[nz]) ** 2))
    assert 0.95 * FP8_EPS_LO <= eps <= 1.05 * FP8_EPS_HI, eps
    # the rope part is copied exactly
    assert np.array_equal(deq[..., 512:], bf16_bits_to_f64(c[..., 512:]))
    ref = decode_expanded(d["q"], d["kv_b"], c, d["block_table"], d["seq_lens"], 1)
    out = decode_expanded(d["q"], d["kv_b"], deq, d["block_table"], d["seq_lens"], 1)
    err = out - ref
    rr = np.sqrt(np.mean(err ** 2) / np.mean(ref ** 2))
    assert 0.5 * FP8_EPS_LO <= rr <= FP8_OUT_BUDGET, (rr, FP8_OUT_BUDGET)
