"""Pins for the query rotation of the fused step (oracle.rotate_q; no GPU).

"深度解读DeepSeek：源码解读 DeepSeek-V3", section MLA: the query branch of the
forward pass rotates q_pe with the same freqs_cis rows as k_pe, those of the
current positions, so new query i of a sequence of post-insert length L sits
at position L - q_len + i.  Checked against the closed form of one pair at
that position and against the property RoPE exists for: a query and a key
rotated at the same position keep their dot product.
"""
import math

import numpy as np

from oracle import bf16_bits_to_f64, f64_to_bf16_bits, rope_pairs_f64, rotate_q
import workloads as wl

NOPE = 128


def test_rotate_q_closed_form_at_the_query_position():
    d = wl.make_inputs(3, 2, 16, [70, 2, 130], permute=True, seed=21)
    q = d["q"].copy()
    q[..., NOPE:] = 0
    q[..., NOPE] = f64_to_bf16_bits(np.array([1.0]))[0]     # pair 0 = (1, 0)
    q[..., NOPE + 2] = f64_to_bf16_bits(np.array([1.0]))[0]  # pair 1 = (1, 0)
    r = rotate_q(q, d["seq_lens"], 2, wl.ROPE_BASE, NOPE)
    assert np.array_equal(r[..., :NOPE], q[..., :NOPE])     # the nope part is untouched
    for b, length in enumerate(d["seq_lens"]):
        for i in range(2):
            p = int(length) - 2 + i
            th1 = p * wl.ROPE_BASE ** (-2.0 / 64)
            want = f64_to_bf16_bits(np.array([math.cos(p), math.sin(p), math.cos(th1),
                                              math.sin(th1)]))
            for h in range(16):
                assert np.array_equal(r[b, i, h, NOPE:NOPE + 4], want)
                assert np.all(bf16_bits_to_f64(r[b, i, h, NOPE + 4:]) == 0)


def test_rotated_query_meets_its_own_key_unchanged():
    d = wl.make_inputs(4, 3, 16, [3, 64, 65, 500], permute=True, seed=22)
    rng = np.random.default_rng(23)
    r = rotate_q(d["q"], d["seq_lens"], 3, wl.ROPE_BASE, NOPE)
    worst, worst_shift = 0.0, np.inf
    for b, length in enumerate(d["seq_lens"]):
        for i in range(3):
            p = int(length) - 3 + i
            for h in range(16):
                qv = bf16_bits_to_f64(d["q"][b, i, h, NOPE:])
                k = rng.standard_normal(64)
                ref = qv @ k
                scale = np.linalg.norm(qv) * np.linalg.norm(k)
                got = bf16_bits_to_f64(r[b, i, h, NOPE:]) @ rope_pairs_f64(k, np.array(float(p)),
                                                                           wl.ROPE_BASE)
                worst = max(worst, abs(got - ref) / scale)
                # the key one position away: the product moves far beyond rounding
                off = bf16_bits_to_f64(r[b, i, h, NOPE:]) @ rope_pairs_f64(
                    k, np.array(float(p + 1)), wl.ROPE_BASE)
                worst_shift = min(worst_shift, abs(off - ref) / scale)
    assert worst <= 2.0 ** -8          # one bf16 rounding of the rotated query
    assert worst_shift > 0 and worst_shift < np.inf
