"""The insert's integer double -> bf16 rounding (f64_bits_to_bf16 in
csrc/insert_dev.h, host and device code) against round-to-nearest-even done
exactly in rational arithmetic, on the CPU: the insert is bit-exact only if
this rounding is.  A host program built with hipcc from the header reads
double bit patterns and prints (covered, bf16 bits); cases: ties with an
even and an odd kept bit, mantissa carries into the exponent, the overflow
edge, both ends of the covered exponent ranges, signed zeros and random
doubles."""
import os
import random
import shutil
import struct
import subprocess
from fractions import Fraction

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include "insert_dev.h"
#include <cstdio>
int main() {
  unsigned long long u;
  while (std::scanf("%llx", &u) == 1) {
    bool covered = false;
    const unsigned b = mla::f64_bits_to_bf16(u, covered);
    std::printf("%d %04x\n", covered ? 1 : 0, b);
  }
  return 0;
}
"""


def exact_bf16(u: int) -> int:
    """bf16 bits of the double with bits u, rounded to nearest even (finite u)."""
    d = struct.unpack("<d", struct.pack("<Q", u))[0]
    sign = 0x8000 if u >> 63 else 0
    x = abs(Fraction(d))
    if x == 0:
        return sign
    e = x.numerator.bit_length() - x.denominator.bit_length()
    if Fraction(2) ** e > x:
        e -= 1
    quantum = Fraction(2) ** (max(e, -126) - 7)  # bf16 spacing (subnormal below 2^-126)
    n = x / quantum
    k = n.numerator // n.denominator
    rem = n - k
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and k % 2 == 1):
        k += 1
    v = k * quantum
    if v >= Fraction(2) ** 128:
        return sign | 0x7F80  # past the largest finite bf16: infinity
    if v < Fraction(2) ** -126:
        return sign | int(v / Fraction(2) ** -133)
    ev = v.numerator.bit_length() - v.denominator.bit_length()
    if Fraction(2) ** ev > v:
        ev -= 1
    m = (v / Fraction(2) ** ev - 1) * 128
    assert m.denominator == 1
    return sign | ((ev + 127) << 7) | int(m)


def cases() -> list:
    rng = random.Random(7)
    out = []
    mants = [0, 1, 2**44 - 1, 2**44, 2**44 + 1, 2**45 + 2**44, 3 * 2**44, 2**45 - 1,
             2**52 - 1, 2**52 - 2**44, 2**52 - 2**44 - 1, 2**51, 2**51 + 2**44]
    for be in list(range(0, 4)) + list(range(880, 905)) + list(range(1018, 1029)) + \
            list(range(1140, 1160)) + [2046]:
        for m in mants:
            for s in (0, 1):
                out.append((s << 63) | (be << 52) | m)
    for _ in range(4000):
        be = rng.choice([rng.randint(0, 888), rng.randint(897, 1150), rng.randint(889, 896),
                         rng.randint(1151, 2046)])
        out.append((rng.getrandbits(1) << 63) | (be << 52) | rng.getrandbits(52))
    out += [0x7FF0000000000000, 0xFFF0000000000000, 0x7FF8000000000000]  # inf, -inf, NaN
    return out


@pytest.fixture(scope="module")
def rounding_program(tmp_path_factory):
    from mla_latent_kv_07_amd import build as B
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    if not shutil.which(hipcc) and not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("rnd")
    src, exe = d / "rnd.hip", d / "rnd"
    src.write_text(PROGRAM)
    r = subprocess.run([hipcc, *B.common_flags(), str(src), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return str(exe)


def test_integer_rounding_is_exact_where_it_claims_to_be(rounding_program):
    us = cases()
    r = subprocess.run([rounding_program], input="\n".join(f"{u:x}" for u in us) + "\n",
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    lines = r.stdout.split("\n")
    bad = []
    n_covered = 0
    for u, line in zip(us, lines):
        cov, bits = line.split()
        be = (u >> 52) & 0x7FF
        want_cov = be <= 888 or 897 <= be <= 1150
        assert (cov == "1") == want_cov, (hex(u), cov)
        if want_cov:
            n_covered += 1
            if int(bits, 16) != exact_bf16(u):
                bad.append((hex(u), bits, hex(exact_bf16(u))))
    assert len(lines) >= len(us)
    assert n_covered > 2000
    assert not bad, bad[:10]


def test_exact_reference_on_printed_values():
    """The reference itself on values whose bf16 rounding is known: 1 + 2^-8
    (a tie, kept bit even) stays 1, 1 + 3 * 2^-8 (a tie, kept bit odd) goes
    up, the largest finite bf16 and the first value that rounds past it."""
    bits = lambda x: struct.unpack("<Q", struct.pack("<d", x))[0]
    assert exact_bf16(bits(1.0)) == 0x3F80
    assert exact_bf16(bits(1.0 + 2**-8)) == 0x3F80
    assert exact_bf16(bits(1.0 + 3 * 2**-8)) == 0x3F82
    assert exact_bf16(bits(-2.0)) == 0xC000
    assert exact_bf16(bits((2 - 2**-7) * 2.0**127)) == 0x7F7F
    assert exact_bf16(bits((2 - 2**-8) * 2.0**127)) == 0x7F80
    assert exact_bf16(bits(2.0**-133)) == 0x0001
    assert exact_bf16(bits(2.0**-134)) == 0x0000  # tie to even (zero)
