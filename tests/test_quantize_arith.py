"""Exactness of the quantize kernel's division-free arithmetic, checked over every fp16 input.

The activation quantize (quantization record of "Atom: Low-bit Quantization for Efficient and
Accurate LLM Serving", Fields "Bits" and "Weight group size": per-group scale
s = fp16(a / qmax) and codes rint(x / s)) avoids IEEE divides on the GPU:

- the scale: q0 = fl(a * fl(1/qmax)), q1 = fma(fma(-q0, qmax, a), fl(1/qmax), q0); the kernel
  stores fp16(q1), which must equal fp16(fl32(a / qmax));
- the reciprocal: from any r0 within one ulp of 1/s (the hardware reciprocal's accuracy),
  fma(fma(-s, r0, 1), r0, r0) must be the correctly rounded fl32(1 / s);
- the INT4 code: fp16(u + 1536), rounded once from the exact sum, minus 1536, must be the
  integer nearest u with ties to even.

Every claim is checked with exact rational arithmetic: fp32 and fp16 rounding are written out
here (round to nearest, ties to even), the fused operations round once.
"""
from fractions import Fraction as F
import os
import struct

import numpy as np
import pytest


def _round(q, mant_bits):
    """q rounded to a binary float with mant_bits fraction bits, nearest, ties to even
    (normal range only; every value below stays in it)."""
    if q == 0:
        return F(0)
    sign = -1 if q < 0 else 1
    q = abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if F(2) ** e > q:
        e -= 1
    m = q * F(2) ** (mant_bits - e)
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > F(1, 2) or (rem == F(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * F(fl) * F(2) ** (e - mant_bits)


def rn32(q):
    return _round(q, 23)


def fp16_bits(q):
    """fp16 bits of a value that is already an fp32 value (numpy rounds to nearest even)."""
    return int(np.float16(np.float32(float(q))).view(np.uint16))


def f32_step(q, d):
    b = struct.unpack("<I", struct.pack("<f", float(q)))[0] + d
    return F(struct.unpack("<f", struct.pack("<I", b))[0])


POSITIVE_FP16 = [F(float(h)) for h in np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16)]


@pytest.mark.parametrize("qmax", [7, 127])
def test_scale_without_divide_matches_fp16_of_fp32_quotient(qmax):
    c = rn32(F(1, qmax))
    bad = []
    for a in POSITIVE_FP16:
        q0 = rn32(a * c)
        q1 = rn32(rn32(a - q0 * qmax) * c + q0)
        if fp16_bits(q1) != fp16_bits(rn32(a / qmax)):
            bad.append(float(a))
    assert not bad, bad[:10]


def test_refined_reciprocal_is_correctly_rounded():
    bad = []
    for s in POSITIVE_FP16:
        exact = rn32(1 / s)
        for r0 in (f32_step(exact, -1), exact, f32_step(exact, 1)):
            r1 = rn32(rn32(1 - s * r0) * r0 + r0)
            if r1 != exact:
                bad.append((float(s), float(r0)))
    assert not bad, bad[:10]


def test_biased_fp16_rounding_gives_integer_code_ties_to_even():
    # every half-integer in [-7.5, 7.5], its fp32 neighbours, and a spread of other values
    vals = []
    for k in range(-15, 16):
        h = F(k, 2)
        vals.append(h)
        vals.append(f32_step(h, 1) if h > 0 else f32_step(h, -1) if h < 0 else F(2) ** -149)
        if h != 0:
            vals.append(f32_step(h, -1) if h > 0 else f32_step(h, 1))
    vals += [F(i, 64) for i in range(-7 * 64, 7 * 64 + 1)]
    for u in vals:
        n = _round(u + 1536, 10) - 1536        # fp16 has 10 fraction bits; spacing 1 on [1024, 2048)
        fl = u.numerator // u.denominator
        rem = u - fl
        want = fl + 1 if rem > F(1, 2) or (rem == F(1, 2) and fl % 2 == 1) else fl
        assert n == want, (float(u), n, want)


# --------------------------------------------------------------------------- the code quotient, exhaustively
def _reachable_scales(qmax):
    """(scale, largest absmax with that scale) for every fp16 absmax a >= 0, as fp16 bit
    patterns: s = fp16_rne(fl32(a / qmax)) (numpy's fp32 division and fp32 -> fp16 conversion
    are IEEE round to nearest even)."""
    a = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16)            # 0 and every positive finite fp16
    s = (a.astype(np.float32) / np.float32(qmax)).astype(np.float16).view(np.uint16)
    # s is non-decreasing in a, so the last a of each run of equal s is that scale's largest absmax
    last = np.nonzero(np.append(s[1:] != s[:-1], True))[0]
    return np.stack([s[last], a.view(np.uint16)[last]], axis=1).astype(np.uint16)


@pytest.mark.parametrize("qmax", [7, 127])
def test_code_quotient_exhaustive(qmax, tmp_path):
    """rint(clamp(u)) with u = fma(fma(-t, s, x), r, t), t = fl32(x * r), r = fl32(1/s), equals
    clamp(rint(fl32(x / s))) for every reachable fp16 scale s and every fp16 x with |x| at most
    the largest absmax that produces s: about 0.9 * 10^9 pairs per qmax, checked by a C program with
    IEEE binary32 fused multiply-adds (tests/quotient_exhaustive.c).  For every normal scale the
    same walk checks that rint(u) needs no clamp (the kernel clamps only for subnormal scales)."""
    import shutil
    import subprocess

    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "quotient_exhaustive.c")
    exe = str(tmp_path / "quotient_exhaustive")
    subprocess.run([gcc, "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", src, "-o", exe, "-lm"],
                   check=True)
    pairs = _reachable_scales(qmax)
    assert pairs[0, 0] == 0 and pairs[-1, 1] == 0x7BFF        # zero scale first, fp16 max last
    payload = struct.pack("<ii", qmax, len(pairs)) + pairs.tobytes()
    env = dict(os.environ, OMP_NUM_THREADS=str(min(8, os.cpu_count() or 1)))
    r = subprocess.run([exe], input=payload, capture_output=True, env=env, timeout=600)
    out = r.stdout.decode()
    assert r.returncode == 0, out + r.stderr.decode()
    n = int(out.split()[1])
    # the whole domain was walked: x = +-0 .. +-absmax for every scale (positive fp16 bit
    # patterns are ordered like their values)
    assert n == 2 * int((pairs[:, 1].astype(np.int64) + 1).sum()), out
    assert " mismatches 0 " in out and "unclamped_mismatches 0" in out, out
