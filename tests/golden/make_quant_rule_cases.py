"""Writes quant_rule_cases.json: int8 block-32 quantization cases that tell the stated
rounding rule apart from rules a plausible mistake would use.

Rule (workload definition: symmetric int8 block-32 activation quantization, halves to
even; reading taken: the code is the rounded product of x with the correctly rounded
binary32 reciprocal scale 127/amax):

    amax  = max |x| over the block            (binary32)
    scale = fl32(amax / 127)
    inv   = fl32(127 / amax)
    code  = round_half_even(fl32(x * inv)), clamped to [-127, 127]

Every value here is computed with exact rational arithmetic (fractions.Fraction) and an
explicit round-to-nearest-even onto binary32; nothing calls the oracle, numpy's float
arithmetic or the GPU library. For each case the file also records the codes of three
alternative rules, so a reader can see that each block separates them:

    div    round_half_even(fl32(x / scale))
    exact  round_half_even(x * 127 / amax)          (no intermediate rounding)
    mul127 round_half_even(fl32(fl32(x * 127) / amax))

Blocks named h64_* hold only values 64*u with u a binary16 number, so that a decode layer
whose gate rows evaluate to 64 and whose up rows evaluate to u (see the GPU test) produces
exactly these values as its SwiGLU output h = silu(64) * u.

Run:  python tests/golden/make_quant_rule_cases.py
"""
from __future__ import annotations

import json
import os
import struct
from fractions import Fraction

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "quant_rule_cases.json")


def f32_bits(v: float) -> int:
    return struct.unpack("<I", struct.pack("<f", v))[0]


def from_f32_bits(b: int) -> float:
    return struct.unpack("<f", struct.pack("<I", b))[0]


def half_values():
    """All finite positive normal binary16 values, as exact Fractions."""
    out = []
    for e in range(1, 31):
        for m in range(1024):
            out.append(Fraction(1024 + m, 1024) * Fraction(2) ** (e - 15))
    return out


def rne_int(v: Fraction) -> int:
    fl = v.numerator // v.denominator
    rem = v - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def fl32(v: Fraction) -> Fraction:
    """Round a rational to the nearest binary32 value (ties to even); normal range only."""
    if v == 0:
        return Fraction(0)
    s = -1 if v < 0 else 1
    a = -v if v < 0 else v
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    assert -126 <= e <= 127, "outside the normal binary32 range"
    ulp = Fraction(2) ** (e - 23)
    return s * rne_int(a / ulp) * ulp


def clamp(c: int) -> int:
    return max(-127, min(127, c))


def codes_all_rules(amax: Fraction, x: Fraction) -> dict:
    inv = fl32(Fraction(127) / amax)
    scale = fl32(amax / 127)
    rule = clamp(rne_int(fl32(x * inv)))
    div = clamp(rne_int(fl32(x / scale)))
    exact = clamp(rne_int(x * 127 / amax))
    mul127 = clamp(rne_int(fl32(fl32(x * 127) / amax)))
    return dict(rule=rule, div=div, exact=exact, mul127=mul127)


def as_float(v: Fraction) -> float:
    f = float(v)
    assert Fraction(f) == v and Fraction(from_f32_bits(f32_bits(f))) == v, "not a binary32 value"
    return f


def make_block(name: str, amax: Fraction, xs: list, derivation: str) -> dict:
    vals = [amax] + xs
    vals += [Fraction(0)] * (32 - len(vals))
    assert len(vals) == 32
    assert max(abs(v) for v in vals) == amax
    per = [codes_all_rules(amax, v) for v in vals]
    return {
        "name": name,
        "x": [as_float(v) for v in vals],
        "q": [c["rule"] for c in per],
        "scale": as_float(fl32(amax / 127)),
        "inv_f32": as_float(fl32(Fraction(127) / amax)),
        "q_div": [c["div"] for c in per],
        "q_exact": [c["exact"] for c in per],
        "q_mul127": [c["mul127"] for c in per],
        "derivation": derivation,
    }


def separating(amax: Fraction, candidates, limit: int) -> list:
    """Candidates (|x| < amax) whose rule code differs from at least one alternative,
    preferring those that differ from all three."""
    strong, weak = [], []
    for x in candidates:
        if abs(x) >= amax:
            continue
        c = codes_all_rules(amax, x)
        diffs = sum(c[k] != c["rule"] for k in ("div", "exact", "mul127"))
        if diffs == 3:
            strong.append(x)
        elif diffs:
            weak.append(x)
    picked = strong[:limit]
    picked += weak[: limit - len(picked)]
    return picked


def near_boundaries(amax: Fraction, ulps: int = 3) -> list:
    """binary32 values within a few ulps of (m + 1/2) * amax / 127, m = 0..126, both signs."""
    out = []
    for m in range(127):
        centre = fl32((m + Fraction(1, 2)) * amax / 127)
        if centre == 0:
            continue
        b = f32_bits(float(centre))
        for o in range(-ulps, ulps + 1):
            v = Fraction(from_f32_bits(b + o))
            out += [v, -v]
    return out


def main() -> None:
    cases = []
    # a binary32 block maximum with binary32 values near the rounding boundaries
    amax = Fraction(from_f32_bits(f32_bits(1.1137987375)))
    x0 = Fraction(from_f32_bits(f32_bits(0.0131551027)))
    xs = [x0] + separating(amax, near_boundaries(amax), 30)
    cases.append(make_block(
        "f32_boundaries_amax_1.1137987375", amax, xs,
        "binary32 values within 3 ulps of the code boundaries (m + 1/2) * amax / 127 whose "
        "code under the rule differs from at least one of x/scale, exact rounding and "
        "(x*127)/amax; the first listed x (0.0131551027) gets code 2 from the rule and 1 "
        "from x/scale"))
    # blocks of values 64*u, u binary16, for the GPU's h quantizers
    halves = half_values()
    for ua_bits in (0x2771, 0x298E, 0x2908):
        ua = half_from_bits(ua_bits)
        amax = 64 * ua
        cands = []
        for u in halves:
            if u < ua:
                cands += [64 * u, -64 * u]
        xs = separating(amax, cands, 31)
        cases.append(make_block(
            f"h64_amax_{float(amax)!r}", amax, xs,
            "values 64*u with u binary16 (a SwiGLU output silu(64)*u is exact in binary32): "
            "every nonzero x after the maximum gets a rule code different from at least "
            "one alternative rule"))
    with open(OUT, "w") as fh:
        json.dump({"source": __doc__.strip().splitlines()[0], "rule":
                   "code = round_half_even(fl32(x * fl32(127/amax))), clamp +-127",
                   "cases": cases}, fh, indent=1)
    print(f"wrote {len(cases)} cases to {OUT}")


def half_from_bits(b: int) -> Fraction:
    e, m = (b >> 10) & 31, b & 1023
    assert 0 < e < 31 and not (b >> 15)
    return Fraction(1024 + m, 1024) * Fraction(2) ** (e - 15)


if __name__ == "__main__":
    main()
