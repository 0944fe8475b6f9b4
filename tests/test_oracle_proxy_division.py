"""Pin of the proxy mean's division for member counts that are not powers of two.

The proxy of a group is the binary32 mean of its members, added in ascending
position and then divided by the member count with one IEEE division
(molayo1419.me "PIVOT explained", How It Works: the proxy is the group mean;
the binary32 order is the reading that lets the GPU match it bit for bit).
For n in {3, 5, 6, 7} a multiply by the rounded reciprocal 1/n differs from the
division by one unit in the last place for some sums.  The inputs below are
built so that this unit decides the stored result:

  * bf16: sums whose correctly rounded quotient lies one binary32 unit below a
    bf16 rounding midpoint while the reciprocal product lands on it (or the
    reverse), so the two give different bf16 codes.  Such sums exist for
    n = 3, 6 and 7 but not for n = 5: a binary32 sum of five members' mean is a
    multiple of 4/5 of the mean's unit, while bf16 midpoints are multiples of
    2^15 units, so the two results never fall on both sides of a midpoint;
  * the head weights w: sums where the two binary32 results differ;
  * fp8: a group whose largest mean is such a quotient, so the proxy scale
    amax/448 differs.

Expected values come from exact rational arithmetic rounded to binary32 by
hand (round to nearest, ties to even) and from PyTorch's bf16 / E4M3 casts,
which the codec pins tie to the formats; nothing here calls the oracle's own
arithmetic.  Each case also checks, with a numpy model of the mistake, that the
reciprocal product would have given another result.  CPU only.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

COUNTS = (3, 5, 6, 7)


def round_f32(x: Fraction) -> np.float32:
    """The binary32 value nearest to the rational x (ties to the even
    significand); normal range only."""
    if x == 0:
        return np.float32(0.0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    assert -126 <= e <= 127, "normal binary32 range only"
    ulp = Fraction(2) ** (e - 23)
    q = a / ulp
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return np.float32(sign * float(n * ulp))


def bf16_code(x: np.float32) -> int:
    return int(torch.tensor([x], dtype=torch.float32).to(torch.bfloat16).view(torch.int16)[0]) & 0xFFFF


def e4m3_code(x: np.float32) -> int:
    return int(torch.tensor([x], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)[0])


def recip_mean(s: np.float32, n: int) -> np.float32:
    """The mistake: multiply by the binary32 reciprocal of n."""
    return np.float32(np.float32(s) * (np.float32(1.0) / np.float32(n)))


def bf16_pieces(s: np.float32, n: int):
    """n bf16 values whose binary32 sum, added in order, is exactly s (the
    24-bit significand in three 8-bit pieces, then zeros)."""
    parts = []
    r = np.float32(s)
    for _ in range(3):
        top = np.array([r], np.float32).view(np.uint32)[0] & np.uint32(0xFFFF0000)
        p = np.array([top], np.uint32).view(np.float32)[0]
        parts.append(p)
        r = np.float32(r - p)
    assert r == 0
    parts += [np.float32(0.0)] * (n - 3)
    acc = np.float32(0.0)
    for p in parts:
        acc = np.float32(acc + p)
    assert acc == s
    return parts


def bf16_cases(n: int, want: int):
    """Sums s for which bf16(s / n) differs from bf16(s * (1/n))."""
    found = []
    for ex in range(-3, 4):
        for j in range(128):
            mid = Fraction(256 + 2 * j + 1, 256) * Fraction(2) ** ex  # a bf16 rounding midpoint
            s0 = np.float32(float(mid * n))
            for k in range(-6, 7):
                s = np.float32(s0)
                step = np.float32(np.inf if k > 0 else -np.inf)
                for _ in range(abs(k)):
                    s = np.nextafter(s, step, dtype=np.float32)
                good = bf16_code(round_f32(Fraction(float(s)) / n))
                bad = bf16_code(recip_mean(s, n))
                if good != bad:
                    found.append(s)
                    break
            if len(found) >= want:
                return found
    return found


def f32_cases(n: int, want: int, seed: int):
    rng = np.random.default_rng(seed)
    found = []
    while len(found) < want:
        s = np.float32(rng.uniform(0.5, 4.0))
        if round_f32(Fraction(float(s)) / n) != recip_mean(s, n):
            found.append(s)
    return found


@pytest.mark.parametrize("n", COUNTS)
def test_bf16_proxy_division_is_correctly_rounded(n):
    D = 32
    H = 4
    cases = bf16_cases(n, H * D) if n != 5 else [np.float32(1.0)] * (H * D)
    assert len(cases) == H * D, f"only {len(cases)} sensitive sums found for n={n}"
    # member t holds piece t of every element's sum
    q = np.zeros((n, H, D), np.float32)
    for e, s in enumerate(cases):
        for t, p in enumerate(bf16_pieces(s, n)):
            q[t].reshape(-1)[e] = p
    qc = (q.view(np.uint32) >> 16).astype(np.uint16)  # exact: every piece is a bf16 value
    wsums = f32_cases(n, H, seed=10 + n)
    w = np.zeros((n, H), np.float32)
    w[0] = wsums
    v = oracle.View("bf16", qc, None, w, np.zeros((1, D), np.uint16), None)
    codes, scale, wbar = oracle.proxy(v, 0, n)
    expected = np.array([bf16_code(round_f32(Fraction(float(s)) / n)) for s in cases], np.uint16)
    mistaken = np.array([bf16_code(recip_mean(s, n)) for s in cases], np.uint16)
    assert np.array_equal(codes.reshape(-1), expected)
    if n != 5:
        assert np.all(mistaken != expected)  # the reciprocal product fails every element
    exp_w = np.array([round_f32(Fraction(float(s)) / n) for s in wsums], np.float32)
    assert np.array_equal(wbar, exp_w)
    assert np.all(np.array([recip_mean(s, n) for s in wsums]) != exp_w)
    assert scale == 1.0


@pytest.mark.parametrize("n", COUNTS)
def test_fp8_proxy_scale_and_codes_use_the_correctly_rounded_mean(n):
    """fp8 members carry per-row scales; element 0's member values are
    fl(s_t * 448) in row 0 and 0 elsewhere, so its mean is the group's largest
    and sets the proxy scale amax/448."""
    H, D = 2, 64
    rng = np.random.default_rng(100 + n)
    for trial in range(200):
        scales = rng.uniform(0.005, 0.01, n).astype(np.float32)
        codes_in = rng.integers(0, 0x48, (n, H, D)).astype(np.uint8)  # values up to 7.5
        codes_in[:, 0, 0] = 0
        codes_in[0, 0, 0] = 0x7E  # 448
        # binary32 member values fl(s_t * e4m3(c)), exact rationals rounded by hand
        e4m3 = torch.from_numpy(codes_in.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        vals = np.empty((n, H * D), np.float32)
        for t in range(n):
            for e in range(H * D):
                vals[t, e] = round_f32(Fraction(float(scales[t])) * Fraction(float(e4m3[t].reshape(-1)[e])))
        sums = np.zeros(H * D, np.float32)
        for t in range(n):
            sums = (sums + vals[t]).astype(np.float32)
        means = np.array([round_f32(Fraction(float(s)) / n) for s in sums], np.float32)
        amax = np.abs(means).max()
        sp = round_f32(Fraction(float(amax)) / 448)
        bad_means = np.array([recip_mean(s, n) for s in sums], np.float32)
        bad_sp = np.float32(np.abs(bad_means).max() / np.float32(448))
        if bad_sp == sp:
            continue  # this draw does not separate the two; try another
        v = oracle.View("fp8", codes_in, scales, np.ones((n, H), np.float32),
                        np.zeros((1, D), np.uint8), np.ones(1, np.float32))
        got_codes, got_sp, _ = oracle.proxy(v, 0, n)
        assert got_sp == sp
        exp_codes = np.array([e4m3_code(round_f32(Fraction(float(m)) / Fraction(float(sp))))
                              for m in means], np.uint8)
        assert np.array_equal(got_codes.reshape(-1), exp_codes)
        return
    pytest.fail(f"no separating draw found for n={n}")


def test_partial_last_group_uses_the_member_count():
    """A sequence of 8 + 7 queries with g = 8: the last group's proxy is the
    mean over its 7 members (the same division as above)."""
    n = 7
    cases = bf16_cases(n, 32)
    q = np.zeros((8 + n, 1, 32), np.float32)
    for e, s in enumerate(cases):
        for t, p in enumerate(bf16_pieces(s, n)):
            q[8 + t, 0, e] = p
    qc = (q.view(np.uint32) >> 16).astype(np.uint16)
    v = oracle.View("bf16", qc, None, np.ones((8 + n, 1), np.float32), np.zeros((1, 32), np.uint16), None)
    codes, _, _ = oracle.proxy(v, 8, n)
    expected = np.array([bf16_code(round_f32(Fraction(float(s)) / n)) for s in cases], np.uint16)
    assert np.array_equal(codes.reshape(-1), expected)
    assert np.all(np.array([bf16_code(recip_mean(s, n)) for s in cases], np.uint16) != expected)


def test_round_f32_matches_ieee_division_on_simple_cases():
    """The hand rounding agrees with the binary32 division numpy performs,
    including exact ties (ties to even)."""
    rng = np.random.default_rng(5)
    for _ in range(2000):
        a = np.float32(rng.uniform(-100, 100))
        b = np.float32(rng.choice([3, 5, 6, 7, 9, 11]))
        assert round_f32(Fraction(float(a)) / Fraction(float(b))) == np.float32(a / b)
    one_plus_half_ulp = Fraction(1) + Fraction(1, 2 ** 24)
    assert round_f32(one_plus_half_ulp) == np.float32(1.0)  # tie -> even
    assert round_f32(Fraction(1) + Fraction(3, 2 ** 24)) == np.float32(1.0 + 2 ** -22)
