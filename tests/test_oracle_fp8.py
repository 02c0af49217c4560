"""Pins of the oracle's FP8 E4M3 static-scale tier (CPU only).

The per-tensor FP8 tier of the Coder390 calibration note (§3, layer table of
the mixed W4A4+W8A8 tier) is checked against things other than the oracle:
exact rational arithmetic and brute force, torch's float8_e4m3fn casts, and
closed-form special cases."""
from fractions import Fraction

import numpy as np
import torch

import datagen
from oracle import fp8 as P8
from oracle import formats as F


def _round_f32(q: Fraction) -> Fraction:
    """Exact round-to-nearest-even of a positive rational to float32 (integer
    arithmetic; subnormals on the 2^-149 grid)."""
    if q == 0:
        return Fraction(0)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1                                     # now 2^e <= q < 2^(e+1)
    ulp = Fraction(2) ** (max(e, -126) - 23)
    n = q / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    r = fl + (1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1) else 0)
    return r * ulp


def _e4m3_mags():
    return [Fraction(float(v)) for v in F.E4M3_VALUES[:127]]


def _brute_code(x: float, s: float) -> int:
    """Nearest finite E4M3 magnitude to |x|/s by exhaustive search (ties to the
    even code), sign in bit 7; s = 0 saturates any nonzero x."""
    mags = _e4m3_mags()
    ax = Fraction(abs(x))
    sign = 0x80 if np.signbit(x) else 0
    if s == 0.0:
        return (0x7E if ax > 0 else 0) | sign
    q = ax / Fraction(s)
    best, bd = 0, None
    for c, m in enumerate(mags):
        dd = abs(q - m)
        if bd is None or dd < bd or (dd == bd and c % 2 == 0):
            best, bd = c, dd
    return best | sign


def test_fp8_scale_is_correctly_rounded_for_every_bf16_amax():
    bits = np.arange(1, 0x7F80, dtype=np.uint16)          # every positive finite bf16
    _, s = zip(*[P8.fp8_tensor_scale(np.array([b], np.uint16)) for b in bits[::7]])
    vals = F.bf16_bits_to_f64(bits[::7])
    for a, got in zip(vals, s):
        assert Fraction(got) == _round_f32(Fraction(float(a)) / 448), a
    # and the whole range at once against float32 division of exact inputs,
    # which IEEE rounds correctly (a library primitive)
    all_s = np.float32(F.bf16_bits_to_f64(bits)) / np.float32(448.0)
    ref = np.array([P8.fp8_tensor_scale(np.array([b], np.uint16))[1] for b in bits[::97]])
    assert np.array_equal(ref, all_s[::97].astype(np.float64))


def test_fp8_quantize_equals_brute_force():
    rng = np.random.default_rng(8)
    for s in (0.02, 1.0 / 3.0, 2.0 ** -20, 7.5e-3, 1e-30, 123.456):
        s = float(np.float32(s))
        mags = F.E4M3_VALUES[:127]
        picks = rng.integers(0, 127, 300)
        exact = mags[picks] * s                                          # on the grid
        mids = 0.5 * (mags[picks[:150] % 126] + mags[picks[:150] % 126 + 1]) * s   # midpoints
        rand = np.exp(rng.uniform(-12, 7, 300)) * s                       # anywhere, incl. > 448 s
        x = np.concatenate([exact, mids, rand, [0.0, 470.0 * s, 1e3 * s]])
        x = x * rng.choice([-1.0, 1.0], x.size)
        bits = F.f64_to_bf16_bits(F.f32(x))
        xs = F.bf16_bits_to_f64(bits)
        got = P8.fp8_quantize(bits, s)
        want = np.array([_brute_code(v, s) for v in xs], dtype=np.uint8)
        assert np.array_equal(got, want), s


def test_fp8_quantize_matches_torch_cast_on_exact_quotients():
    """With a power-of-two scale the quotient is exact in float32, so torch's
    float8_e4m3fn cast (nearest even) must agree below the saturation point."""
    bits = np.arange(0, 0x10000, dtype=np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]                 # finite only
    for s in (2.0 ** -4, 1.0, 2.0 ** 6):
        x = F.bf16_bits_to_f64(bits)
        keep = np.abs(x / s) <= 448.0
        q = torch.from_numpy((x[keep] / s).astype(np.float32)).to(torch.float8_e4m3fn)
        want = q.view(torch.uint8).numpy()
        got = P8.fp8_quantize(bits[keep], s)
        assert np.array_equal(got, want), s


def test_fp8_dequant_matches_torch_decode():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    for s in (0.0123, 1.0, 3.0e-5, 2.0 ** -130):
        s = float(np.float32(s))
        v = torch.from_numpy(codes).view(torch.float8_e4m3fn).float() * torch.tensor(s, dtype=torch.float32)
        want = v.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(P8.fp8_dequant(codes, s), want), s


def test_fp8_round_trip_and_special_cases():
    s = 2.0 ** -7
    mags = F.E4M3_VALUES[:127]
    x = np.concatenate([mags, -mags]) * s                   # bf16-exact (4 significant bits)
    bits = F.f64_to_bf16_bits(x)
    codes = P8.fp8_quantize(bits, s)
    assert np.array_equal(codes[:127], np.arange(127, dtype=np.uint8))
    assert np.array_equal(codes[127:], (np.arange(127) | 0x80).astype(np.uint8))
    assert np.array_equal(P8.fp8_dequant(codes, s), bits)
    # negative zero and negative tiny values keep the sign; saturation at 448 s
    tiny = F.f64_to_bf16_bits(np.array([-0.0, -1e-6 * s, 1e-6 * s, 500 * s, -1e5 * s]))
    assert list(P8.fp8_quantize(tiny, s)) == [0x80, 0x80, 0x00, 0x7E, 0xFE]
    # s = 0: zero stays zero, anything else saturates
    assert list(P8.fp8_quantize(F.f64_to_bf16_bits(np.array([0.0, -0.0, 1.5, -2.0])), 0.0)) == [0, 0x80, 0x7E, 0xFE]
    # scale of a tensor whose max is exactly 448 * 2^-3 is 2^-3
    t = F.f64_to_bf16_bits(np.array([448.0 * 2 ** -3, -1.0, 0.5]))
    assert P8.fp8_tensor_scale(t) == (56.0, 0.125)


def test_fp8_error_bound_on_activations():
    """|dequant(quantize(x)) - x| is at most half an E4M3 step at |x| (plus the
    two FP32/bf16 roundings) for unsaturated values."""
    x = datagen.config1()[1][:64]
    amax, s = P8.fp8_tensor_scale(x)
    xv = F.bf16_bits_to_f64(x)
    y = F.bf16_bits_to_f64(P8.fp8_dequant(P8.fp8_quantize(x, s), s))
    q = np.abs(xv) / s
    step = np.where(q < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(q, 2.0 ** -6))) - 3))
    assert np.all(np.abs(y - xv) <= 0.5 * step * s * (1 + 2.0 ** -7) + 2.0 ** -8 * np.abs(xv))
