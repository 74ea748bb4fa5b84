"""Number-format primitives of the oracle (test infrastructure only).

The QATFactory project page's "Supported formats" table names the element and
scale types: E2M1 (FP4) elements with E4M3 block scales and an FP32 tensor
scale (NVFP4), E2M1 elements with E8M0 block scales (MXFP4), unsigned INT4
codes with 6-bit block scales under FP16 super-block scales (Q4_K).  The page
does not spell out their bit layouts or rounding; the readings used here are
the standard ones for these type names:

* bf16: the top 16 bits of a binary32.  Widening is exact; narrowing is
  round-to-nearest-even (RNE) on the 16 dropped bits.
* fp16: IEEE binary16 with subnormals, RNE; finite values beyond the largest
  finite fp16 saturate to +-65504 (a stated choice; never reached by the
  workloads).
* E4M3 (the "FN" flavour: bias 7, no infinities, 0x7F is NaN): finite
  magnitudes 0, k*2^-9 (k = 1..7) and (1 + m/8)*2^(e-7) for e = 1..15,
  m = 0..7 except e = 15, m = 7; largest finite value 448.  Encoding takes the
  nearest finite value with ties to the even code (RNE), so anything above 448
  saturates to 448.
* E8M0: byte E means 2^(E-127), E = 0..254.
* E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0; magnitudes
  {0, 0.5, 1, 1.5, 2, 3, 4, 6}.  Encoding takes the nearest magnitude with ties
  to the even code (mantissa bit 0); anything above 6 saturates to 6.  A NaN
  scaled value (only 0 * inf can produce one) encodes to magnitude 0, which is
  what a comparison-based encoder gives, since every comparison with NaN fails.

Nearest-value encoders are written as the plain definition: the sorted table of
representable magnitudes, the exact midpoints between neighbours, and a count
of the midpoints strictly below the input, with an exact tie sending the input
to the even code.  All comparisons are exact (float64 holds every value
involved exactly).

Pins (tests/test_oracle_primitives.py): bf16 narrowing against torch's
float32->bfloat16 cast; fp16 against a brute-force nearest search; E4M3 against
torch's float8_e4m3fn cast (after clamping to 448) and a brute-force search;
E2M1 against a brute-force argmin over all 65,536 bf16 inputs; E8M0 against
torch's float8_e8m0fnu decode.
"""

import numpy as np

F32 = np.float32


# ---------------------------------------------------------------- bf16 -----
def bf16_to_f32(bits):
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    return (b << np.uint32(16)).view(np.float32)


def f32_to_bf16(x):
    """Round float32 to bf16 bit patterns, round-to-nearest-even.

    Keep the high 16 bits; round the magnitude up by one bf16 ulp when the
    dropped 16 bits exceed half an ulp, or equal half an ulp and the kept
    pattern is odd.  Finite inputs only (the only ones the method produces).
    """
    b = np.asarray(x, dtype=np.float32).view(np.uint32)
    hi = (b >> np.uint32(16)).astype(np.uint32)
    rem = b & np.uint32(0xFFFF)
    up = (rem > 0x8000) | ((rem == 0x8000) & ((hi & 1) == 1))
    return (hi + up.astype(np.uint32)).astype(np.uint16)


# ---------------------------------------------------------------- fp16 -----
FP16_MAX = 65504.0


def f32_to_f16_bits(x):
    """float32 -> IEEE binary16 bits, RNE with subnormals, saturating at 65504."""
    x = np.asarray(x, dtype=np.float32)
    clipped = np.clip(x, F32(-FP16_MAX), F32(FP16_MAX))
    return clipped.astype(np.float16).view(np.uint16)


def f16_bits_to_f32(bits):
    """Exact widening of binary16 bits to float32."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


# ------------------------------------------------ nearest-value encoders ---
def _nearest_code(u, table):
    """Index of the nearest entry of the increasing table ``table`` to each u >= 0.

    Ties go to the even index.  ``u`` above the last entry maps to the last
    entry (saturation).  NaN maps to index 0.
    """
    u = np.asarray(u, dtype=np.float64)
    mid = (table[:-1] + table[1:]) / 2.0           # exact: few significant bits
    below = np.searchsorted(mid, u, side="left")   # midpoints strictly below u
    at_mid = np.zeros(u.shape, dtype=bool)
    inside = below < mid.size
    at_mid[inside] = u[inside] == mid[below[inside]]
    # tie between index `below` and `below + 1`: choose the even one
    code = np.where(at_mid & (below % 2 == 1), below + 1, below)
    code = np.where(np.isnan(u), 0, code)
    return code.astype(np.uint8)


# ---------------------------------------------------------------- E2M1 -----
E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def e2m1_value(code):
    """Signed value of a 4-bit E2M1 code (bit 3 = sign), as float32."""
    code = np.asarray(code, dtype=np.uint8)
    mag = E2M1_MAG[code & 7].astype(np.float32)
    return np.where((code & 8) != 0, -mag, mag).astype(np.float32)


def e2m1_encode_mag(y):
    """Magnitude code 0..7 of y >= 0: nearest E2M1 magnitude, ties to even, saturating."""
    return _nearest_code(y, E2M1_MAG)


# ---------------------------------------------------------------- E4M3 -----
def _e4m3_table():
    vals = []
    for code in range(0x7F):                       # 0x7F is NaN
        e, m = code >> 3, code & 7
        if e == 0:
            vals.append(m * 2.0 ** -9)
        else:
            vals.append((1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals, dtype=np.float64)


E4M3_POS = _e4m3_table()                            # codes 0x00..0x7E, increasing
E4M3_MAX = 448.0


def e4m3_value(code):
    """Value of a non-negative E4M3 code 0x00..0x7E, as float32."""
    return E4M3_POS[np.asarray(code, dtype=np.uint8)].astype(np.float32)


def e4m3_encode(u):
    """E4M3 code of u >= 0: RNE to the nearest finite value, saturating at 448."""
    return _nearest_code(u, E4M3_POS)


# ---------------------------------------------------------------- E8M0 -----
def e8m0_value(E):
    """2^(E-127) as float32 (E = 0..254; E = 0 gives the binary32 subnormal 2^-127)."""
    E = np.asarray(E, dtype=np.int64)
    return np.ldexp(np.float64(1.0), E - 127).astype(np.float32)


def floor_log2(a):
    """floor(log2 a) for finite a > 0 (exact, via frexp)."""
    _, ex = np.frexp(np.asarray(a, dtype=np.float64))
    return ex.astype(np.int64) - 1


def rint(x):
    """Round half to even to an integer value (float input, float output)."""
    return np.rint(x)
