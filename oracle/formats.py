"""Oracle: number formats of the expert weights (test infrastructure only).

The FreeToken pages list BF16 and MXFP4 among the expert-weight formats its
GPU kernels run ("FreeToken 753b Model Explained", section "Performance
Benchmarks and Model Fit"; fervorai.dev article, section "What to know before
you commit").  They do not define MXFP4 bit by bit.  The definitions used
here are the public OCP Microscaling (MX) v1.0 ones:

* an MXFP4 block is 32 consecutive elements along the reduction axis K;
* each element is a 4-bit e2m1 code (1 sign, 2 exponent, 1 mantissa bit,
  exponent bias 1, no inf/NaN), value (-1)^s * 2^(E-1) * (1 + m/2) for E > 0
  and (-1)^s * m/2 for E = 0;
* the block shares one 8-bit e8m0 scale byte s, value 2^(s-127), s = 255 is
  NaN;
* packing (a reading, the pages are silent): element 2j is the low nibble of
  byte j and element 2j+1 its high nibble.

Encoding (a reading stated once, used everywhere): per block a = max|v|;
a == 0 gives scale byte 0 and all codes 0; otherwise the shared exponent is
X = floor(log2 a) - 2 (2 = the largest e2m1 exponent), clamped to
[-127, 127], scale byte X + 127; each element v / 2^X is rounded to the e2m1
grid with round-to-nearest, ties to the even code, saturating at +-6, sign
kept (so -0 encodes as code 8).

NVFP4 (the pages' format for their GLM and laptop builds, "FreeToken 753b
Model Explained", "Performance Benchmarks and Model Fit"; not defined there)
follows the public NVIDIA definition: e2m1 elements in blocks of 16 along K,
each block with an FP8 E4M3 scale (OCP E4M3FN: bias 7, 3 mantissa bits,
max 448, no infinities, 0x7F/0xFF NaN), and one fp32 scale per matrix.
Encoding (a reading; the steps are stated in fp32 so that an implementation
can reproduce them exactly): g = amax(matrix) / 2688 (= 6 * 448; g = 1 for
an all-zero matrix); per block t = amax(block) / (6 * g), rounded to E4M3
with round-to-nearest-even, saturating at 448; with d = E4M3(scale) * g
(fp32 product) each element v / d (fp32 quotient) is rounded to e2m1 as for
MXFP4; a block whose scale is 0 has all codes 0.  Value = e2m1 * E4M3 * g.

BF16 values are the top 16 bits of an IEEE binary32; fp32 -> bf16 uses
round-to-nearest-even (NaN kept quiet).

Pins (tests/test_oracle_formats.py):
  * the 16-entry e2m1 table (tests/golden/e2m1_codes.txt, from the OCP MX
    spec) against ``e2m1_decode``;
  * the RNE tie table and saturation, enumerated by hand in
    tests/golden/e2m1_rne_ties.txt;
  * encode(decode(b)) == b for every block whose largest code magnitude is
    >= 4 (the scale rule then reproduces the scale);
  * a block whose max is exactly 2^n gets scale byte n - 2 + 127;
  * ``bf16_round`` against PyTorch-CPU's fp32 -> bf16 cast (library routine)
    on random and edge values;
  * ``e4m3_decode`` on all 256 codes and ``e4m3_round`` on random values and
    every tie against PyTorch-CPU's float8_e4m3fn casts (library routine);
  * NVFP4: every code is the nearest e2m1 grid value to its quotient (brute
    force), scales and the global scale follow the stated fp32 steps, and
    values built exactly on the grid encode back to themselves.
"""

import numpy as np

# e2m1 magnitudes indexed by the low three bits (E1 E0 M) of a code.
# Written out from the format's definition, not derived from a formula.
_E2M1_MAGNITUDE = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def e2m1_decode(codes):
    """Value of each 4-bit e2m1 code (ints 0..15) as fp64."""
    codes = np.asarray(codes, dtype=np.int64)
    if np.any((codes < 0) | (codes > 15)):
        raise ValueError("e2m1 codes are 4-bit")
    mag = np.array(_E2M1_MAGNITUDE, dtype=np.float64)[codes & 7]
    sign = np.where((codes >> 3) & 1, -1.0, 1.0)
    return sign * mag


def e8m0_decode(s):
    """Value 2^(s-127) of an e8m0 scale byte as fp64 (255 -> NaN)."""
    s = np.asarray(s, dtype=np.int64)
    out = np.ldexp(np.ones(s.shape, dtype=np.float64), (s - 127).astype(np.int64))
    return np.where(s == 255, np.nan, out)


def unpack_nibbles(codes_u8):
    """[rows, K/2] bytes -> [rows, K] codes, low nibble first."""
    codes_u8 = np.asarray(codes_u8, dtype=np.uint8)
    lo = codes_u8 & 0x0F
    hi = codes_u8 >> 4
    out = np.empty(codes_u8.shape[:-1] + (codes_u8.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def pack_nibbles(codes):
    """[rows, K] codes (0..15) -> [rows, K/2] bytes, low nibble first."""
    codes = np.asarray(codes, dtype=np.uint8)
    if codes.shape[-1] % 2:
        raise ValueError("K must be even")
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def mxfp4_decode(codes_u8, scales_u8):
    """Exact fp64 values of an MXFP4 matrix.

    codes_u8  [rows, K/2] uint8, two e2m1 codes per byte (low nibble first)
    scales_u8 [rows, K/32] uint8, one e8m0 scale per 32-element block
    """
    codes = unpack_nibbles(codes_u8)
    rows, K = codes.shape
    scales_u8 = np.asarray(scales_u8, dtype=np.uint8)
    if scales_u8.shape != (rows, K // 32) or K % 32:
        raise ValueError("scale shape must be [rows, K/32]")
    vals = e2m1_decode(codes)
    scale = np.repeat(e8m0_decode(scales_u8), 32, axis=1)
    return vals * scale


def e2m1_round(r):
    """Round fp64 values (already divided by the block scale) to e2m1 codes.

    Nearest representable magnitude in {0, .5, 1, 1.5, 2, 3, 4, 6}; a value
    exactly half way between two neighbours takes the one whose code has
    mantissa bit 0 (the even code); magnitudes above 6 saturate to 6.  The
    sign bit is the sign of r (so -0.0 and small negatives give code 8).
    """
    r = np.asarray(r, dtype=np.float64)
    flat = r.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    step = 1 << 15          # work in cache-sized pieces; no effect on results
    for lo in range(0, flat.size, step):
        out[lo:lo + step] = _e2m1_round_piece(flat[lo:lo + step])
    return out.reshape(r.shape)


def _e2m1_round_piece(r):
    mag = np.minimum(np.abs(r), 6.0)
    # scan the 8 grid magnitudes keeping the closest; on an exact tie the
    # candidate with the even code (mantissa bit 0) wins
    best_idx = np.zeros(mag.shape, dtype=np.uint8)
    best_d = np.abs(mag - _E2M1_MAGNITUDE[0])
    for g in range(1, 8):
        d = np.abs(mag - _E2M1_MAGNITUDE[g])
        take = d < best_d
        if g % 2 == 0:
            take |= (d == best_d) & ((best_idx & 1) == 1)
        best_idx[take] = g
        best_d[take] = d[take]
    sign = np.signbit(r).astype(np.uint8)
    return best_idx | (sign << 3)


def mxfp4_encode(v):
    """Quantise fp32/fp64 values [rows, K] (K % 32 == 0) to MXFP4.

    Returns (codes_u8 [rows, K/2], scales_u8 [rows, K/32]).
    """
    v = np.asarray(v, dtype=np.float64)
    if v.ndim != 2 or v.shape[1] % 32:
        raise ValueError("expected [rows, K] with K a multiple of 32")
    rows, K = v.shape
    blocks = v.reshape(rows, K // 32, 32)
    amax = np.max(np.abs(blocks), axis=-1)
    # floor(log2 a) from frexp: a = m * 2^e with m in [0.5, 1) -> e - 1
    _, e = np.frexp(amax)
    X = np.clip(e.astype(np.int64) - 1 - 2, -127, 127)
    X = np.where(amax == 0, -127, X)
    scales = (X + 127).astype(np.uint8)
    r = np.ldexp(blocks, -X[..., None])
    codes = e2m1_round(r)
    codes = np.where((amax == 0)[..., None], np.uint8(0), codes)
    return pack_nibbles(codes.reshape(rows, K)), scales


def bf16_round(x32):
    """fp32 array -> bf16 bit patterns (uint16), round to nearest even."""
    x32 = np.ascontiguousarray(np.asarray(x32, dtype=np.float32))
    u = x32.view(np.uint32).astype(np.uint64)
    is_nan = np.isnan(x32)
    lsb = (u >> 16) & 1
    rounded = (u + 0x7FFF + lsb) >> 16
    out = (rounded & 0xFFFF).astype(np.uint16)
    nan_bits = ((u >> 16) | 0x40).astype(np.uint16)
    return np.where(is_nan, nan_bits, out)


def bf16_decode(bits):
    """bf16 bit patterns (uint16) -> exact fp64 values."""
    bits = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return bits.view(np.float32).astype(np.float64)


def e4m3_decode(s):
    """Value of each FP8 E4M3FN byte (OCP) as fp64; 0x7F / 0xFF are NaN."""
    s = np.asarray(s, dtype=np.int64)
    sign = np.where(s & 0x80, -1.0, 1.0)
    e = (s >> 3) & 0xF
    m = (s & 7).astype(np.float64)
    val = np.where(e == 0, m * 2.0 ** -9,
                   np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64)))
    val = np.where((s & 0x7F) == 0x7F, np.nan, val)
    return sign * val


# non-negative E4M3 magnitudes of codes 0 .. 126, increasing with the code
_E4M3_MAG = e4m3_decode(np.arange(127))


def e4m3_round(t):
    """Non-negative values -> E4M3 codes (0 .. 126): nearest magnitude, a tie
    going to the even code, values above 448 saturating to 448 (0x7E)."""
    t = np.asarray(t, dtype=np.float64)
    flat = np.minimum(t.reshape(-1), 448.0)
    if np.any(flat < 0) or np.any(np.isnan(flat)):
        raise ValueError("E4M3 scales are rounded from non-negative values")
    hi = np.clip(np.searchsorted(_E4M3_MAG, flat, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_lo = np.abs(flat - _E4M3_MAG[lo])
    d_hi = np.abs(_E4M3_MAG[hi] - flat)
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((hi & 1) == 0))
    return np.where(take_hi, hi, lo).astype(np.uint8).reshape(t.shape)


def nvfp4_encode(v):
    """Quantise values [rows, K] (K % 16 == 0) to NVFP4 with the fp32 steps
    above.  Returns (codes_u8 [rows, K/2], scales_u8 [rows, K/16], g fp32)."""
    v = np.asarray(v, dtype=np.float32)
    if v.ndim != 2 or v.shape[1] % 16:
        raise ValueError("expected [rows, K] with K a multiple of 16")
    rows, K = v.shape
    amax_t = np.float32(np.max(np.abs(v))) if v.size else np.float32(0)
    g = np.float32(amax_t / np.float32(2688.0)) if amax_t > 0 else np.float32(1.0)
    blocks = v.reshape(rows, K // 16, 16)
    amax_b = np.max(np.abs(blocks), axis=-1).astype(np.float32)
    t = (amax_b / np.float32(np.float32(6.0) * g)).astype(np.float32)
    scales = e4m3_round(t.astype(np.float64))
    d = (e4m3_decode(scales).astype(np.float32) * g).astype(np.float32)
    safe = np.where(d > 0, d, np.float32(1.0)).astype(np.float32)
    q = (blocks / safe[..., None]).astype(np.float32)
    codes = e2m1_round(q.astype(np.float64))
    codes = np.where((d > 0)[..., None], codes, np.uint8(0))
    return pack_nibbles(codes.reshape(rows, K)), scales, g


def nvfp4_decode(codes_u8, scales_u8, g):
    """Exact fp64 values of an NVFP4 matrix: e2m1 * E4M3 scale * g."""
    codes = unpack_nibbles(codes_u8)
    rows, K = codes.shape
    scales_u8 = np.asarray(scales_u8, dtype=np.uint8)
    if scales_u8.shape != (rows, K // 16) or K % 16:
        raise ValueError("scale shape must be [rows, K/16]")
    scale = np.repeat(e4m3_decode(scales_u8), 16, axis=1)
    return e2m1_decode(codes) * scale * float(np.float32(g))
