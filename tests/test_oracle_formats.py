"""Pins of the oracle's number formats (CPU only)."""

import os

import numpy as np
import pytest
import torch

from conftest import GOLDEN
from oracle import formats


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                a, b = line.split()
                rows.append((a, b))
    return rows


def test_e2m1_table_matches_spec_fixture():
    rows = _read_table("e2m1_codes.txt")
    assert len(rows) == 16
    codes = np.array([int(a) for a, _ in rows])
    want = np.array([float(b) for _, b in rows])
    got = formats.e2m1_decode(codes)
    assert np.array_equal(got, want)
    # the sign of zero is kept: code 8 is -0.0
    assert np.signbit(got[8]) and not np.signbit(got[0])


def test_e2m1_table_matches_closed_form():
    # (-1)^s * 2^(E-1) * (1 + m/2) for E > 0, (-1)^s * m/2 for E == 0
    for c in range(16):
        s, E, m = c >> 3, (c >> 1) & 3, c & 1
        mag = 2.0 ** (E - 1) * (1 + m / 2) if E > 0 else m / 2
        want = -mag if s else mag
        assert formats.e2m1_decode([c])[0] == want


def test_e8m0_scale_values():
    s = np.arange(255)
    got = formats.e8m0_decode(s)
    assert np.array_equal(got, 2.0 ** (s.astype(np.float64) - 127))
    assert np.isnan(formats.e8m0_decode([255])[0])


def test_rne_tie_table_and_saturation():
    for r, code in _read_table("e2m1_rne_ties.txt"):
        got = int(formats.e2m1_round(np.array([float(r)]))[0])
        assert got == int(code), (r, got, code)


def test_decode_nibble_order_and_scale():
    # one row, K = 32: byte j holds element 2j (low) and 2j+1 (high)
    codes = np.zeros((1, 16), dtype=np.uint8)
    codes[0, 0] = 0x71          # elem0 = code 1 (0.5), elem1 = code 7 (6)
    codes[0, 15] = 0xA3         # elem30 = code 3 (1.5), elem31 = code 10 (-1)
    scales = np.array([[127 + 3]], dtype=np.uint8)   # 2^3
    v = formats.mxfp4_decode(codes, scales)
    assert v.shape == (1, 32)
    assert v[0, 0] == 4.0 and v[0, 1] == 48.0
    assert v[0, 30] == 12.0 and v[0, 31] == -8.0
    assert np.all(v[0, 2:30] == 0.0)


def test_encode_zero_block_and_negative_zero():
    v = np.zeros((2, 64))
    v[1, 32:] = 1.0
    v[1, 33] = -0.0
    codes, scales = formats.mxfp4_encode(v)
    assert scales[0, 0] == 0 and scales[0, 1] == 0 and scales[1, 0] == 0
    assert np.all(codes[0] == 0) and np.all(codes[1, :16] == 0)
    # block of ones: X = floor(log2 1) - 2 = -2 -> byte 125, r = 4 -> code 6;
    # -0.0 keeps its sign -> code 8
    assert scales[1, 1] == 125
    unpacked = formats.unpack_nibbles(codes)
    assert unpacked[1, 32] == 6 and unpacked[1, 33] == 8


@pytest.mark.parametrize("n", [-20, -7, 0, 3, 60])
def test_scale_rule_power_of_two_max(n):
    rng = np.random.default_rng(n + 100)
    v = rng.uniform(-1, 1, size=(3, 32)) * 2.0 ** n
    v[:, 5] = 2.0 ** n
    codes, scales = formats.mxfp4_encode(v)
    assert np.all(scales[:, 0] == n - 2 + 127)
    assert np.all(formats.unpack_nibbles(codes)[:, 5] == 6)


def test_encode_decode_idempotent():
    rng = np.random.default_rng(7)
    rows, K = 64, 256
    codes = rng.integers(0, 16, size=(rows, K), dtype=np.uint8)
    # make every block's largest magnitude code >= 4 (code & 7 >= 6)
    for b in range(K // 32):
        codes[:, b * 32 + rng.integers(0, 32)] = rng.choice([6, 7, 14, 15], size=rows)
    scales = rng.integers(1, 254, size=(rows, K // 32), dtype=np.uint8)
    packed = formats.pack_nibbles(codes)
    v = formats.mxfp4_decode(packed, scales)
    c2, s2 = formats.mxfp4_encode(v)
    assert np.array_equal(s2, scales)
    assert np.array_equal(c2, packed)


def test_encode_error_bound_random():
    # RNE on the e2m1 grid: |r - q(r)| <= half the local grid step, with
    # step 0.5 below 2, 1 in [2, 4), 2 in [4, 6]; saturation above 6.
    rng = np.random.default_rng(3)
    v = rng.standard_normal((128, 128)) * 0.02
    codes, scales = formats.mxfp4_encode(v)
    dq = formats.mxfp4_decode(codes, scales)
    scale = np.repeat(formats.e8m0_decode(scales), 32, axis=1)
    r = np.abs(v) / scale
    step = np.where(r < 2, 0.5, np.where(r < 4, 1.0, 2.0))
    err = np.abs(v - dq) / scale
    bound = np.where(r > 6, r - 6, step / 2)
    assert np.all(err <= bound + 1e-12)


def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(11)
    vals = np.concatenate([
        rng.standard_normal(500_000).astype(np.float32),
        (rng.standard_normal(200_000) * 1e-38).astype(np.float32),   # denormals
        (rng.standard_normal(200_000) * 1e30).astype(np.float32),
        rng.integers(0, 2**32, size=100_000, dtype=np.uint64).astype(np.uint32).view(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.4028235e38, -3.4028235e38,
                  1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-8 + 2**-20], dtype=np.float32),
    ])
    ours = formats.bf16_round(vals)
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    finite = ~np.isnan(vals)
    assert np.array_equal(ours[finite], ref[finite])
    # NaN stays NaN
    assert np.all(np.isnan(formats.bf16_decode(ours[~finite])))


def test_bf16_decode_exact():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    vals = formats.bf16_decode(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ok = ~np.isnan(ref)
    assert np.array_equal(vals[ok], ref[ok])


# ------------------------------------------------------------------ NVFP4
def test_e4m3_decode_matches_torch_float8_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = formats.e4m3_decode(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_e4m3_round_matches_torch_cast_with_ties():
    rng = np.random.default_rng(11)
    mags = formats.e4m3_decode(np.arange(127))
    mids = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)   # every tie
    t = np.concatenate([rng.uniform(0, 448, 50000), rng.uniform(0, 0.05, 50000),
                        mids, mags.astype(np.float32)]).astype(np.float32)
    ref = torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(formats.e4m3_round(t.astype(np.float64)), ref)
    assert formats.e4m3_round(np.array([1000.0]))[0] == 0x7E      # saturation


def _nearest_e2m1_brute(q):
    """Nearest e2m1 magnitude by exhaustive search, ties to the even code."""
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    out = np.empty(q.shape, dtype=np.uint8)
    for i, x in np.ndenumerate(q):
        a = min(abs(float(x)), 6.0)
        best = min(range(8), key=lambda c: (abs(a - grid[c]), c & 1))
        out[i] = best | (8 if np.signbit(x) else 0)
    return out


def test_nvfp4_steps_and_nearest_codes():
    rng = np.random.default_rng(12)
    v = (rng.normal(0, 0.02, (8, 64)) * rng.uniform(0.1, 10, (8, 1))).astype(np.float32)
    codes_u8, scales, g = formats.nvfp4_encode(v)
    assert g == np.float32(np.float32(np.abs(v).max()) / np.float32(2688.0))
    blocks = v.reshape(8, 4, 16)
    amax_b = np.abs(blocks).max(-1).astype(np.float32)
    t = (amax_b / np.float32(np.float32(6.0) * g)).astype(np.float32)
    ref_s = torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(scales, ref_s)
    d = (formats.e4m3_decode(scales).astype(np.float32) * g).astype(np.float32)
    q = (blocks / d[..., None]).astype(np.float32)
    codes = formats.unpack_nibbles(codes_u8).reshape(8, 4, 16)
    assert np.array_equal(codes, _nearest_e2m1_brute(q))
    # values are e2m1 * scale * g
    dec = formats.nvfp4_decode(codes_u8, scales, g)
    ref = formats.e2m1_decode(codes.reshape(8, 64)) * np.repeat(
        formats.e4m3_decode(scales), 16, axis=1) * float(g)
    assert np.array_equal(dec, ref)


def test_nvfp4_zero_and_on_grid_round_trip():
    codes_u8, scales, g = formats.nvfp4_encode(np.zeros((2, 32), np.float32))
    assert g == 1.0 and not scales.any() and not codes_u8.any()
    # a block holding +-6, 4, ... at scale 1 with the matrix max 6 * 448 * g
    grid = np.array([6, -6, 4, -4, 3, 2, 1.5, 1, 0.5, 0, -0.5, -1, -1.5, -2, -3, 6],
                    np.float32)
    v = np.stack([grid * np.float32(448.0), grid]).astype(np.float32)   # two rows
    codes_u8, scales, g = formats.nvfp4_encode(v)
    assert np.array_equal(formats.nvfp4_decode(codes_u8, scales, g), v.astype(np.float64))
