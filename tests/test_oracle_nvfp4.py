"""Pins for the oracle's number codecs and its NVFP4 quantiser (O3).

The quantiser decides integer codes, so these pins are exact: a hand-worked
example, brute-force nearest-value searches written here from the format
definitions (OCP 8-bit Floating Point Specification for E4M3FN, OCP
Microscaling Formats v1.0 for E2M1), torch's own float8 and bfloat16 casts as
independent library routines, and closed-form properties of the recipe.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from workloads import make_qkv

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _e4m3_table():
    """All 127 finite non-negative E4M3FN values, from the bit layout."""
    vals = []
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        vals.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(vals)


E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)


def _nearest_even(x, table):
    """Index of the nearest table entry, ties to the even index (the one whose
    lowest code bit is 0); table is sorted ascending."""
    d = np.abs(table - x)
    best = np.flatnonzero(d == d.min())
    even = [i for i in best if i % 2 == 0]
    return int(even[0] if even else best[0])


# -------------------------------------------------------------- bf16 codec

def test_bf16_roundtrip_every_pattern():
    bits = np.arange(65536, dtype=np.uint16)
    vals = oracle.bf16_bits_to_f64(bits)
    nan = np.isnan(vals)
    assert nan.sum() == 2 * 127
    back = oracle.to_bf16_bits(vals[~nan])
    np.testing.assert_array_equal(back, bits[~nan])
    # widening agrees with torch's exact bf16 -> float64
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(vals[~nan], t[~nan])


def test_bf16_rounding_matches_torch_on_random_floats():
    rng = np.random.default_rng(0)
    u = rng.integers(0, 2 ** 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    u = u[(u & 0x7F800000) != 0x7F800000]            # finite only
    ties = (rng.integers(0, 2 ** 16, size=20000).astype(np.uint32) << 16) | 0x8000
    ties = ties[(ties & 0x7F800000) != 0x7F800000]
    f = np.concatenate([u, ties]).view(np.float32)
    mine = oracle.to_bf16_bits(f.astype(np.float64))
    ref = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(mine, ref)


def test_bf16_rounds_doubles_once():
    """Straight from binary64: 1 + 2^-8 + 2^-30 sits just above a bf16 tie and
    must round up, although its binary32 rounding (1 + 2^-8) is an exact tie
    that rounds to even (down)."""
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert oracle.to_bf16_bits(np.array([x]))[0] == 0x3F81
    assert oracle.to_bf16_bits(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80


# -------------------------------------------------------------- E4M3

def test_e4m3_values_from_bits():
    t = _e4m3_table()
    for c in range(0x7F):
        assert oracle.e4m3_value(c) == t[c]
    assert np.isnan(oracle.e4m3_value(0x7F))
    assert oracle.e4m3_value(0x7E) == 448.0 and oracle.e4m3_value(0x01) == 2.0 ** -9


def _e4m3_probe_points():
    t = _e4m3_table()
    mids = (t[1:] + t[:-1]) / 2
    pts = np.concatenate([t, mids, np.linspace(0, 500, 20001)])
    f = pts.astype(np.float32)
    up = np.nextafter(f, np.float32(np.inf))
    dn = np.nextafter(f, np.float32(0))
    return np.unique(np.concatenate([f, up, dn, [np.float32(464), np.float32(1e9)]]))


def test_e4m3_encode_is_nearest_even_with_saturation():
    t = _e4m3_table()
    x = _e4m3_probe_points()
    got = oracle.e4m3_encode_array(x)
    for xi, gi in zip(x, got):
        want = 0x7E if xi >= 448 else _nearest_even(float(xi), t)
        assert gi == want, (float(xi), gi, want)


def test_e4m3_encode_matches_torch_float8_in_range():
    x = _e4m3_probe_points()
    x = x[x <= 448]
    ref = torch.from_numpy(x.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.e4m3_encode_array(x), ref)


# -------------------------------------------------------------- E2M1

def test_e2m1_tie_table():
    table = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6,
             0.0: 0, 0.5: 1, 1.0: 2, 1.5: 3, 2.0: 4, 3.0: 5, 4.0: 6, 6.0: 7, 7.0: 7, 100.0: 7}
    for x, c in table.items():
        assert oracle.e2m1_encode(x) == c, x
        assert oracle.e2m1_encode(-x) == c | 8, -x


def test_e2m1_encode_brute_force_around_every_midpoint():
    mids = (E2M1[1:] + E2M1[:-1]) / 2
    pts = np.concatenate([E2M1, mids, np.linspace(0, 7, 7001)]).astype(np.float32)
    pts = np.unique(np.concatenate([pts, np.nextafter(pts, np.float32(np.inf)),
                                    np.nextafter(pts, np.float32(0))]))
    pts = np.concatenate([pts, -pts])
    got = oracle.e2m1_encode_array(pts)
    for x, g in zip(pts, got):
        sign = 8 if np.signbit(x) else 0
        want = 7 if abs(x) >= 6 else _nearest_even(abs(float(x)), E2M1)
        assert g == (sign | want), (float(x), g)


# -------------------------------------------------------------- quantiser

def test_hand_worked_example():
    with open(os.path.join(GOLDEN, "nvfp4_hand_example.json")) as f:
        ex = json.load(f)
    x = np.array(ex["x"], dtype=np.float32)
    bits = torch.from_numpy(x).to(torch.bfloat16)
    assert torch.equal(bits.float(), torch.from_numpy(x)), "fixture values must be bf16-exact"
    codes, scales, g = oracle.nvfp4_quantize(bits, ex["rows"], ex["cols"])
    assert g == np.float32(ex["expected_global_scale"])
    np.testing.assert_array_equal(scales, np.array(ex["expected_scales"], np.uint8))
    want = np.array([[int(h, 16) for h in row] for row in ex["expected_codes_hex"]], np.uint8)
    np.testing.assert_array_equal(codes, want)


def test_zero_tensor():
    x = torch.zeros((3, 64), dtype=torch.bfloat16)
    codes, scales, g = oracle.nvfp4_quantize(x, 3, 64)
    assert g == 0 and not codes.any() and not scales.any()


def _decode(codes, scales, g, rows, cols):
    lo = codes & 0xF
    hi = codes >> 4
    c = np.stack([lo, hi], axis=-1).reshape(rows, cols)
    mag = E2M1[c & 7] * np.where(c & 8, -1.0, 1.0)
    s = np.array([oracle.e4m3_value(int(v)) for v in scales.ravel()]).reshape(scales.shape)
    return mag * np.repeat(s, 16, axis=1) * float(g), c


def test_amax_block_and_dequantisation_bound():
    rows, cols = 64, 128
    q, _, _ = make_qkv(1, 1, 1, rows, 1, cols, seed=42)
    x = q.reshape(rows, cols)
    codes, scales, g = oracle.nvfp4_quantize(x, rows, cols)
    xf = x.double().numpy()
    amax = np.abs(xf).max()
    assert g == np.float32(np.float32(amax) / np.float32(2688.0))
    r, cidx = np.unravel_index(np.argmax(np.abs(xf)), xf.shape)
    assert scales[r, cidx // 16] == 0x7E
    deq, c = _decode(codes, scales, g, rows, cols)
    assert (c[r, cidx] & 7) == 7
    # every element lies within half an E2M1 step of its reconstruction; the
    # widest step is 2 (between 4 and 6), so |x - deq| <= t, plus fp32 slack
    t = np.repeat(np.array([oracle.e4m3_value(int(v)) for v in scales.ravel()])
                  .reshape(scales.shape), 16, axis=1) * float(g)
    assert np.all(np.abs(xf - deq) <= t * (1 + 1e-6) + 1e-30)
    # block amax elements map to a top code (6 or 4 after a downward E4M3 rounding)
    blk = np.abs(xf).reshape(rows, cols // 16, 16)
    top = c.reshape(rows, cols // 16, 16)[np.arange(rows)[:, None], np.arange(cols // 16)[None],
                                          blk.argmax(-1)] & 7
    assert np.all(top >= 6)


def test_block_of_equal_values():
    x = torch.full((2, 32), -1.5, dtype=torch.bfloat16)
    codes, scales, g = oracle.nvfp4_quantize(x, 2, 32)
    assert (scales == 0x7E).all()
    assert (codes == 0xFF).all()


def test_planted_mistake_is_caught():
    """Swapping the nibble order breaks the hand example: the packing rule is
    pinned."""
    with open(os.path.join(GOLDEN, "nvfp4_hand_example.json")) as f:
        ex = json.load(f)
    x = torch.from_numpy(np.array(ex["x"], np.float32)).to(torch.bfloat16)
    codes, _, _ = oracle.nvfp4_quantize(x, 2, 32)
    swapped = ((codes & 0xF) << 4) | (codes >> 4)
    want = np.array([[int(h, 16) for h in row] for row in ex["expected_codes_hex"]], np.uint8)
    assert not np.array_equal(swapped, want)


# ------------------------------------------------- given global scale (fused)

def test_given_scale_hand_worked_blocks():
    """g = 0.5, worked by hand from the format definitions.
    Block 0: amax 6 -> s = E4M3((6/6)/0.5) = E4M3(2) = 0x40 (exponent 1 + bias 7,
    mantissa 0); t = 2 * 0.5 = 1, so the codes are E2M1(x) itself:
    1 -> 2, -2 -> 0xC, 3 -> 5, 0.25 -> 0 (tie between 0 and 0.5: even code),
    0.5 -> 1, 6 -> 7, -6 -> 0xF, 1.5 -> 3.
    Block 1: amax 0.75 -> (0.75/6)/0.5 = 0.25 = E4M3 0x28 (exponent -2 + 7);
    t = 0.125: 0.75 -> 6 -> 7, 0.375 -> 3 -> 5, -0.1875 -> -1.5 -> 0xB."""
    x = np.zeros((1, 32), np.float32)
    x[0, :8] = [1.0, -2.0, 3.0, 0.25, 0.5, 6.0, -6.0, 1.5]
    x[0, 16:19] = [0.75, 0.375, -0.1875]
    bits = torch.from_numpy(x).to(torch.bfloat16)
    codes, scales = oracle.nvfp4_quantize_with_scale(bits, 1, 32, 0.5)
    np.testing.assert_array_equal(scales, np.array([[0x40, 0x28]], np.uint8))
    want = [0xC2, 0x05, 0x71, 0x3F, 0, 0, 0, 0, 0x57, 0x0B, 0, 0, 0, 0, 0, 0]
    np.testing.assert_array_equal(codes, np.array([want], np.uint8))


def test_given_scale_saturation_and_zero():
    x = torch.full((1, 16), 3.0, dtype=torch.bfloat16)
    # (3/6)/g >= 448 saturates the block scale to 0x7E = 448; t = 448 g and
    # every x / t = 3 / (448 * 2^-12) ... = 27.4 saturates E2M1 to 6 (code 7)
    codes, scales = oracle.nvfp4_quantize_with_scale(x, 1, 16, 2.0 ** -12)
    assert (scales == 0x7E).all() and (codes == 0x77).all()
    codes, scales = oracle.nvfp4_quantize_with_scale(x, 1, 16, 0.0)
    assert not scales.any() and not codes.any()


def test_given_scale_with_the_tensor_scale_is_the_tensor_recipe():
    rows, cols = 16, 64
    q, _, _ = make_qkv(1, 1, 1, rows, 1, cols, seed=7)
    x = q.reshape(rows, cols)
    codes, scales, g = oracle.nvfp4_quantize(x, rows, cols)
    amax = np.float32(np.abs(x.float().numpy()).max())
    assert g == np.float32(amax / np.float32(2688.0))
    c2, s2 = oracle.nvfp4_quantize_with_scale(x, rows, cols, g)
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(s2, scales)
