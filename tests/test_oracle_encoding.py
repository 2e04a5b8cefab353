"""Pins for the oracle's number encoding, chunking and RoPE (CPU only)."""
import math
import os

import numpy as np
import pytest
import torch

from oracle import msa_oracle as O
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- bf16 (R16)

def test_bf16_roundtrip_exact_values():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, size=20000, dtype=np.uint16)
    x = O.bf16_bits_to_f64(bits)
    fin = np.isfinite(x)
    back = O.f64_to_bf16_bits(x[fin])
    # canonical zero sign aside, every finite bf16 value encodes back to its own bits
    same = (back == bits[fin]) | ((x[fin] == 0) & ((back & 0x7FFF) == 0))
    assert same.all()


def test_bf16_known_values():
    assert O.bf16_bits_to_f64(np.array([0x3F80]))[0] == 1.0
    assert O.bf16_bits_to_f64(np.array([0xC000]))[0] == -2.0
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties go to the even mantissa (1.0)
    assert O.round_to_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    # 1 + 3*2^-8 lies halfway between 1+2^-7 (odd) and 1+2^-6 (even)
    assert O.round_to_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
    # just above a tie rounds up
    assert O.round_to_bf16(np.array([1 + 2.0 ** -8 + 2.0 ** -30]))[0] == 1 + 2.0 ** -7
    assert O.round_to_bf16(np.array([1e39]))[0] == np.inf
    assert O.round_to_bf16(np.array([-0.0]))[0] == 0.0


def test_bf16_matches_torch_on_float32_values():
    # For values that are exactly float32, torch's float32 -> bfloat16 cast is a single
    # round-to-nearest-even, so it must agree with the float64 route.
    rng = np.random.default_rng(2)
    x32 = (rng.standard_normal(50000) * np.exp(rng.uniform(-30, 30, 50000))).astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_to_bf16(x32.astype(np.float64))
    assert np.array_equal(ref, got)


def test_bf16_single_rounding_differs_from_double_rounding():
    # 1 + 2^-8 + 2^-40 : float64 -> bf16 directly rounds up; via float32 the tail is lost
    # and the tie then rounds to even (down).  The oracle must round once.
    x = 1 + 2.0 ** -8 + 2.0 ** -40
    assert O.round_to_bf16(np.array([x]))[0] == 1 + 2.0 ** -7


# ----------------------------------------------------------------------------- chunking (R4)

def test_chunk_count_worked_example():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "chunking_worked_example.txt"))
            if l.strip() and not l.startswith("#")]
    for tokens, chunk, chunks in rows:
        assert O.chunk_counts([int(tokens)], int(chunk))[0] == int(chunks)


def test_chunk_offsets_edges():
    assert list(O.chunk_counts([1, 63, 64, 65, 128, 129], 64)) == [1, 1, 1, 2, 2, 3]
    off = O.chunk_offsets([180, 1, 64], 64)
    assert list(off) == [0, 3, 4, 5]
    with pytest.raises(ValueError):
        O.chunk_offsets([10, 0], 64)


# ----------------------------------------------------------------------------- RoPE (R2)

def test_rope_matches_complex_form():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((7, 3, 16))
    pos = np.array([0, 1, 2, 5, 100, 4000, 8191])
    got = O.rope_rotate(x, pos, 1e6)
    for t in range(7):
        for h in range(3):
            ref = brute.rope_pairs(x[t, h], int(pos[t]), 1e6)
            np.testing.assert_allclose(got[t, h], ref, rtol=0, atol=1e-12)


def test_rope_closed_forms():
    # theta_0 = 1: pair (0, D/2) turns by exactly `pos` radians; theta_1 = base^(-2/D).
    d = 32
    th = O.rope_inv_freq(d, 1e6)
    assert th[0] == 1.0
    assert math.isclose(th[1], 10 ** (-0.375), rel_tol=1e-15)
    e0 = np.zeros((1, 1, d))
    e0[0, 0, 0] = 1.0
    r = O.rope_rotate(e0, np.array([2]), 1e6)[0, 0]
    assert math.isclose(r[0], math.cos(2.0), abs_tol=1e-15)
    assert math.isclose(r[d // 2], math.sin(2.0), abs_tol=1e-15)
    # position 0 is the identity, bit for bit
    x = np.random.default_rng(4).standard_normal((3, 2, d))
    assert np.array_equal(O.rope_rotate(x, np.zeros(3), 1e6), x)


def test_rope_norm_and_relative_position():
    rng = np.random.default_rng(5)
    d = 64
    x = rng.standard_normal((1, 1, d))
    y = rng.standard_normal((1, 1, d))
    for p in (0, 3, 77, 5000):
        rp = O.rope_rotate(x, np.array([p]), 1e4)
        assert math.isclose(np.linalg.norm(rp), np.linalg.norm(x), rel_tol=1e-13)
    # <R_p x, R_q y> depends only on q - p
    base_ip = None
    for p in (0, 10, 1234):
        ip = float(np.sum(O.rope_rotate(x, np.array([p]), 1e4) * O.rope_rotate(y, np.array([p + 7]), 1e4)))
        base_ip = ip if base_ip is None else base_ip
        assert math.isclose(ip, base_ip, rel_tol=1e-10, abs_tol=1e-10)
