"""Pins of the oracle's number formats against the format definitions and
torch's own casts (library routines), exhaustively where possible."""
import numpy as np
import pytest
import torch

import oracle


def test_e4m3fn_known_codes():
    v = oracle.E4M3FN_VALUES
    assert v[0x00] == 0.0 and not np.signbit(v[0x00])
    assert v[0x80] == 0.0 and np.signbit(v[0x80])
    assert v[0x01] == 2.0 ** -9            # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9        # largest subnormal
    assert v[0x08] == 2.0 ** -6            # smallest normal
    assert v[0x38] == 1.0
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.sum(np.isnan(v)) == 2        # no infinities, two NaNs


def test_e4m3fn_decode_matches_torch_all_codes():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3fn_decode(np.arange(256, dtype=np.uint8))
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.all(both_nan | (ref == got))
    assert np.array_equal(np.signbit(ref[~both_nan]), np.signbit(got[~both_nan]))


def test_e4m3fn_encode_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.e4m3fn_decode(codes).astype(np.float32)
    assert np.array_equal(oracle.e4m3fn_encode(vals), codes)


def test_e4m3fn_encode_midpoints_go_to_even_code():
    pos = oracle.E4M3FN_VALUES[:127]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (pos[:-1] + pos[1:]) / 2)  # exact in f32
    got = oracle.e4m3fn_encode(mids)
    lo = np.arange(126)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got, want.astype(np.uint8))
    # a hair either side of every midpoint goes to the nearer neighbour
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(-np.inf))
    assert np.array_equal(oracle.e4m3fn_encode(up), (lo + 1).astype(np.uint8))
    assert np.array_equal(oracle.e4m3fn_encode(dn), lo.astype(np.uint8))


def test_e4m3fn_encode_saturates_and_keeps_sign():
    big = np.array([448.0, 449.0, 463.9, 464.0, 480.0, 1e4, 3e38], dtype=np.float32)
    assert np.all(oracle.e4m3fn_encode(big) == 0x7E)
    assert np.all(oracle.e4m3fn_encode(-big) == 0xFE)
    assert oracle.e4m3fn_encode(np.array([-1e-30], np.float32))[0] == 0x80


def test_e4m3fn_encode_matches_torch_cast_in_range():
    rng = np.random.default_rng(1)
    v = np.concatenate([rng.uniform(-448, 448, 200000), rng.normal(0, 1, 200000),
                        rng.normal(0, 1e-2, 100000)]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3fn_encode(v)
    # torch may flip the sign bit of a zero result; compare values, then signs of nonzeros
    rv, gv = oracle.e4m3fn_decode(ref), oracle.e4m3fn_decode(got)
    assert np.array_equal(rv, gv)


def test_bf16_decode_matches_torch():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_bits_to_f64(bits)
    nan = np.isnan(t)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], t[~nan])


def test_normwise_rel_err():
    assert oracle.normwise_rel_err(np.array([1.0, 2.0]), np.array([1.0, 2.0])) == 0.0
    assert oracle.normwise_rel_err(np.array([1.1, 2.0]), np.array([1.0, 2.0])) == pytest.approx(0.05)
