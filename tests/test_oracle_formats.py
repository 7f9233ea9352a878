"""Pins of the oracle's number formats against library casts and the OCP spec."""
import numpy as np
import pytest
import torch

from conftest import golden
from oracle import bf16_round, e4m3_decode, e4m3_encode, e4m3_values, E4M3_MAX


def _torch_bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def test_bf16_matches_torch_on_every_bf16_neighbourhood():
    # every bf16 bit pattern (finite), its midpoints with the next one, and +-1 ulp around them
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    v = (bits << 16).view(np.float32)
    v = v[np.isfinite(v)]
    nxt = np.nextafter(v, np.float32(np.inf))
    up = ((bits[: len(v)] + 1) << 16).view(np.float32)
    ok = np.isfinite(up)
    mid = (v[ok].astype(np.float64) + up[ok].astype(np.float64)) / 2
    mid32 = mid.astype(np.float32)
    sel = mid32.astype(np.float64) == mid           # representable midpoints: exact ties
    cases = np.concatenate([v, nxt, mid32, np.nextafter(mid32, np.float32(0)),
                            np.nextafter(mid32, np.float32(np.inf)), -v, -mid32])
    cases = cases[np.isfinite(cases) & (np.abs(cases) < 3.3e38)]
    ours = bf16_round(cases)
    ref = _torch_bf16(cases).astype(np.float64)
    assert sel.sum() > 60000
    np.testing.assert_array_equal(ours, ref)


def test_bf16_random_fp32():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) < 3.3e38)]
    np.testing.assert_array_equal(bf16_round(v), _torch_bf16(v).astype(np.float64))


def test_e4m3_ocp_points():
    g = golden("e4m3fn_ocp_points.json")
    for p in g["points"]:
        assert e4m3_decode(p["code"]) == p["value"]
        assert int(e4m3_encode(p["value"])) == p["code"]
    for c in g["nan_codes"]:
        assert np.isnan(e4m3_decode(c))
    vals = e4m3_values()
    assert len(vals) == g["finite_nonnegative_codes"]
    assert np.all(np.diff(vals) > 0) and vals[-1] == E4M3_MAX


def test_e4m3_matches_torch_below_saturation():
    vals = e4m3_values()
    mids = (vals[:-1] + vals[1:]) / 2                        # exact ties in fp32
    m32 = mids.astype(np.float32)
    assert np.all(m32.astype(np.float64) == mids)
    grid = np.concatenate([vals.astype(np.float32), m32,
                           np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(np.inf))])
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    bf = (bits << 16).view(np.float32)                       # every bf16 pattern
    rng = np.random.default_rng(1)
    rnd = rng.integers(0, 0x43E00001, size=3_000_000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    v = np.concatenate([grid, bf, rnd])
    v = v[np.isfinite(v) & (np.abs(v) <= E4M3_MAX)]
    v = np.concatenate([v, -v])
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = e4m3_encode(v)
    # torch keeps the sign of a value that rounds to zero; the codec only encodes
    # non-negative scales, so compare magnitudes for zero results
    zero = (ref & 0x7F) == 0
    np.testing.assert_array_equal(ours[~zero], ref[~zero])
    np.testing.assert_array_equal(ours[zero] & 0x7F, 0)


def test_e4m3_saturates():
    big = np.array([448.0, 448.0001, 463.99, 464.0, 480.0, 672.0, 1e4, 3e38], np.float32)
    assert np.all(e4m3_encode(big) == 0x7E)
    assert np.all(e4m3_encode(-big) == 0xFE)


def test_e4m3_roundtrip_of_representable_values():
    codes = np.arange(0x7F)
    np.testing.assert_array_equal(e4m3_encode(e4m3_decode(codes)), codes)
