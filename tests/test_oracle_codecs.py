"""Pins for the oracle's scalar codecs (E2M1, E4M3, E8M0, bf16) and its
stochastic rounding, against format definitions, library decodes and brute force."""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _grid():
    with open(os.path.join(GOLD, "e2m1_grid.json")) as f:
        return json.load(f)


def test_e2m1_decode_matches_grid():
    g = _grid()
    for c, v in zip(g["codes"], g["values"]):
        got = oracle.e2m1_decode(c)
        assert got == v and np.signbit(got) == np.signbit(v), (c, got, v)


def test_e4m3_decode_all_bytes_vs_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    for b in range(256):
        got = oracle.e4m3_decode(b)
        if np.isnan(ref[b]):
            assert np.isnan(got), b
        else:
            assert got == ref[b] and np.signbit(got) == np.signbit(ref[b]), (b, got, ref[b])
    assert oracle.e4m3_decode(0x7E) == 448.0


def test_e8m0_decode_all_bytes_vs_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).float().numpy()
    for b in range(256):
        got = oracle.e8m0_decode(b)
        if np.isnan(ref[b]):
            assert np.isnan(got)
        else:
            assert got == ref[b], (b, got, ref[b])


def test_e2m1_rne_hand_cases():
    g = _grid()["rne_cases"]
    for x, want in zip(g["inputs"], g["expected"]):
        assert oracle.e2m1_rne(np.float32(x)) == want, (x, want)


def _brute_nearest(vals, grid, even_mask):
    """Nearest grid magnitude to |v| with ties to the even entry, by exhaustive search."""
    a = np.abs(vals.astype(np.float64))[:, None]
    d = np.abs(a - grid[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    # among tied candidates prefer the even one
    pick_even = cand & even_mask[None, :]
    idx = np.where(pick_even.any(axis=1), pick_even.argmax(axis=1), cand.argmax(axis=1))
    return idx


def _probe_values(grid, n_random, lo, hi, seed):
    g = np.random.default_rng(seed)
    mids = (grid[1:] + grid[:-1]) / 2
    pts = np.concatenate([grid, mids]).astype(np.float32)
    near = [pts]
    for k in range(1, 4):
        near.append(np.nextafter(pts, np.float32(np.inf)))
        pts_dn = pts.copy()
        for _ in range(k):
            pts_dn = np.nextafter(pts_dn, np.float32(0))
        near.append(pts_dn)
    rnd = (g.uniform(lo, hi, n_random)).astype(np.float32)
    logu = np.exp(g.uniform(np.log(1e-12), np.log(hi * 4), n_random)).astype(np.float32)
    v = np.concatenate(near + [rnd, logu])
    return np.concatenate([v, -v])


def test_e2m1_rne_vs_brute_force():
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    vals = _probe_values(grid, 20000, 0.0, 8.0, 1)
    want = _brute_nearest(vals, grid, np.arange(8) % 2 == 0)
    for v, w in zip(vals, want):
        got = oracle.e2m1_rne(v)
        assert got & 7 == w and (got >> 3) == int(np.signbit(v)), (float(v), got, w)


def _e4m3_grid():
    return np.array([oracle.e4m3_decode(b) for b in range(0x7F)], dtype=np.float64)


def test_e4m3_rne_vs_brute_force_and_torch():
    grid = _e4m3_grid()
    vals = _probe_values(grid, 20000, 0.0, 480.0, 2)
    want = _brute_nearest(vals, grid, np.arange(0x7F) % 2 == 0)
    got = np.array([oracle.e4m3_rne_sat(v) for v in vals], dtype=np.uint8)
    assert np.array_equal(got & 0x7F, want.astype(np.uint8))
    assert np.array_equal(got >> 7, np.signbit(vals).astype(np.uint8))
    # library check (torch converts with nearest-even; it gives NaN from 464 up,
    # so only magnitudes below that are compared)
    m = np.abs(vals) < 464
    ref = torch.from_numpy(vals[m]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got[m], ref)


def test_e4m3_saturates():
    for v in [448.0, 463.9, 464.0, 480.0, 1e6, 3.0e38]:
        assert oracle.e4m3_rne_sat(np.float32(v)) == 0x7E
        assert oracle.e4m3_rne_sat(np.float32(-v)) == 0xFE
        assert oracle.e4m3_sr(np.float32(v), 0) == 0x7E


def test_bf16_rounding_vs_torch():
    g = np.random.default_rng(3)
    v = np.concatenate([g.standard_normal(5000) * 10.0 ** g.integers(-40, 38, 5000),
                        np.array([1e-45, 1e-40, 1.1754942e-38, 3.0e38])]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f64_to_bf16(v.astype(np.float64))
    assert np.array_equal(got, ref)
    v64 = g.standard_normal(20000) * 10.0 ** g.integers(-30, 30, 20000)
    assert np.array_equal(oracle.f64_to_bf16_fast(v64), oracle.f64_to_bf16(v64))


@pytest.mark.parametrize("y", [0.1, 0.3, 0.74, 1.2, 1.6, 2.2, 3.3, 4.9, 5.99, -0.6, -3.7])
def test_e2m1_sr_exact_expectation(y):
    """Over all 2^16 draws the mean of the rounded value equals y to within
    2^-16 of one grid step, and every result is one of the two neighbours."""
    y = np.float32(y)
    vals = np.array([oracle.e2m1_decode(oracle.e2m1_sr(y, u)) for u in range(65536)])
    a = abs(float(y))
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    lo = grid[grid <= a].max()
    hi = grid[grid > a].min()
    assert set(np.abs(vals)) <= {lo, hi}
    assert abs(vals.mean() - float(y)) <= (hi - lo) / 65536 + 1e-12


@pytest.mark.parametrize("y", [0.0013, 0.017, 0.6, 3.3, 47.0, 300.0, 447.0, -0.2])
def test_e4m3_sr_exact_expectation(y):
    y = np.float32(y)
    vals = np.array([oracle.e4m3_decode(oracle.e4m3_sr(y, u)) for u in range(65536)])
    grid = _e4m3_grid()
    a = abs(float(y))
    lo = grid[grid <= a].max()
    hi = grid[grid > a].min()
    assert set(np.abs(vals)) <= {lo, hi}
    assert abs(vals.mean() - float(y)) <= (hi - lo) / 65536 + 1e-12


def test_sr_on_grid_points_is_exact():
    for c in range(8):
        v = oracle.e2m1_decode(c)
        assert all(oracle.e2m1_sr(np.float32(v), u) == c for u in (0, 1, 12345, 65535))
    for b in range(0x7F):
        v = oracle.e4m3_decode(b)
        assert all(oracle.e4m3_sr(np.float32(v), u) == b for u in (0, 777, 65535))
