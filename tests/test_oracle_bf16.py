"""Pins of the oracle's bf16 decode and round-to-nearest-even encode.

The decode is checked against torch's own bf16 -> float64 conversion over all
65,536 bit patterns; the encode against torch's float32 -> bf16 conversion
(a library round-to-nearest-even) and, for doubles that are not float32
values, against a brute-force nearest-neighbour search.
"""
import numpy as np
import torch

import oracle


def _torch_decode(bits):
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)
    return t.double().numpy()


def test_decode_all_patterns_match_library():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.bf16_decode(bits)
    want = _torch_decode(bits)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # the scalar C entry point agrees with the vectorised decode
    sample = bits[::97]
    c = oracle.bf16_to_double(sample)
    assert np.array_equal(np.isnan(c), np.isnan(want[::97]))
    m = ~np.isnan(c)
    assert np.array_equal(c[m], want[::97][m])


def test_encode_matches_library_rne_on_float32_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(4000).astype(np.float32),
        (rng.standard_normal(1000) * 1e-39).astype(np.float32),   # subnormal
        (rng.standard_normal(1000) * 3e38).astype(np.float32),    # near overflow
        np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf], dtype=np.float32),
    ])
    got = oracle.double_to_bf16(x.astype(np.float64))
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_encode_ties_go_to_even_and_is_nearest():
    # exact midpoints between consecutive bf16 values
    rng = np.random.default_rng(1)
    lo_bits = rng.integers(0x0001, 0x7F7F, size=2000).astype(np.uint16)
    lo = oracle.bf16_decode(lo_bits)
    hi = oracle.bf16_decode(lo_bits + 1)
    mid = (lo + hi) / 2
    got = oracle.double_to_bf16(mid)
    want = np.where(lo_bits % 2 == 0, lo_bits, lo_bits + 1).astype(np.uint16)
    assert np.array_equal(got, want)
    # a hair above / below the midpoint goes to the nearer neighbour; these
    # doubles are not float32 values, so a float32 detour would double-round
    above = oracle.double_to_bf16(mid + (hi - lo) * 2.0 ** -30)
    below = oracle.double_to_bf16(mid - (hi - lo) * 2.0 ** -30)
    assert np.array_equal(above, lo_bits + 1)
    assert np.array_equal(below, lo_bits)


def test_encode_is_nearest_by_brute_force():
    rng = np.random.default_rng(2)
    x = rng.standard_normal(3000) * np.exp(rng.uniform(-20, 20, 3000))
    got = oracle.double_to_bf16(x)
    allbits = np.arange(0, 0x7F80, dtype=np.uint16)      # finite non-negatives
    allv = oracle.bf16_decode(allbits)
    for xi, gi in zip(x, got):
        a = abs(xi)
        j = np.searchsorted(allv, a)
        cands = [k for k in (j - 1, j) if 0 <= k < allv.size]
        dist = [abs(allv[k] - a) for k in cands]
        best = min(dist)
        ok = [allbits[k] for k, dd in zip(cands, dist) if dd == best]
        mag = gi & 0x7FFF
        assert mag in ok
        assert (gi >> 15) == (1 if xi < 0 else 0)
