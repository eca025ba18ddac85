"""Pins of the oracle's number formats (CPU only).

`widen` turns bf16 bit patterns (the storage format of keys, values and queries on
the bf16 workloads) into their exact float64 values.  Every attention pin pushes its
inputs through it, so it is pinned here against things other than itself:

* hand-decoded bit patterns: sign, 8 exponent bits (bias 127), 7 fraction bits;
* torch's own bfloat16 -> float64 conversion of all 65 536 bit patterns (a library
  routine, bit-for-bit, NaN for NaN);
* float32 input: the exact value Python's float() gives each element.
"""
import math

import numpy as np
import torch

from oracle import widen

HAND = [
    (0x3F80, 1.0),
    (0xC040, -3.0),
    (0x4049, 3.140625),
    (0x0001, 2.0 ** -133),              # smallest subnormal: 2^-126 * 2^-7
    (0x007F, 127 * 2.0 ** -133),        # largest subnormal
    (0x0080, 2.0 ** -126),              # smallest normal
    (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127),   # largest finite
    (0x3F81, 1.0 + 2.0 ** -7),          # one ulp above 1
    (0xBF00, -0.5),
    (0x7F80, math.inf),
    (0xFF80, -math.inf),
]


def test_hand_patterns():
    bits = np.array([b for b, _ in HAND], dtype=np.uint16)
    got = widen(bits)
    assert got.dtype == np.float64
    for (b, v), g in zip(HAND, got.tolist()):
        assert g == v, f"0x{b:04X}: {g!r} != {v!r}"
    z = widen(np.array([0x0000, 0x8000], dtype=np.uint16))
    assert z.tolist() == [0.0, 0.0]
    assert not math.copysign(1.0, z[0]) < 0 and math.copysign(1.0, z[1]) < 0  # -0.0 keeps its sign
    assert np.isnan(widen(np.array([0x7FC0, 0xFFC1, 0x7F81], dtype=np.uint16))).all()


def test_every_pattern_matches_torch_bfloat16():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = widen(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint64), ref[~nan].view(np.uint64))  # signed zeros too


def test_float32_input_is_exact():
    r = np.random.default_rng(11)
    x = (r.standard_normal(1000) * np.exp(r.uniform(-60, 60, 1000))).astype(np.float32)
    x[:4] = [0.0, -0.0, np.float32(1e-45), np.float32(3.4e38)]
    got = widen(x)
    assert [float(v) for v in x] == got.tolist()
    assert math.copysign(1.0, got[1]) < 0
