"""Shared check for the oracles' bf16 bit-pattern reading.

Each oracle module converts uint16 arrays as bf16 bit patterns (the upper half
of an IEEE binary32) to float64.  The check compares that conversion, for all
65,536 patterns, with torch's own bfloat16 -> float64 conversion: the same value
bit for bit (signed zeros, subnormals, infinities), NaN exactly where torch gives
NaN.  A shift by the wrong amount, an fp16 reading or a sign slip fails it."""
from __future__ import annotations

import numpy as np
import torch


def check_bf16_bits(to_f64):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = np.asarray(to_f64(bits))
    assert got.dtype == np.float64 and got.shape == bits.shape
    want = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), "NaN patterns differ"
    assert np.array_equal(got[~nan].view(np.uint64), want[~nan].view(np.uint64)), "values differ"
    # a few patterns by hand: 1.0, -2.0, the smallest subnormal, the largest finite
    hand = {0x3F80: 1.0, 0xC000: -2.0, 0x0001: 2.0 ** -133, 0x7F7F: (2 - 2 ** -7) * 2.0 ** 127}
    for b, v in hand.items():
        assert to_f64(np.array([b], dtype=np.uint16))[0] == v, hex(b)
