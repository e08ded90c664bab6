"""Pins for the oracle's Philox4x32-10 and dropout mask.

* The generator is compared with an independent implementation: the
  Philox4x32-10 engine in PyTorch's ATen headers, compiled here into a small
  host program (its counter = (offset lo, offset hi, subsequence lo,
  subsequence hi), key = (seed lo, seed hi), four successive calls give the
  four output words).
* The key-bump constants are the closed forms floor(2^32 (sqrt 5 - 1)/2) and
  floor(2^32 (sqrt 3 - 1)) from the Philox paper.
* The keep mask keeps a fraction 1 - p within binomial error and differs
  between heads, batch entries and seeds.
"""

import math
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
import torch

from oracle import philox

CASES = [
    # (seed, subsequence, offset)
    (0x0123456789ABCDEF, 0, 0),
    (0, 0, 0),
    (0xFFFFFFFFFFFFFFFF, 0xFFFFFFFFFFFFFFFF, 0xFFFFFFFFFFFFFFFE),
    (0x243F6A8885A308D3, (7 << 32) | 3, (1234 << 32) | 77),
    (0xA4093822299F31D0, 5, 1 << 40),
    (1, (15 << 32) | 11, (4095 << 32) | 511),
]

PROG = r"""
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>
#include <cstdint>
#include <cstdlib>
int main(int argc, char** argv) {
  for (int a = 1; a + 2 < argc; a += 3) {
    uint64_t seed = strtoull(argv[a], 0, 0), sub = strtoull(argv[a+1], 0, 0), off = strtoull(argv[a+2], 0, 0);
    at::Philox4_32 e(seed, sub, off);
    for (int i = 0; i < 4; i++) printf("%u ", e());
    printf("\n");
  }
  return 0;
}
"""


def _torch_philox_outputs(cases):
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(inc, "ATen/core/PhiloxRNGEngine.h")):
        pytest.skip("g++ or the ATen Philox header is not available")
    with tempfile.TemporaryDirectory() as tmp:
        src, exe = os.path.join(tmp, "p.cpp"), os.path.join(tmp, "p")
        with open(src, "w") as f:
            f.write(PROG)
        subprocess.run([gxx, "-std=c++17", "-O1", "-I", inc, src, "-o", exe], check=True,
                       capture_output=True)
        args = [str(x) for c in cases for x in c]
        out = subprocess.run([exe] + args, check=True, capture_output=True, text=True).stdout
    return np.array([[int(w) for w in line.split()] for line in out.strip().splitlines()],
                    dtype=np.uint64)


def test_matches_aten_philox_engine():
    ref = _torch_philox_outputs(CASES)
    ctr = [[off & 0xFFFFFFFF, off >> 32, sub & 0xFFFFFFFF, sub >> 32] for _, sub, off in CASES]
    keys = [[s & 0xFFFFFFFF, s >> 32] for s, _, _ in CASES]
    got = philox.philox4x32_10(np.array(ctr, dtype=np.uint64), np.array(keys, dtype=np.uint64))
    np.testing.assert_array_equal(got.astype(np.uint64), ref)


def test_keep_mask_uses_word_j_mod_4_of_counter():
    seed, b, h, i = 0x1122334455667788, 3, 5, 77
    rows, cols = np.array([i]), np.arange(16)
    m = philox.keep_mask(seed, b, h, rows, cols, 0.5)
    ref = _torch_philox_outputs([(seed, (b << 32) | h, (i << 32) | (j >> 2)) for j in range(0, 16, 4)])
    words = ref.reshape(-1)  # column j -> word j&3 of counter j>>2
    np.testing.assert_array_equal(m[0], words >= philox.dropout_threshold(0.5))


def test_weyl_constants_closed_form():
    w0 = (math.isqrt(5 << 64) - (1 << 32)) // 2
    w1 = math.isqrt(3 << 64) - (1 << 32)
    assert philox.PHILOX_W0 == w0
    assert philox.PHILOX_W1 == w1


def test_threshold_and_scale():
    assert philox.dropout_threshold(0.0) == 0
    assert philox.dropout_threshold(0.5) == 1 << 31
    p32 = float(np.float32(0.1))
    assert philox.dropout_threshold(0.1) == math.floor(p32 * 2 ** 32)
    # Literals, worked by hand: fp32(0.1) = 13421773 * 2^-27, so
    # T = 13421773 * 2^5 = 429496736 exactly, and the keep scale
    # 1 / (1 - p) = 2^27 / 120795955 = 1.11111111...4 rounds to the fp32 value
    # 1.1111111640930176 (= 9320676 * 2^-23).
    assert p32 == 13421773 * 2.0 ** -27
    assert philox.dropout_threshold(0.1) == 429496736
    assert philox.dropout_scale(0.1) == 1.1111111640930176
    assert philox.dropout_scale(0.1) == 9320676 * 2.0 ** -23
    assert philox.dropout_scale(0.5) == 2.0
    assert philox.dropout_scale(0.25) == 1.3333333730697632  # 11184811 * 2^-23
    assert philox.dropout_scale(0.0) == 1.0
    with pytest.raises(ValueError):
        philox.dropout_threshold(1.0)


@pytest.mark.parametrize("p", [0.1, 0.5])
def test_keep_fraction_is_binomial(p):
    m = philox.keep_mask(0x0123456789ABCDEF, 2, 7, np.arange(512), np.arange(512), p)
    n = m.size
    sigma = math.sqrt(n * p * (1 - p))
    assert abs(m.sum() - n * (1 - p)) <= 6 * sigma


def test_masks_differ_between_heads_batches_and_seeds():
    rows, cols = np.arange(64), np.arange(64)
    base = philox.keep_mask(1, 0, 0, rows, cols, 0.5)
    for other in (philox.keep_mask(1, 0, 1, rows, cols, 0.5),
                  philox.keep_mask(1, 1, 0, rows, cols, 0.5),
                  philox.keep_mask(2, 0, 0, rows, cols, 0.5)):
        assert 0.3 < np.mean(base != other) < 0.7


def test_word_equal_to_threshold_is_kept():
    # Find an element whose Philox word w (from the ATen engine) is exactly an
    # fp32 multiple of 2^-32, set p = w / 2^32 so T = w, and check it is kept
    # (keep iff word >= T) while a word of w - 1 would not be.
    seed, b, h = 0x5151515151515151, 1, 2
    cases = [(seed, (b << 32) | h, (i << 32) | jq) for i in range(16) for jq in range(16)]
    words = _torch_philox_outputs(cases)
    for (s, sub, off), w4 in zip(cases, words):
        for t, w in enumerate(w4):
            w = int(w)
            if w >= (1 << 31) and (w & 0xFF) == 0:
                p = w / 2.0 ** 32
                assert float(np.float32(p)) == p and philox.dropout_threshold(p) == w
                i, j = off >> 32, 4 * (off & 0xFFFFFFFF) + t
                m = philox.keep_mask(seed, b, h, np.array([i]), np.arange(j + 1), p)
                assert m[0, j]
                p_above = (w + 256) / 2.0 ** 32
                m2 = philox.keep_mask(seed, b, h, np.array([i]), np.arange(j + 1), p_above)
                assert not m2[0, j]
                return
    pytest.fail("no suitable word found")
