"""The two premises of the step kernel's key-norm bound on the reference, checked on the CPU
with the kernel's own precisions (no GPU involved):

* Cauchy-Schwarz with rounding: a score accumulated in fp32 from bf16 products never exceeds
  |q| |k| (each norm from an fp32 sum of squares and an fp32 square root) times the margin
  1 + 2^-9 on each norm, including the tight case of a key parallel to its query;
* the scalar compare: for a bound k >= 0 and any threshold T (infinities included), the bit
  patterns compared as signed 32-bit integers never pass a tile the floats would not, and
  order exactly like the floats for every T but -0 (which (32 + m) / (|q| |c|) cannot take:
  a sum of finite values is never -0, and |q| |c| >= 0); the NaN pattern 0x7fffffff that
  stands for "no bound" exceeds every threshold's pattern."""

import numpy as np
import pytest

MARGIN = np.float32(1.0 + 2.0 ** -9)


def to_bf16(x):
    """Round float32 to the nearest bfloat16 (ties to even), kept as float32."""
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16 << 16
    return b.astype(np.uint32).view(np.float32)


def fp32_dot(a, b):
    """Products and sums rounded to fp32 one at a time (no wider accumulator)."""
    acc = np.float32(0.0)
    for x, y in zip(a, b):
        acc = np.float32(acc + np.float32(x * y))
    return acc


def fp32_norm(a):
    return np.float32(np.sqrt(fp32_dot(a, a))) * MARGIN


@pytest.mark.parametrize("d", [64, 128])
def test_fp32_scores_stay_within_the_margined_norm_product(d):
    rng = np.random.default_rng(d)
    worst = 0.0
    for trial in range(400):
        scale = np.float32(10.0 ** rng.uniform(-3, 3))
        q = to_bf16(rng.standard_normal(d).astype(np.float32) * scale)
        if trial % 4 == 0:
            k = q.copy()                                   # parallel: Cauchy-Schwarz is tight
        elif trial % 4 == 1:
            k = to_bf16(q * np.float32(rng.uniform(0.1, 10.0)))
        else:
            k = to_bf16(rng.standard_normal(d).astype(np.float32) * np.float32(10.0 ** rng.uniform(-3, 3)))
        x = fp32_dot(q, k)
        bound = np.float32(fp32_norm(q) * fp32_norm(k))
        assert abs(float(x)) <= float(bound)
        worst = max(worst, abs(float(x)) / float(bound))
    # the tight cases come close to the bound: the margin is not hiding a loose check
    assert worst > 0.99


def test_signed_pattern_compare_orders_like_the_floats():
    rng = np.random.default_rng(5)
    kn = np.concatenate([np.abs(rng.standard_normal(2000)).astype(np.float32) * 100,
                         np.float32([0.0, 1e-38, 3.4e38, np.inf])])
    t = np.concatenate([rng.standard_normal(2000).astype(np.float32) * 100,
                        np.float32([0.0, -0.0, -1e30, 1e30, np.inf, -np.inf])])
    kb = kn.view(np.int32)
    tb = t.view(np.int32)
    not_minus_zero = ~((t == 0) & np.signbit(t))
    for a, ab in zip(kn, kb):
        bits, floats = ab <= tb, a <= t
        assert not (bits & ~floats).any()                      # never passes wrongly
        assert np.array_equal(bits[not_minus_zero], floats[not_minus_zero])
    nan_bits = np.int32(0x7FFFFFFF)
    assert (nan_bits > tb).all()
