"""The storage rounding of the expert outputs O (fp16 of v * 2^-8 between the
down GEMM and the combine, whose sum is rounded once more to bf16).

With a single contribution per output row the combine's bf16 rounding acts on
the stored fp16 value itself, so O is rounded to odd: for a binary format with
at least two more significand bits than the final one, round-to-odd followed by
round-to-nearest-even gives the same result as one round-to-nearest-even of the
exact value (fp16 keeps 11 significand bits, bf16 8). This pins that property
on the value range where the scaled outputs are normal fp16 numbers, and that
plain nearest rounding twice would not have it. (Independent of the GPU code:
both roundings are written out here from their definitions.)"""
import numpy as np
import torch

SCALE = 2.0 ** -8


def bf16_rne(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.asarray(a, np.float32)).to(torch.bfloat16).float().numpy()


def fp16_rne(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, np.float32).astype(np.float16).astype(np.float32)


def fp16_round_to_odd(a: np.ndarray) -> np.ndarray:
    """Truncate toward zero to fp16, then take the neighbour with an odd last
    significand bit when the truncation was inexact."""
    a = np.asarray(a, np.float32)
    h = a.astype(np.float16)
    bits = h.view(np.uint16).copy()
    away = np.abs(h.astype(np.float32)) > np.abs(a)   # nearest rounding went away from zero
    bits[away] -= 1
    inexact = bits.view(np.float16).astype(np.float32) != a
    bits[inexact] |= 1
    return bits.view(np.float16).astype(np.float32)


def sample_values(n: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    # |v| in [2^-6, 2^23]: v * 2^-8 is a normal fp16 number
    e = rng.integers(-6, 23, size=n)
    m = rng.random(n, dtype=np.float64) + 1.0
    v = (np.where(rng.random(n) < 0.5, -1.0, 1.0) * m * np.exp2(e)).astype(np.float32)
    # plus values near bf16 rounding midpoints, where double rounding bites
    b = bf16_rne(v[: n // 2])
    ulp = np.exp2(np.floor(np.log2(np.abs(b))) - 7).astype(np.float32)
    near = b + np.float32(0.5) * ulp * np.sign(b) + (rng.integers(-3, 4, size=b.shape) * ulp / np.float32(4096)).astype(np.float32)
    return np.concatenate([v, near.astype(np.float32)])


def test_round_to_odd_then_nearest_equals_one_rounding():
    v = sample_values(400_000, seed=1)
    direct = bf16_rne(v)
    stored = fp16_round_to_odd(v * np.float32(SCALE)) / np.float32(SCALE)
    assert np.array_equal(bf16_rne(stored), direct)


def test_nearest_twice_can_differ():
    v = sample_values(400_000, seed=2)
    twice = bf16_rne(fp16_rne(v * np.float32(SCALE)) / np.float32(SCALE))
    assert np.count_nonzero(twice != bf16_rne(v)) > 0


def test_round_to_odd_definition_on_small_cases():
    # exact values stay; an inexact value lands on the odd neighbour of its truncation
    assert fp16_round_to_odd(np.array([1.0, -2.0, 0.5], np.float32)).tolist() == [1.0, -2.0, 0.5]
    one_ulp = 2.0 ** -10
    x = np.array([1.0 + 0.25 * one_ulp, 1.0 + 1.5 * one_ulp, -(1.0 + 0.75 * one_ulp)], np.float32)
    assert fp16_round_to_odd(x).tolist() == [1.0 + one_ulp, 1.0 + one_ulp, -(1.0 + one_ulp)]
