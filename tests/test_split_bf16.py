"""The arithmetic behind the fp32 projections at embed_dim 128 (split-bf16
matrix-core products, CPU only): every fp32 value away from the ends of the
exponent range is the exact sum of three bf16 values obtained by rounding to
nearest even three times, and the six part products the kernel keeps differ
from the exact product by less than an fp32 rounding. bf16 rounding here is
the input generators' (itself pinned against torch in test_oracle_bf16.py)."""
import numpy as np

from graph_sparse_head_amd import synth


def _bf16(x):
    return synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(np.asarray(x, np.float32)))


def _split3(x):
    x = np.asarray(x, np.float32)
    hi = _bf16(x)
    r1 = (x - hi).astype(np.float32)       # exact in fp32
    mid = _bf16(r1)
    r2 = (r1 - mid).astype(np.float32)     # exact in fp32
    lo = _bf16(r2)
    return hi, mid, lo


def _values(n, seed):
    g = np.random.default_rng(seed)
    mant = g.uniform(1.0, 2.0, n)
    exp = g.integers(-100, 100, n)
    sign = g.choice([-1.0, 1.0], n)
    return (sign * mant * np.exp2(exp)).astype(np.float32)


def test_three_bf16_parts_sum_to_the_fp32_value_exactly():
    x = np.concatenate([_values(200_000, 1), np.float32([1.0, -1.0, 3.0, 1 / 3, np.pi, 0.0]),
                        np.nextafter(np.float32(1.0), np.float32(2.0), dtype=np.float32)[None]])
    hi, mid, lo = _split3(x)
    assert (hi.astype(np.float64) + mid + lo == x.astype(np.float64)).all()
    # and each part is a bf16 value (its low 16 bits are zero)
    for part in (hi, mid, lo):
        assert (part.view(np.uint32) & 0xFFFF == 0).all()


def test_six_part_products_are_within_an_fp32_rounding():
    x, w = _values(100_000, 2), _values(100_000, 3)
    xs, ws = _split3(x), _split3(w)
    keep = [(0, 0), (0, 1), (1, 0), (0, 2), (2, 0), (1, 1)]
    approx = sum(xs[i].astype(np.float64) * ws[j] for i, j in keep)
    exact = x.astype(np.float64) * w.astype(np.float64)
    rel = np.abs(approx - exact) / np.abs(exact)
    assert rel.max() < 2.0 ** -22
    # dropping a kept product (mid x mid) is visibly worse: the pin has teeth
    worse = approx - xs[1].astype(np.float64) * ws[1]
    assert (np.abs(worse - exact) / np.abs(exact)).max() > 2.0 ** -20
