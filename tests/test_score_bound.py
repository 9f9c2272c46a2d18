"""The error bound behind the exact top-K of the scoring kernel.

The scoring kernel ranks chunks by s^ = scale q_s.k' + b' (hyper.ai HiLS
summary, 方法, surrogate-score equation) on bf16 MFMA: an fp32 operand x
enters as a two-term split t1 = bf16(x), t2 = bf16(x - t1), the products
t1 k1 + t1 k2 + t2 k1 are summed in fp32 and the t2 k2 term is dropped.
The kernel keeps every candidate whose approximate score lies within 2E of
the K-th, E = scale * kappa * ||q_s|| * max ||k'||, and recomputes those in
fp32, so the selection is exact as long as |approx - exact| <= E.  Its
kappa is 2^-14 for the fp32 accumulation plus 2^-16 (1 + 2^-7) for each
split operand and for the dropped term.  These tests check the
representation part of that claim against bf16 rounding (torch's
round-to-nearest-even conversion on the CPU): on random values, on values
constructed to maximise both rounding errors, and on whole dot products of
such values with equal signs, the worst case of Cauchy-Schwarz.
"""
import numpy as np
import torch

SPLIT_TERM = 2.0 ** -16 * (1 + 2.0 ** -7)


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def _split(x):
    x = np.asarray(x, np.float32)
    t1 = _bf16(x)
    r = (x - t1).astype(np.float32)  # exact: x and t1 agree in their leading bits
    t2 = _bf16(r)
    return t1.astype(np.float64), t2.astype(np.float64)


def _adversarial(n, rng):
    """fp32 values whose first bf16 rounding loses close to half a unit
    (the 16 dropped fraction bits just above one half) and whose residual's
    own rounding then loses up to half a unit (its 7 lowest bits random)."""
    e = rng.integers(-20, 20, n)
    m = (1 << 23) | (1 << 15) | (1 << 7) | rng.integers(0, 1 << 7, n)
    x = np.ldexp(m.astype(np.float64), e - 23)
    return (x * rng.choice([-1.0, 1.0], n)).astype(np.float32)


def test_two_term_split_within_2_pow_minus_16():
    rng = np.random.default_rng(5)
    for x in (rng.standard_normal(200000).astype(np.float32) * np.exp(rng.uniform(-8, 8, 200000)).astype(np.float32),
              _adversarial(200000, rng)):
        t1, t2 = _split(x)
        xd = x.astype(np.float64)
        ratio = np.abs(xd - t1 - t2) / np.abs(xd)
        assert ratio.max() <= 2.0 ** -16
        assert np.all(np.abs(t2) <= 2.0 ** -8 * (1 + 2.0 ** -8) * np.abs(xd))
    # the bound is attained up to a small factor: 2^-18 would be too small
    assert ratio.max() > 2.0 ** -17.5


def test_dot_product_representation_error_within_kappa_terms():
    rng = np.random.default_rng(6)
    d = 128
    for trial in range(200):
        q = _adversarial(d, rng) if trial % 2 else rng.standard_normal(d).astype(np.float32)
        k = _adversarial(d, rng)
        if trial % 4 == 3:  # equal signs everywhere: the errors add up
            q, k = np.abs(q), np.abs(k)
        qd, kd = q.astype(np.float64), k.astype(np.float64)
        exact = qd @ kd
        t1, t2 = _split(q)
        k1, k2 = _split(k)
        bound_scale = np.linalg.norm(qd) * np.linalg.norm(kd)
        # fp32 query and fp32 summary: three terms of the split product
        approx = t1 @ k1 + t1 @ k2 + t2 @ k1
        assert abs(approx - exact) <= 3 * SPLIT_TERM * bound_scale
        # bf16 query (t2 = 0 exactly) with an fp32 summary: one term
        qb = _bf16(q).astype(np.float64)
        assert abs(qb @ k1 + qb @ k2 - qb @ kd) <= SPLIT_TERM * np.linalg.norm(qb) * np.linalg.norm(kd)
