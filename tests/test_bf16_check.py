"""CPU tests of the elementwise bf16 output checks (tests/bf16_check.py) that the GPU parity tests
use: an independent fp32 evaluation of the recurrence, rounded to bf16 to nearest even, passes;
the same values rounded by truncation, or an fp32 evaluation with a planted mistake, fail."""
import numpy as np
import pytest

from oracle import recurrence
from tests.bf16_check import (U, bf16_order, check_bf16_outputs, check_state_columns, kernel_dot_depth,
                              output_error_bounds, rne_bf16_bits)


def _bf16_exact(x):
    """Round fp64 samples to bf16 values (kept as fp64): the io dtype of the workloads."""
    u = np.asarray(x, np.float64).astype(np.float32).view(np.uint32)
    u = ((u + (0x7FFF + ((u >> 16) & 1))) >> 16 << 16).astype(np.uint32)
    return u.view(np.float32).astype(np.float64)


def _inputs(seed, T=400, H=2, d=16):
    """The workloads' distributions: q, v ~ N(0, 1); k unit-norm per token; a = exp(-softplus(x)),
    b = sigmoid(y); q, k, v in bf16, a and b in fp32."""
    r = np.random.default_rng(seed)
    q = _bf16_exact(r.standard_normal((T, H, d)))
    k = r.standard_normal((T, H, d))
    k = _bf16_exact(k / np.linalg.norm(k, axis=-1, keepdims=True))
    v = _bf16_exact(r.standard_normal((T, H, d)))
    a = np.exp(-np.logaddexp(0.0, r.standard_normal((T, H)))).astype(np.float32).astype(np.float64)
    b = (1 / (1 + np.exp(-r.standard_normal((T, H))))).astype(np.float32).astype(np.float64)
    return q, k, v, a, b


def _fp32_run(q, k, v, a, b, plant=None):
    """The recurrence in numpy float32 (unfused, library dot products): an fp32 evaluation that
    shares nothing with the kernels.  plant: (t, h) where the correction's sign is flipped."""
    T, H, d = k.shape
    f = np.float32
    o = np.zeros((T, H, d), f)
    S = np.zeros((H, d, d), f)
    for t in range(T):
        for h in range(H):
            kt, qt = k[t, h].astype(f), q[t, h].astype(f)
            u = S[h].T @ kt
            sign = f(-1) if plant == (t, h) else f(1)
            w = v[t, h].astype(f) - sign * f(a[t, h]) * u
            c = f(b[t, h]) * w
            S[h] = f(a[t, h]) * S[h] + np.outer(kt, c)
            o[t, h] = S[h].T @ qt
    return o, S


def _oracle(q, k, v, a, b):
    T, H, d = k.shape
    o = np.zeros((T, H, d))
    S = np.zeros((H, d, d))
    for h in range(H):
        o[:, h], S[h], _ = recurrence(q[:, h], k[:, h], v[:, h], a[:, h], b[:, h])
    return o, S


@pytest.fixture(scope="module")
def case():
    x = _inputs(0)
    ref_o, ref_S = _oracle(*x)
    o32, S32 = _fp32_run(*x)
    E, D, N = output_error_bounds(x[0], x[1], x[2], x[3], x[4], depth=x[1].shape[-1])
    return x, ref_o, ref_S, o32, S32, E, D


def test_rne_rounded_fp32_run_passes(case):
    x, ref_o, ref_S, o32, S32, E, D = case
    stats = check_bf16_outputs(rne_bf16_bits(o32), ref_o, E, "numpy fp32")
    assert stats["ulp_more"] == 0 or stats["ill_conditioned"] > 0
    assert stats["ulp0"] > 0.99 * stats["elements"]
    assert stats["ill_conditioned"] < 0.02 * stats["elements"]
    for h in range(S32.shape[0]):
        check_state_columns(S32[h].astype(np.float64), ref_S[h], D[h], f"state head {h}")
    # the bound is not vacuous: well below a bf16 spacing for typical outputs
    assert np.median(E) < 2.0 ** -12 * np.median(np.abs(ref_o))


def test_truncated_rounding_fails(case):
    x, ref_o, ref_S, o32, S32, E, D = case
    trunc = (np.ascontiguousarray(o32).view(np.uint32) >> 16).astype(np.uint16)
    with pytest.raises(AssertionError, match="outside h/2"):
        check_bf16_outputs(trunc, ref_o, E, "truncated")


def test_rounding_away_from_zero_fails(case):
    x, ref_o, ref_S, o32, S32, E, D = case
    u = np.ascontiguousarray(o32).view(np.uint32)
    up = ((u + np.uint32(0xFFFF)) >> 16).astype(np.uint16)          # round magnitude up
    with pytest.raises(AssertionError):
        check_bf16_outputs(up, ref_o, E, "away from zero")


def test_planted_sign_error_fails(case):
    x, ref_o, ref_S, o32, S32, E, D = case
    bad, _ = _fp32_run(*x, plant=(200, 1))
    with pytest.raises(AssertionError):
        check_bf16_outputs(rne_bf16_bits(bad), ref_o, E, "planted")


def test_one_ulp_rule_and_order():
    """bf16_order counts ulps across zero and binades; two fp32 values closer than half a spacing
    round at most one ulp apart."""
    bits = np.array([0x3F80, 0x3F81, 0x3F7F, 0x0000, 0x8000, 0x8001, 0x0001], np.uint16)
    o = bf16_order(bits)
    assert o[1] - o[0] == 1 and o[0] - o[2] == 1 and o[3] == o[4] and o[6] - o[5] == 2
    r = np.random.default_rng(3).standard_normal(200000)
    x = r * (1 + np.random.default_rng(4).uniform(-1, 1, r.size) * 2.0 ** -10)
    near = np.abs(x - r) < 2.0 ** -9 * np.abs(r) - U * np.abs(r)
    d = np.abs(bf16_order(rne_bf16_bits(x)) - bf16_order(rne_bf16_bits(r)))
    assert near.mean() > 0.9 and d[near].max() <= 1


def test_kernel_depth():
    assert kernel_dot_depth(128) == 12 and kernel_dot_depth(16) == 9 and kernel_dot_depth(8) == 8
