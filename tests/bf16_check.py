"""Elementwise checks of bf16 outputs against the fp64 oracle, with a forward error bound of the
fp32 arithmetic that produced them.

The kernels evaluate the recurrence in fp32 and round each output once to bf16 (round to nearest
even).  An output can therefore differ from the exact value by half a bf16 spacing (its own
rounding) plus the error the fp32 arithmetic made before it.  This module bounds that fp32 error
per (token, value head, column) from the inputs alone, so that every output element can be checked
against a bound instead of only a norm over a (sequence, head) block.

Forward error bound (u = 2^-24, gamma_n = n u / (1 - n u), n the depth of the dot's summation:
8 + log2(d_k / 8) for the kernels' 8-row leaves and pairwise tree).  Per column j:
  exact state norm   N_t >= ||S_t[:, j]||_2:  N_t = a_t N_{t-1} + b_t ||k_t|| |v_tj|, since
                     ||a (I - b k k^T)||_2 <= a when b ||k||^2 <= 2;
  fp32 state error   D_t >= ||S~_t[:, j] - S_t[:, j]||_2:  the previous error, contracted the same way,
                     plus the step's own roundings -- the prediction dot (gamma_n ||S~|| ||k|| times
                     a b ||k||), w, c and the product k c (4u b ||k|| |w|), the decay product (u a ||S~||)
                     and the update sum (u (a ||S~|| + b ||k|| |w|)) -- with ||S~|| <= N + D and
                     |w| <= |v| + a ||k|| (N + D);
  output error       |o~_tj - o_tj| <= ||q_t||_2 (D_t + gamma_n (N_t + D_t))   (Cauchy-Schwarz on the dot).
The step's constants cover both a fused (fma) and an unfused evaluation.

What is asserted for every output element g (bf16) with exact value r and bound E:
  |g - r| <= h(g)/2 + E            h(g) the bf16 spacing at g's binade (RNE error <= h/2);
and where the element is well conditioned, 2^-9 |r| > E + u |r|, its distance from the oracle's
value rounded to fp32 and then to bf16 is at most one bf16 ulp (the two fp32 values lie within less
than one spacing of each other, so at most one rounding midpoint falls between them).  Elements
that are not well conditioned (|r| small against the bound: cancellation in the output dot) are
counted, and their share is capped.  A truncating or otherwise wrong rounding fails the first
assertion on about half of all elements.
"""
from __future__ import annotations

import numpy as np

U = 2.0 ** -24


def gamma(n: int) -> float:
    return n * U / (1.0 - n * U)


def kernel_dot_depth(dk: int) -> int:
    """Summation depth of the kernels' pinned dot: 8-row leaves, then a pairwise tree."""
    return 8 + int(np.log2(max(dk // 8, 1)))


def output_error_bounds(q, k, v, a, b, depth: int, N0=None):
    """Bounds for one sequence, all value heads at once.

    q, k: [T, H, d_k] (key heads already expanded to value heads); v: [T, H, d_v]; a, b: [T, H]
    (fp64 copies of the exact inputs).  N0: [H, d_v] column norms of the initial state (None: 0).
    Returns (E [T, H, d_v] bound on each fp32 output's error, D [H, d_v] bound on each column of the
    final state's error, N [H, d_v] bound on each column norm of the exact final state)."""
    T, H, _ = k.shape
    dv = v.shape[-1]
    g = gamma(depth)
    kn = np.linalg.norm(k, axis=-1)                  # [T, H]
    qn = np.linalg.norm(q, axis=-1)
    if np.any(b * kn * kn > 2.0) or np.any(np.abs(a) > 1.0):
        raise ValueError("the norm bound needs b ||k||^2 <= 2 and |a| <= 1")
    N = np.zeros((H, dv)) if N0 is None else np.array(N0, dtype=np.float64)
    D = np.zeros((H, dv))
    E = np.empty((T, H, dv))
    for t in range(T):
        at, bt, kt = a[t][:, None], b[t][:, None], kn[t][:, None]
        St = N + D                                   # bound on the fp32 state's column norm
        w = np.abs(v[t]) + at * kt * St
        N_new = at * N + bt * kt * np.abs(v[t])
        local = at * bt * kt * kt * g * St + 5 * U * bt * kt * w + 2 * U * at * St
        D = at * D + local
        N = N_new
        E[t] = qn[t][:, None] * (D + g * (N + D))
    return E, D, N


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def rne_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 -> bf16, each step round to nearest even (finite values), as uint16 bits."""
    u = np.ascontiguousarray(np.asarray(x, np.float64).astype(np.float32)).view(np.uint32)
    return ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)).astype(np.uint16)


def bf16_spacing(g: np.ndarray) -> np.ndarray:
    """Spacing of bf16 values in the binade of |g| (upper spacing at a power of two)."""
    m, e = np.frexp(np.abs(g))                       # |g| = m 2^e, m in [0.5, 1)
    return np.maximum(np.ldexp(1.0, e - 8), 2.0 ** -133)


def bf16_order(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns as integers in value order (+0 and -0 meet), so differences count ulps."""
    x = np.asarray(bits, np.uint16).astype(np.int64)
    return np.where(x & 0x8000, -(x & 0x7FFF), x)


def check_bf16_outputs(got_bits, ref, E, what: str, max_ill_share: float = 0.03) -> dict:
    """Assert the elementwise bounds above for bf16 outputs `got_bits` (uint16) against exact values
    `ref` (fp64) with fp32 error bounds E (same shape).  Returns counts for the record.
    The share of ill-conditioned elements is capped at 3%: with the workloads' distributions
    (|o| of rms ~0.6 against bounds of ~1e-5) about 1.2% of the outputs fall under 2^9 E."""
    got_bits = np.asarray(got_bits, np.uint16)
    if got_bits.size == 0:
        return {"elements": 0, "ulp0": 0, "ulp1": 0, "ulp_more": 0, "ill_conditioned": 0, "max_err_over_bound": 0.0}
    g = bf16_bits_to_f64(got_bits)
    err = np.abs(g - ref)
    allowed = 0.5 * bf16_spacing(g) + E
    bad = err > allowed
    if bad.any():
        i = np.flatnonzero(bad.ravel())[0]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outputs outside h/2 + E; first at flat "
                             f"index {i}: got {g.ravel()[i]!r}, exact {ref.ravel()[i]!r}, allowed "
                             f"{allowed.ravel()[i]:.3e}")
    dist = np.abs(bf16_order(got_bits) - bf16_order(rne_bf16_bits(ref)))
    well = 2.0 ** -9 * np.abs(ref) > E + U * np.abs(ref)
    far = well & (dist > 1)
    if far.any():
        i = np.flatnonzero(far.ravel())[0]
        raise AssertionError(f"{what}: {int(far.sum())} well-conditioned outputs more than one bf16 ulp from the "
                             f"oracle; first: got {g.ravel()[i]!r}, exact {ref.ravel()[i]!r}")
    ill = int((~well).sum())
    assert ill <= max_ill_share * well.size, f"{what}: {ill} of {well.size} outputs ill-conditioned"
    return {"elements": int(well.size), "ulp0": int((dist == 0).sum()), "ulp1": int((dist == 1).sum()),
            "ulp_more": int((dist > 1).sum()), "ill_conditioned": ill, "max_err_over_bound": float(np.max(err / allowed))}


def check_state_columns(got, ref, D, what: str):
    """Final state: every column's error norm within the bound D.  got, ref: [d_k, d_v] (math
    orientation, fp64), D: [d_v]."""
    col = np.linalg.norm(got - ref, axis=0)
    assert np.all(col <= D * (1 + 1e-6)), f"{what}: column error {col.max():.3e} above its bound"
