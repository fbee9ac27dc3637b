"""Pins for the fp64 oracle: results fixed by the mathematics, not by the oracle itself.

Each test names the plausible oracle mistake it would catch.  The recurrence being pinned is the
gated delta rule that CPR evaluates ("Solving the linear-attention headache", alphasignal.ai page
on IsoExec):  u = S^T k,  S' = a S + b k (v - a u)^T,  o = S'^T q.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import boundary_positions, gdn_varlen, num_boundary_rows, recurrence


def _rand(seed, T, dk, dv, unit_k=True):
    r = np.random.default_rng(seed)
    q = r.standard_normal((T, dk))
    k = r.standard_normal((T, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = r.standard_normal((T, dv))
    a = r.uniform(0.05, 0.99, T)
    b = r.uniform(0.05, 0.99, T)
    S0 = r.standard_normal((dk, dv))
    return q, k, v, a, b, S0


# --- closed forms --------------------------------------------------------------------------------

def test_identity_gate_keeps_state():
    """a=1, b=0: nothing is written or decayed, so S_T = S_0 and o_t = S_0^T q_t exactly."""
    q, k, v, a, b, S0 = _rand(1, 50, 8, 6)
    o, S, _ = recurrence(q, k, v, np.ones(50), np.zeros(50), S0=S0)
    assert np.array_equal(S, S0)
    assert np.allclose(o, q @ S0, rtol=0, atol=1e-13)


def test_delta_rule_projection_unit_key():
    """a=1, b=1, |k|=1: the delta rule overwrites the value stored at k, so S_t^T k_t = v_t.
    Catches a wrong sign in v - a u, a transposed S in u, or a dropped b."""
    q, k, v, a, b, S0 = _rand(2, 40, 16, 16)
    T = len(k)
    S = S0.copy()
    for t in range(T):
        _, S, _ = recurrence(q[t:t + 1], k[t:t + 1], v[t:t + 1], np.ones(1), np.ones(1), S0=S)
        assert np.allclose(S.T @ k[t], v[t], rtol=0, atol=1e-12)


def test_pure_decay():
    """b=0: S_T = (prod a) S_0 and o_t = (prod_{r<=t} a_r) S_0^T q_t.  Catches a dropped decay."""
    q, k, v, a, b, S0 = _rand(3, 30, 8, 8)
    o, S, _ = recurrence(q, k, v, a, np.zeros(30), S0=S0)
    cum = np.cumprod(a)
    assert np.allclose(S, cum[-1] * S0, rtol=1e-13, atol=0)
    assert np.allclose(o, cum[:, None] * (q @ S0), rtol=1e-12, atol=1e-300)


def test_zero_decay_rank_one():
    """a=0: the state is the latest write b_t k_t v_t^T and o_t = b_t (k_t . q_t) v_t.
    Catches w = v - u (a dropped a in the correction) and o read from the old state."""
    q, k, v, a, b, S0 = _rand(4, 20, 8, 5, unit_k=False)
    o, S, _ = recurrence(q, k, v, np.zeros(20), b, S0=S0)
    assert np.allclose(S, b[-1] * np.outer(k[-1], v[-1]), rtol=1e-14, atol=1e-14)
    exp_o = (b * np.sum(k * q, axis=1))[:, None] * v
    assert np.allclose(o, exp_o, rtol=1e-13, atol=1e-14)


def test_exact_integer_vector():
    """a=b=1 with one-hot keys and small integer v, q: every operation is exact in fp64, so the
    oracle must equal integer arithmetic bit for bit.  Each token overwrites row pi(t) with v_t."""
    dk, dv, T = 8, 4, 37
    r = np.random.default_rng(5)
    perm = r.integers(0, dk, T)
    v = r.integers(-8, 9, (T, dv))
    q = r.integers(-4, 5, (T, dk))
    K = np.eye(dk)[perm]
    o, S, _ = recurrence(q.astype(float), K, v.astype(float), np.ones(T), np.ones(T))
    rows = [[0] * dv for _ in range(dk)]           # integer state, row i = S[i, :]
    for t in range(T):
        rows[perm[t]] = [int(x) for x in v[t]]
        exp = [sum(int(q[t, i]) * rows[i][j] for i in range(dk)) for j in range(dv)]
        assert o[t].tolist() == [float(x) for x in exp]
    assert S.tolist() == [[float(x) for x in row] for row in rows]


# --- brute force -----------------------------------------------------------------------------------

def test_unrolled_matrix_products():
    """S_t = A_t S_{t-1} + B_t with A_t = a_t (I - b_t k_t k_t^T), B_t = b_t k_t v_t^T, unrolled as
    S_T = A_T...A_1 S_0 + sum_t (A_T...A_{t+1}) B_t; o_t = S_t^T q_t from the same products."""
    dk, dv, T = 6, 5, 24
    q, k, v, a, b, S0 = _rand(6, T, dk, dv, unit_k=False)
    A = [a[t] * (np.eye(dk) - b[t] * np.outer(k[t], k[t])) for t in range(T)]
    Bm = [b[t] * np.outer(k[t], v[t]) for t in range(T)]
    o_ref = np.zeros((T, dv))
    for t in range(T):
        P = np.eye(dk)
        for r in range(t + 1):
            P = A[r] @ P
        St = P @ S0
        for s in range(t + 1):
            Q = np.eye(dk)
            for r in range(s + 1, t + 1):
                Q = A[r] @ Q
            St = St + Q @ Bm[s]
        o_ref[t] = St.T @ q[t]
    o, S, _ = recurrence(q, k, v, a, b, S0=S0)
    assert np.allclose(S, St, rtol=0, atol=1e-12)
    assert np.allclose(o, o_ref, rtol=0, atol=1e-12)


def test_exact_rational_dyadic():
    """Exact rational arithmetic on 4x4 dyadic inputs bounds the oracle's own rounding error."""
    dk = dv = 4
    T = 12
    r = np.random.default_rng(7)
    dy = lambda *s: r.integers(-16, 17, s) / 16.0
    q, k, v, S0 = dy(T, dk), dy(T, dk), dy(T, dv), dy(dk, dv)
    a = r.integers(1, 16, T) / 16.0
    b = r.integers(1, 16, T) / 16.0
    F = lambda x: Fraction(float(x))
    S = [[F(S0[i, j]) for j in range(dv)] for i in range(dk)]
    o_ex = []
    for t in range(T):
        u = [sum(S[i][j] * F(k[t, i]) for i in range(dk)) for j in range(dv)]
        w = [F(v[t, j]) - F(a[t]) * u[j] for j in range(dv)]
        S = [[F(a[t]) * S[i][j] + F(b[t]) * F(k[t, i]) * w[j] for j in range(dv)] for i in range(dk)]
        o_ex.append([sum(S[i][j] * F(q[t, i]) for i in range(dk)) for j in range(dv)])
    o, Sf, _ = recurrence(q, k, v, a, b, S0=S0)
    assert np.max(np.abs(Sf - np.array([[float(x) for x in row] for row in S]))) < 1e-13
    assert np.max(np.abs(o - np.array([[float(x) for x in row] for row in o_ex]))) < 1e-13


# --- invariants ----------------------------------------------------------------------------------

def test_joint_linearity_in_state_and_values():
    """For fixed gates and keys the map (S_0, v) -> (o, S_T) is linear."""
    q, k, v1, a, b, S1 = _rand(8, 30, 8, 8)
    _, _, v2, _, _, S2 = _rand(9, 30, 8, 8)
    al, be = 0.75, -1.25
    o1, T1, _ = recurrence(q, k, v1, a, b, S0=S1)
    o2, T2, _ = recurrence(q, k, v2, a, b, S0=S2)
    o3, T3, _ = recurrence(q, k, al * v1 + be * v2, a, b, S0=al * S1 + be * S2)
    assert np.allclose(o3, al * o1 + be * o2, atol=1e-12)
    assert np.allclose(T3, al * T1 + be * T2, atol=1e-12)


def test_value_columns_are_independent():
    """Permuting the d_v columns of v and S_0 permutes the columns of o and S_T exactly."""
    q, k, v, a, b, S0 = _rand(10, 25, 8, 7)
    p = np.random.default_rng(10).permutation(7)
    o, S, _ = recurrence(q, k, v, a, b, S0=S0)
    op, Sp, _ = recurrence(q, k, v[:, p], a, b, S0=S0[:, p])
    assert np.allclose(op, o[:, p], rtol=0, atol=1e-14)
    assert np.allclose(Sp, S[:, p], rtol=0, atol=1e-14)


def test_split_and_continue_equals_one_run():
    """Running [0, t1) and continuing from its state at position t1 is the same computation."""
    q, k, v, a, b, S0 = _rand(11, 150, 8, 8)
    o, S, R = recurrence(q, k, v, a, b, S0=S0, chunk=16)
    t1 = 53
    oa, Sa, Ra = recurrence(q[:t1], k[:t1], v[:t1], a[:t1], b[:t1], S0=S0, chunk=16)
    ob, Sb, Rb = recurrence(q[t1:], k[t1:], v[t1:], a[t1:], b[t1:], S0=Sa, pos0=t1, chunk=16)
    assert np.array_equal(np.concatenate([oa, ob]), o)
    assert np.array_equal(Sb, S)
    # recorded states of the two halves: the same chunk starts, plus the hand-over state
    assert np.array_equal(Ra, R[:len(Ra)])
    assert np.array_equal(Rb[0], Sa)
    assert np.array_equal(Rb[1:], R[len(Ra):])


@pytest.mark.parametrize("pos0,length,chunk", [(0, 1, 64), (0, 64, 64), (0, 65, 64), (0, 256, 64),
                                               (5, 59, 64), (5, 60, 64), (63, 2, 64), (64, 64, 64),
                                               (0, 0, 64), (7, 100, 16)])
def test_boundary_rows_are_chunk_start_states(pos0, length, chunk):
    """Recorded row r is the state entering boundary_positions[r], recomputed from scratch."""
    q, k, v, a, b, S0 = _rand(12, max(length, 1), 6, 6)
    q, k, v, a, b = q[:length], k[:length], v[:length], a[:length], b[:length]
    _, _, R = recurrence(q, k, v, a, b, S0=S0, pos0=pos0, chunk=chunk)
    pos = boundary_positions(pos0, length, chunk)
    assert len(R) == len(pos) == num_boundary_rows(pos0, length, chunk)
    for row, p in zip(R, pos):
        n = p - pos0
        _, Sp, _ = recurrence(q[:n], k[:n], v[:n], a[:n], b[:n], S0=S0)
        assert np.array_equal(row, Sp)
    if length:
        assert pos[0] == pos0 and all(p % chunk == 0 for p in pos[1:])
        assert all(pos0 < p < pos0 + length for p in pos[1:])
        expect = 1 + (pos0 + length - 1) // chunk - pos0 // chunk
        assert len(pos) == expect


def test_chunk_size_changes_no_value():
    q, k, v, a, b, S0 = _rand(13, 200, 8, 8)
    o16, S16, _ = recurrence(q, k, v, a, b, S0=S0, chunk=16)
    o64, S64, _ = recurrence(q, k, v, a, b, S0=S0, chunk=64)
    assert np.array_equal(o16, o64) and np.array_equal(S16, S64)


def test_varlen_packing_and_gqa_mapping():
    """The packed driver equals per-sequence, per-head runs, with value head h reading key head
    h // (H_v/H_k) (a catch for h % H_k or a swapped key/value head index)."""
    r = np.random.default_rng(14)
    lens = [5, 0, 33, 64, 1]
    N, hk, hv, dk, dv = sum(lens), 2, 6, 8, 4
    cu = np.concatenate([[0], np.cumsum(lens)])
    q = r.standard_normal((N, hk, dk))
    k = r.standard_normal((N, hk, dk))
    v = r.standard_normal((N, hv, dv))
    a = r.uniform(0.1, 0.9, (N, hv))
    b = r.uniform(0.1, 0.9, (N, hv))
    S0 = r.standard_normal((len(lens), hv, dk, dv))
    pos0 = [0, 3, 70, 64, 127]
    o, S, R = gdn_varlen(q, k, v, a, b, cu, hk, hv, S0=S0, pos0=pos0, chunk=16)
    row = 0
    for i, L in enumerate(lens):
        t0, t1 = cu[i], cu[i + 1]
        nrow = num_boundary_rows(pos0[i], L, 16)
        for h in range(hv):
            g = h // 3
            oh, sh, rh = recurrence(q[t0:t1, g], k[t0:t1, g], v[t0:t1, h], a[t0:t1, h], b[t0:t1, h],
                                    S0=S0[i, h], pos0=pos0[i], chunk=16)
            assert np.array_equal(o[t0:t1, h], oh)
            assert np.array_equal(S[i, h], sh)
            assert np.array_equal(R[row:row + nrow, h], rh)
        row += nrow
    assert row == len(R)
    assert np.array_equal(S[1], S0[1])       # the empty sequence leaves its state alone
    # heads 0..2 share key head 0: with equal values and gates their outputs coincide
    v2, a2, b2 = v.copy(), a.copy(), b.copy()
    v2[:, 1], a2[:, 1], b2[:, 1] = v[:, 0], a[:, 0], b[:, 0]
    v2[:, 3], a2[:, 3], b2[:, 3] = v[:, 0], a[:, 0], b[:, 0]
    o2, _, _ = gdn_varlen(q, k, v2, a2, b2, cu, hk, hv, chunk=16)
    assert np.array_equal(o2[:, 0], o2[:, 1])
    assert not np.allclose(o2[:, 0], o2[:, 3])


# --- bf16 boundary dtype ---------------------------------------------------------------------

def test_round_to_bf16_matches_torch():
    import torch
    from oracle import round_to_bf16
    x = np.random.default_rng(30).standard_normal(100000) * 10.0 ** np.random.default_rng(31).integers(-30, 30, 100000)
    ref = torch.from_numpy(x).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(round_to_bf16(x), ref)


def test_bf16_boundary_rounds_exactly_at_chunk_starts():
    """bf16 mode = f32 mode run to the chunk start, the state rounded there, f32 mode from it on;
    every recorded chunk-start state is bf16-representable; the final state is not rounded."""
    from oracle import round_to_bf16
    q, k, v, a, b, S0 = _rand(32, 150, 8, 8)
    C = 32
    o, S, R = recurrence(q, k, v, a, b, S0=S0, pos0=5, chunk=C, boundary="bf16")
    # by hand: position 5 is not a chunk start; 32, 64, 96, 128 are
    cur, outs, t = S0, [], 0
    for stop in (27, 59, 91, 123, 150):
        ob, cur, _ = recurrence(q[t:stop], k[t:stop], v[t:stop], a[t:stop], b[t:stop], S0=cur)
        outs.append(ob)
        if stop < 150:
            cur = round_to_bf16(cur)
        t = stop
    assert np.array_equal(np.concatenate(outs), o) and np.array_equal(cur, S)
    for row in R[1:]:
        assert np.array_equal(round_to_bf16(row), row)
    assert np.array_equal(R[0], S0)                      # 5 is not a chunk start: no rounding
    assert not np.array_equal(round_to_bf16(S), S)       # the final state is left unrounded


def test_bf16_boundary_is_identity_on_representable_states():
    """With a = 1, b = 0 the state never changes; if S_0 is bf16-representable, rounding is exact
    and bf16 mode equals f32 mode bit for bit."""
    from oracle import round_to_bf16
    q, k, v, a, b, S0 = _rand(33, 100, 8, 8)
    S0 = round_to_bf16(S0)
    o1, S1, _ = recurrence(q, k, v, np.ones(100), np.zeros(100), S0=S0, chunk=16, boundary="bf16")
    o2, S2, _ = recurrence(q, k, v, np.ones(100), np.zeros(100), S0=S0, chunk=16)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)
