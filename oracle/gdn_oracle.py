"""fp64 CPU oracle for chunkwise-parallel recurrent (CPR) Gated DeltaNet.

TEST INFRASTRUCTURE ONLY.  This module is the plain, slow, obviously correct reference that the
GPU path is checked against.  Only the tests, the package's smoke check and the benchmark's CPU
baseline leg may import it; the product path never does.  It shares no code with the HIP kernels
or their host library and imports nothing from them.

What it computes
----------------
Per section "Solving the linear-attention headache" of the alphasignal.ai article on IsoExec,
CPR treats the token-by-token recurrence as the definition of the result: one pass finds the
state where each chunk begins, a second pass computes every chunk's outputs from that starting
state, and decode applies the recurrence one token at a time, re-basing its state once per chunk.
All three evaluate the same recurrence, so the plain definition of the result is that recurrence
run token by token.  The
pages print no formula; the gated delta rule used here is

    u_t = S_{t-1}^T k_t
    S_t = a_t S_{t-1} + b_t k_t (v_t - a_t u_t)^T           (S is d_k x d_v)
    o_t = S_t^T q_t

with one state per (sequence, value head), key head g = h // (H_v / H_k) (repeat-interleave GQA),
a_t a multiplicative decay and b_t the write strength, both given per (token, value head).
Everything here is fp64 on inputs widened exactly from their fp32/bf16 bits.

Chunk bookkeeping (which states are recorded) follows the same page: a chunk covers absolute
positions [cC, (c+1)C) counted from the sequence's first token, and the recorded "boundary" states
are the states at the start of each chunk the call touches (the first one being the state the
call starts from).  With fp32 boundaries recording them changes no value.

Boundary dtype.  Section "The execution contract" of the same article lists boundary dtypes among
the constants a numerical policy pins.  With a bf16 boundary dtype the state is re-synchronised
to bf16 at every chunk start: just before the token at a position that is a multiple of C is
applied, every element of S is rounded to bf16.  The rounding decision is taken in the kernels'
precision (the fp64 value rounded to fp32, then to bf16, each to nearest even).  The state after
a call's last token is not rounded; whoever applies the next token does it.
"""
from __future__ import annotations

import numpy as np

__all__ = ["recurrence", "boundary_positions", "num_boundary_rows", "gdn_varlen", "bf16_bits_to_f64",
           "round_to_bf16"]


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as fp64."""
    w = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return w.view(np.float32).astype(np.float64)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Each element rounded to fp32 and then to bf16 (round to nearest even both times), as fp64."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def boundary_positions(pos0: int, length: int, chunk: int) -> list:
    """Absolute positions whose incoming state is recorded for a call over [pos0, pos0+length).

    The first is pos0 itself (the state the call starts from); the rest are the chunk starts
    strictly inside the range.  A call with no tokens records nothing."""
    if length <= 0:
        return []
    first = (pos0 // chunk + 1) * chunk
    return [pos0] + list(range(first, pos0 + length, chunk))


def num_boundary_rows(pos0: int, length: int, chunk: int) -> int:
    return len(boundary_positions(pos0, length, chunk))


def recurrence(q, k, v, a, b, S0=None, pos0: int = 0, chunk: int = 64, boundary: str = "f32"):
    """The gated delta rule for one (sequence, value head), token by token, in fp64.

    q, k: [T, d_k]; v: [T, d_v]; a, b: [T]; S0: [d_k, d_v] or None (zero state);
    boundary: "f32" (chunk starts change nothing) or "bf16" (S is rounded to bf16 before the
    token at every chunk-start position is applied).
    Returns (o [T, d_v], S_T [d_k, d_v], boundary states [R, d_k, d_v]) where the boundary
    states are the states entering the positions listed by ``boundary_positions`` (after the
    rounding, at a chunk start).
    """
    if boundary not in ("f32", "bf16"):
        raise ValueError(boundary)
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64, copy=True)
    o = np.zeros((T, dv))
    recorded = []
    for t in range(T):
        p = pos0 + t
        if boundary == "bf16" and p % chunk == 0:
            S = round_to_bf16(S)                    # resynchronise at the chunk start
        if t == 0 or p % chunk == 0:
            recorded.append(S.copy())
        u = S.T @ k[t]                              # u_t = S_{t-1}^T k_t
        w = v[t] - a[t] * u                         # v_t - a_t u_t
        S = a[t] * S + b[t] * np.outer(k[t], w)     # S_t
        o[t] = S.T @ q[t]                           # o_t = S_t^T q_t
    R = np.stack(recorded) if recorded else np.zeros((0, dk, dv))
    return o, S, R


def gdn_varlen(q, k, v, a, b, cu_seqlens, h_k: int, h_v: int, S0=None, pos0=None, chunk: int = 64,
               boundary: str = "f32"):
    """The recurrence over a packed batch of sequences.

    q, k: [N, H_k, d_k]; v: [N, H_v, d_v]; a, b: [N, H_v] (any float dtype, widened to fp64);
    cu_seqlens: [B+1]; S0: [B, H_v, d_k, d_v] or None (zero); pos0: [B] start positions or None.
    Returns (o [N, H_v, d_v], S_final [B, H_v, d_k, d_v], boundary [R, H_v, d_k, d_v]) where the
    boundary rows of sequence i are consecutive, in sequence order, as ``recurrence`` records them.
    """
    if h_v % h_k:
        raise ValueError("H_v must be a multiple of H_k")
    group = h_v // h_k
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    B = len(cu) - 1
    N = int(cu[-1])
    dk = np.shape(k)[-1]
    dv = np.shape(v)[-1]
    o = np.zeros((N, h_v, dv))
    S_fin = np.zeros((B, h_v, dk, dv))
    rows = []
    for i in range(B):
        t0, t1 = int(cu[i]), int(cu[i + 1])
        p0 = 0 if pos0 is None else int(pos0[i])
        per_head = []
        for h in range(h_v):
            g = h // group
            s0 = None if S0 is None else S0[i, h]
            o_h, s_h, r_h = recurrence(q[t0:t1, g], k[t0:t1, g], v[t0:t1, h], a[t0:t1, h], b[t0:t1, h],
                                       S0=s0, pos0=p0, chunk=chunk, boundary=boundary)
            o[t0:t1, h] = o_h
            S_fin[i, h] = s_h
            per_head.append(r_h)
        if t1 > t0:
            rows.append(np.stack(per_head, axis=1))         # [R_i, H_v, dk, dv]
    R = np.concatenate(rows, axis=0) if rows else np.zeros((0, h_v, dk, dv))
    return o, S_fin, R
