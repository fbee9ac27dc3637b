"""fp64 CPU oracle for the gradients of the gated delta rule (the trainer's backward pass).

TEST INFRASTRUCTURE ONLY, like gdn_oracle.py: imported by the tests and the benchmark's CPU leg,
never by the product path, and sharing no code with it.

The table in section "Solving the linear-attention headache" (alphasignal.ai article on IsoExec)
times CPR for the trainer's forward and backward.  The pages give no formulas for either; this is
reverse-mode differentiation of the recurrence the forward oracle defines,

    u_t = S_{t-1}^T k_t,  w_t = v_t - a_t u_t,  c_t = b_t w_t,  S_t = a_t S_{t-1} + k_t c_t^T,
    o_t = S_t^T q_t,

for a loss L with upstream gradients dO_t = dL/do_t and dS_T = dL/dS_T.  With G_t = dL/dS_t
(G_T = dS_T), going from the last token to the first:

    Ghat_t = G_t + q_t dO_t^T                      (o_t reads S_t)
    dq_t   = S_t dO_t
    dc_t   = Ghat_t^T k_t;  dk_t = Ghat_t c_t;  da_t = <Ghat_t, S_{t-1}>   (S_t = a S + k c^T)
    db_t   = <dc_t, w_t>;   dw_t = b_t dc_t                               (c = b w)
    dv_t   = dw_t;  da_t -= <dw_t, u_t>;  du_t = -a_t dw_t                 (w = v - a u)
    dk_t  += S_{t-1} du_t                                                 (u = S^T k)
    G_{t-1} = a_t Ghat_t + k_t du_t^T

and dS_0 = G_0.  Key heads receive the sum of their value heads' dq and dk.

Boundary dtype.  With bf16 boundaries the forward rounds S to bf16 just before each token at a
chunk-start position (the forward oracle's resynchronisation).  Rounding has a zero derivative
almost everywhere, so the backward reads it as the identity (straight-through): every formula above
uses the state the token actually read, and G passes through the rounding unchanged.  A caller
may instead hand in the chunk-start states a forward used (`starts`), so that the gradients follow
exactly that trajectory.
"""
from __future__ import annotations

import numpy as np

from .gdn_oracle import round_to_bf16

__all__ = ["recurrence_backward", "gdn_varlen_backward"]


def recurrence_backward(q, k, v, a, b, dO, S0=None, dS_T=None, chunk: int = 64, boundary: str = "f32",
                        starts=None):
    """Gradients for one (sequence, value head), in fp64, for a forward that starts at position 0.

    q, k: [T, d_k]; v: [T, d_v]; a, b: [T]; dO: [T, d_v]; S0, dS_T: [d_k, d_v] or None (zero).
    boundary "bf16": S is rounded to bf16 before every token at a multiple of `chunk` (straight-
    through in the backward).  starts: optional {t: [d_k, d_v]} states that replace S just before
    token t (the chunk-start states a forward used).
    Returns (dq [T, d_k], dk [T, d_k], dv [T, d_v], da [T], db [T], dS0 [d_k, d_v])."""
    q, k, v, a, b, dO = (np.asarray(x, np.float64) for x in (q, k, v, a, b, dO))
    if boundary not in ("f32", "bf16"):
        raise ValueError("boundary must be 'f32' or 'bf16'")
    T, dk_ = k.shape
    dv_ = v.shape[1]
    S = np.zeros((dk_, dv_)) if S0 is None else np.array(S0, dtype=np.float64, copy=True)
    # forward, keeping the state each token read, the state it left and its intermediates
    prev, after = [], []
    us, ws, cs = [], [], []
    for t in range(T):
        if starts is not None and t in starts:
            S = np.array(starts[t], dtype=np.float64, copy=True)
        elif boundary == "bf16" and t % chunk == 0:
            S = round_to_bf16(S)
        prev.append(S)
        u = S.T @ k[t]
        w = v[t] - a[t] * u
        c = b[t] * w
        S = a[t] * S + np.outer(k[t], c)
        after.append(S)
        us.append(u)
        ws.append(w)
        cs.append(c)
    G = np.zeros((dk_, dv_)) if dS_T is None else np.array(dS_T, dtype=np.float64, copy=True)
    dq = np.zeros((T, dk_))
    dkk = np.zeros((T, dk_))
    dv = np.zeros((T, dv_))
    da = np.zeros(T)
    db = np.zeros(T)
    for t in range(T - 1, -1, -1):
        S_prev, S_t = prev[t], after[t]
        Gh = G + np.outer(q[t], dO[t])
        dq[t] = S_t @ dO[t]
        dc = Gh.T @ k[t]
        dkk[t] = Gh @ cs[t]
        da[t] = np.sum(Gh * S_prev)
        db[t] = dc @ ws[t]
        dw = b[t] * dc
        dv[t] = dw
        da[t] -= dw @ us[t]
        du = -a[t] * dw
        dkk[t] += S_prev @ du
        G = a[t] * Gh + np.outer(k[t], du)
    return dq, dkk, dv, da, db, G


def gdn_varlen_backward(q, k, v, a, b, dO, cu_seqlens, h_k: int, h_v: int, S0=None, dS_T=None,
                        chunk: int = 64, boundary: str = "f32", chunk_states=None, row0=None):
    """Gradients over a packed batch.  q, k: [N, H_k, d_k]; v, dO: [N, H_v, d_v]; a, b: [N, H_v];
    S0, dS_T: [B, H_v, d_k, d_v] or None.  chunk_states [rows, H_v, d_k, d_v] with row0[i] the
    first row of sequence i: the chunk-start states a forward used (chunk c of sequence i starts
    from row row0[i] + c).  Returns (dq, dk [N, H_k, d_k], dv [N, H_v, d_v], da, db [N, H_v],
    dS0 [B, H_v, d_k, d_v]); dq and dk of a key head sum its value heads."""
    group = h_v // h_k
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    B, N = len(cu) - 1, int(cu[-1])
    dk_, dv_ = np.shape(k)[-1], np.shape(v)[-1]
    dq = np.zeros((N, h_k, dk_))
    dkk = np.zeros((N, h_k, dk_))
    dv = np.zeros((N, h_v, dv_))
    da = np.zeros((N, h_v))
    db = np.zeros((N, h_v))
    dS0 = np.zeros((B, h_v, dk_, dv_))
    for i in range(B):
        t0, t1 = int(cu[i]), int(cu[i + 1])
        for h in range(h_v):
            g = h // group
            starts = None
            if chunk_states is not None:
                starts = {c * chunk: chunk_states[int(row0[i]) + c, h] for c in range((t1 - t0 + chunk - 1) // chunk)}
            r = recurrence_backward(q[t0:t1, g], k[t0:t1, g], v[t0:t1, h], a[t0:t1, h], b[t0:t1, h],
                                    dO[t0:t1, h], None if S0 is None else S0[i, h],
                                    None if dS_T is None else dS_T[i, h], chunk=chunk, boundary=boundary,
                                    starts=starts)
            dq[t0:t1, g] += r[0]
            dkk[t0:t1, g] += r[1]
            dv[t0:t1, h] = r[2]
            da[t0:t1, h] = r[3]
            db[t0:t1, h] = r[4]
            dS0[i, h] = r[5]
    return dq, dkk, dv, da, db, dS0
