"""Pins for the backward oracle: central finite differences of the forward oracle, torch fp64
autograd of an independently written forward, and planted mistakes that must be caught."""
import numpy as np
import pytest
import torch

import oracle.gdn_backward_oracle as gbo
from oracle import gdn_varlen, gdn_varlen_backward, recurrence, recurrence_backward


def _case(seed, T=7, dk=4, dv=3):
    r = np.random.default_rng(seed)
    q, k, v = r.standard_normal((T, dk)), r.standard_normal((T, dk)), r.standard_normal((T, dv))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    a, b = r.uniform(0.2, 0.95, T), r.uniform(0.2, 0.95, T)
    S0, dO, dST = r.standard_normal((dk, dv)), r.standard_normal((T, dv)), r.standard_normal((dk, dv))
    return q, k, v, a, b, S0, dO, dST


def _loss(q, k, v, a, b, S0, dO, dST):
    o, S, _ = recurrence(q, k, v, a, b, S0=S0)
    return float(np.sum(o * dO) + np.sum(S * dST))


@pytest.mark.parametrize("seed", [0, 1])
def test_backward_matches_finite_differences(seed, fn=None):
    fn = fn or recurrence_backward
    q, k, v, a, b, S0, dO, dST = _case(seed)
    grads = dict(zip(["q", "k", "v", "a", "b", "S0"], fn(q, k, v, a, b, dO, S0=S0, dS_T=dST)))
    grads["S0"] = grads["S0"]
    args = dict(q=q, k=k, v=v, a=a, b=b, S0=S0)
    eps = 1e-6
    for name, x in args.items():
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            num[idx] = (_loss(**{**args, name: xp}, dO=dO, dST=dST) - _loss(**{**args, name: xm}, dO=dO, dST=dST)) / (2 * eps)
        assert np.allclose(grads[name], num, rtol=1e-6, atol=1e-7), name


def test_backward_matches_torch_autograd():
    """torch fp64 autograd of a separately written forward gives the same gradients."""
    q, k, v, a, b, S0, dO, dST = _case(3, T=20, dk=8, dv=6)
    T_ = lambda x: torch.tensor(x, dtype=torch.float64, requires_grad=True)
    tq, tk, tv, ta, tb, tS = T_(q), T_(k), T_(v), T_(a), T_(b), T_(S0)
    S = tS
    outs = []
    for t in range(q.shape[0]):
        kt = tk[t]
        corr = tv[t] - ta[t] * (kt @ S)          # v - a S^T k
        S = ta[t] * S + tb[t] * torch.outer(kt, corr)
        outs.append(tq[t] @ S)                   # S^T q
    loss = (torch.stack(outs) * torch.tensor(dO)).sum() + (S * torch.tensor(dST)).sum()
    loss.backward()
    ours = recurrence_backward(q, k, v, a, b, dO, S0=S0, dS_T=dST)
    for g, t in zip(ours, (tq, tk, tv, ta, tb, tS)):
        assert np.allclose(g, t.grad.numpy(), rtol=1e-11, atol=1e-12)


def test_bf16_boundaries_match_torch_straight_through_autograd():
    """With bf16 boundaries the oracle's gradients are those of the rounded forward with the
    rounding read as the identity: torch fp64 autograd of a separately written forward in which each
    chunk start does S = S + (bf16(S) - S).detach() gives the same gradients."""
    q, k, v, a, b, S0, dO, dST = _case(4, T=19, dk=8, dv=6)
    C = 4
    T_ = lambda x: torch.tensor(x, dtype=torch.float64, requires_grad=True)
    tq, tk, tv, ta, tb, tS = T_(q), T_(k), T_(v), T_(a), T_(b), T_(S0)
    S = tS
    outs = []
    for t in range(q.shape[0]):
        if t % C == 0:
            r = S.detach().to(torch.float32).to(torch.bfloat16).to(torch.float64)
            S = S + (r - S).detach()
        kt = tk[t]
        corr = tv[t] - ta[t] * (kt @ S)
        S = ta[t] * S + tb[t] * torch.outer(kt, corr)
        outs.append(tq[t] @ S)
    loss = (torch.stack(outs) * torch.tensor(dO)).sum() + (S * torch.tensor(dST)).sum()
    loss.backward()
    ours = recurrence_backward(q, k, v, a, b, dO, S0=S0, dS_T=dST, chunk=C, boundary="bf16")
    for g, t in zip(ours, (tq, tk, tv, ta, tb, tS)):
        assert np.allclose(g, t.grad.numpy(), rtol=1e-11, atol=1e-12)
    # the rounding is real: the f32-boundary gradients differ
    plain = recurrence_backward(q, k, v, a, b, dO, S0=S0, dS_T=dST)
    assert not np.allclose(plain[3], ours[3], rtol=1e-6, atol=0)


def test_given_chunk_starts_reproduce_the_trajectory():
    """Handing the backward the chunk-start states its own bf16-boundary forward used gives the
    same gradients as letting it round; with f32 boundaries the f32 forward's own starts change
    nothing."""
    q, k, v, a, b, S0, dO, dST = _case(5, T=13, dk=8, dv=4)
    C = 4
    _, _, rows = recurrence(q, k, v, a, b, S0=S0, chunk=C, boundary="bf16")
    starts = {c * C: rows[c] for c in range(len(rows))}
    ref = recurrence_backward(q, k, v, a, b, dO, S0=S0, dS_T=dST, chunk=C, boundary="bf16")
    got = recurrence_backward(q, k, v, a, b, dO, S0=S0, dS_T=dST, chunk=C, starts=starts)
    for g, r in zip(got, ref):
        assert np.array_equal(g, r)
    _, _, rows32 = recurrence(q, k, v, a, b, S0=S0, chunk=C)
    got32 = recurrence_backward(q, k, v, a, b, dO, S0=S0, dS_T=dST, chunk=C,
                                starts={c * C: rows32[c] for c in range(len(rows32))})
    for g, r in zip(got32, recurrence_backward(q, k, v, a, b, dO, S0=S0, dS_T=dST)):
        assert np.allclose(g, r, rtol=1e-12, atol=1e-13)


def test_varlen_backward_sums_value_heads_into_key_heads():
    r = np.random.default_rng(4)
    lens, hk, hv, dk, dv = [5, 0, 9], 1, 2, 4, 3
    N = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k = r.standard_normal((N, hk, dk)), r.standard_normal((N, hk, dk))
    v, dO = r.standard_normal((N, hv, dv)), r.standard_normal((N, hv, dv))
    a, b = r.uniform(0.2, 0.9, (N, hv)), r.uniform(0.2, 0.9, (N, hv))
    dq, dkk, dvv, da, db, dS0 = gdn_varlen_backward(q, k, v, a, b, dO, cu, hk, hv)
    for i in (0, 2):
        t0, t1 = cu[i], cu[i + 1]
        r0 = recurrence_backward(q[t0:t1, 0], k[t0:t1, 0], v[t0:t1, 0], a[t0:t1, 0], b[t0:t1, 0], dO[t0:t1, 0])
        r1 = recurrence_backward(q[t0:t1, 0], k[t0:t1, 0], v[t0:t1, 1], a[t0:t1, 1], b[t0:t1, 1], dO[t0:t1, 1])
        assert np.allclose(dq[t0:t1, 0], r0[0] + r1[0]) and np.allclose(dkk[t0:t1, 0], r0[1] + r1[1])
        assert np.array_equal(dvv[t0:t1, 1], r1[2]) and np.array_equal(db[t0:t1, 0], r0[4])
    # the loss-gradient identity on the packed batch: d/d(scale of v) of sum(o * dO) = <dv, v>
    o, _, _ = gdn_varlen(q, k, v, a, b, cu, hk, hv)
    eps = 1e-6
    lp = np.sum(gdn_varlen(q, k, v * (1 + eps), a, b, cu, hk, hv)[0] * dO)
    lm = np.sum(gdn_varlen(q, k, v * (1 - eps), a, b, cu, hk, hv)[0] * dO)
    assert np.isclose((lp - lm) / (2 * eps), np.sum(dvv * v), rtol=1e-6)


@pytest.mark.parametrize("kind", ["no_state_term_in_dk", "da_uses_new_state", "dq_uses_old_state",
                                  "no_decay_in_adjoint", "db_sign"])
def test_finite_differences_reject_backward_mutants(kind):
    def mutant(q, k, v, a, b, dO, S0=None, dS_T=None):
        T, dk_ = k.shape
        dv_ = v.shape[1]
        S = np.array(S0, dtype=float)
        states, us, ws, cs = [S], [], [], []
        for t in range(T):
            u = S.T @ k[t]; w = v[t] - a[t] * u; c = b[t] * w
            S = a[t] * S + np.outer(k[t], c)
            states.append(S); us.append(u); ws.append(w); cs.append(c)
        G = np.array(dS_T, dtype=float)
        out = [np.zeros((T, dk_)), np.zeros((T, dk_)), np.zeros((T, dv_)), np.zeros(T), np.zeros(T)]
        for t in range(T - 1, -1, -1):
            Sp, St = states[t], states[t + 1]
            Gh = G + np.outer(q[t], dO[t])
            out[0][t] = (Sp if kind == "dq_uses_old_state" else St) @ dO[t]
            dc = Gh.T @ k[t]
            out[1][t] = Gh @ cs[t]
            out[3][t] = np.sum(Gh * (St if kind == "da_uses_new_state" else Sp))
            out[4][t] = (-1 if kind == "db_sign" else 1) * (dc @ ws[t])
            dw = b[t] * dc
            out[2][t] = dw
            out[3][t] -= dw @ us[t]
            du = -a[t] * dw
            if kind != "no_state_term_in_dk":
                out[1][t] += Sp @ du
            G = (1.0 if kind == "no_decay_in_adjoint" else a[t]) * Gh + np.outer(k[t], du)
        return (*out, G)
    with pytest.raises(AssertionError):
        test_backward_matches_finite_differences(0, fn=mutant)
