"""Seeded random configurations of the trainer backward: head dim, io dtype, GQA ratio, chunk size,
boundary dtype, ragged lengths (empty sequences included), an upstream dL/dS_T or none, a given or
zero initial state, and which forward kept the stash (two-pass, one-pass, or the trainer forward
with its c and w) drawn together, so that combinations the targeted tests do not list are exercised
too.  For each one:

- every gradient of every sequence (dq, dk per key head; dv, da, db, dL/dS_0 per value head)
  matches the fp64 adjoint oracle at the fp32 bound of tests/test_gpu_backward.py; with bf16
  boundaries the oracle follows the forward's own chunk-start rows (the trajectory it took);
- with fp32 boundaries the gradients equal, bit for bit, those of the same backward after a
  64-token forward: under fp32 boundaries the chunk size moves no bit of the forward, and the
  backward always differentiates on a 64-token stash.
"""
import dataclasses

import numpy as np
import pytest
import torch

import gdn_inputs as gi
from tests.gpu_util import lib, say, sha
from tests.test_gpu_backward import _backward, _compare_all, _oracle

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "da", "db", "d_state0")


def _cases(n=10, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        d = int(rng.choice([16, 32, 64, 128]))
        io = str(rng.choice(["f32", "bf16"]))
        h_k = int(rng.choice([1, 2]))
        ratio = int(rng.choice([1, 2, 4]))
        boundary = str(rng.choice(["f32", "bf16"]))
        chunks = [8, 16, 20, 32, 64] + ([100] if boundary == "f32" else [])
        chunk = int(rng.choice(chunks))
        lens = [int(t) for t in rng.integers(0, 160, size=int(rng.integers(1, 6)))]
        with_ds = bool(rng.integers(0, 2))
        with_s0 = bool(rng.integers(0, 2))
        fwd = str(rng.choice(["two-pass", "one-pass", "trainer"]))
        out.append((c, d, io, h_k, ratio, boundary, chunk, lens, with_ds, with_s0, fwd))
    return out


def _forward(x, pol, s0, fwd):
    """The forward the case names; returns (chunk-state stash, the trainer forward's c and w or None)."""
    cpr = lib()
    xd = x.to("cuda")
    pool = cpr.StatePool(pol, max(x.num_seqs, 1))
    if s0 is not None:
        pool.state[: x.num_seqs].copy_(s0.to("cuda"))
    if fwd == "trainer":
        _, cs, cw = cpr.gdn_trainer_forward(pool, x.cu_seqlens, xd.q, xd.k, xd.v, xd.a, xd.b,
                                            from_state=s0 is not None)
        return cs, cw
    rows = cpr.gdn_chunk_rows_bound(x.total_tokens, x.num_seqs, pol.chunk)
    cs = torch.empty((max(rows, 1), x.h_v, x.dv, x.dk), dtype=torch.float32, device="cuda")
    fn = cpr.gdn_prefill_fused if fwd == "one-pass" else cpr.gdn_prefill
    fn(pool, x.cu_seqlens, xd.q, xd.k, xd.v, xd.a, xd.b, from_state=s0 is not None, chunk_states=cs)
    return cs, None


def _grads(x, ct, pol, fwd):
    cpr = lib()
    cs, cw = _forward(x, pol, ct["s0"], fwd)
    xd = x.to("cuda")
    d_state = None if ct["d_state"] is None else ct["d_state"].to("cuda")
    if cw is not None:
        g = cpr.gdn_backward(pol, x.cu_seqlens, xd.q, xd.k, xd.v, xd.a, xd.b, cs, ct["d_o"].to("cuda"),
                             d_state=d_state, want_d_state0=True, cw=cw)
        torch.cuda.synchronize()
    else:
        g = _backward(x, ct, cs, policy=pol)
    return g, cs


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"case{c[0]}-d{c[1]}-{c[2]}-r{c[4]}-{c[5]}-C{c[6]}-{c[10]}")
def test_random_backward_configuration(case):
    c, d, io, h_k, ratio, boundary, chunk, lens, with_ds, with_s0, fwd = case
    cpr = lib()
    say(f"random backward config {case}")
    x = gi.make_inputs(4000 + c, lens, h_k=h_k, h_v=h_k * ratio, dk=d, dv=d, chunk=chunk, io=io)
    ct = gi.make_cotangents(x, 5000 + c, with_d_state=with_ds, with_s0=with_s0)
    pol = cpr.Policy(h_k, h_k * ratio, d, d, chunk, io, boundary=boundary)
    g, cs = _grads(x, ct, pol, fwd)
    n = int(cpr.gdn_chunk_rows(x.cu_seqlens, chunk)[-1])
    _compare_all(x, g, _oracle(x, ct, starts=cs[:n] if boundary == "bf16" else None))
    if boundary == "f32" and chunk != 64:
        x64 = dataclasses.replace(x, chunk=64)                # the same tensors
        pol64 = cpr.Policy(h_k, h_k * ratio, d, d, 64, io)
        g64, _ = _grads(x64, ct, pol64, fwd)
        for name in GRADS:
            assert sha(g[name]) == sha(g64[name]), f"case {c}: {name} moved with the chunk size"
