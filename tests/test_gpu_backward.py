"""Trainer backward on the GPU (gdn_backward) against the fp64 adjoint oracle, plus bitwise
determinism and packing invariance of the gradients.

Tolerance.  Every gradient is produced in fp32 from exactly representable inputs (bf16 io only
changes what the inputs are, not the arithmetic), so the bound is the fp32 one, read relative to
the gradient's own scale, which reaches ~1e2 for dk at d_k = 128:
    max |got - ref| <= 1e-4 * max(1, max |ref|)   and   ||got - ref|| / ||ref|| <= 1e-5
per gradient tensor of a sequence (dq, dk per key head; dv, da, db, dS_0 per value head).  fp32
autograd of the same recurrence on the CPU lands at ~2e-7 normwise and ~1.5e-7 of the scale at
these sizes, so both bounds leave a wide margin while still catching any wrong term.
"""
import dataclasses

import numpy as np
import pytest
import torch

import gdn_inputs as gi
from oracle import gdn_varlen_backward, recurrence_backward
from tests.gpu_util import lib, normwise, policy_of, say, sha

pytestmark = pytest.mark.gpu

REL_MAX = 1e-4
NORMWISE = 1e-5
GRADS = ("dq", "dk", "dv", "da", "db")


def _close(got, ref, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return
    err = float(np.max(np.abs(got - ref)))
    scale = max(1.0, float(np.max(np.abs(ref))))
    assert err <= REL_MAX * scale, f"{what}: max-abs {err:.3e} > {REL_MAX} * {scale:.3e}"
    assert normwise(got, ref) <= NORMWISE, f"{what}: normwise {normwise(got, ref):.3e}"


def _forward(x, s0=None, fused=False, policy=None):
    """Trainer forward on the GPU; returns the chunk-state stash."""
    cpr = lib()
    xd = x.to("cuda")
    pool = cpr.StatePool(policy or policy_of(x), max(x.num_seqs, 1))
    if s0 is not None:
        pool.state[: x.num_seqs].copy_(s0)
    fn = cpr.gdn_prefill_fused if fused else cpr.gdn_prefill
    rows = cpr.gdn_chunk_rows_bound(x.total_tokens, x.num_seqs, x.chunk)
    cs = torch.empty((max(rows, 1), x.h_v, x.dv, x.dk), dtype=torch.float32, device="cuda")
    fn(pool, x.cu_seqlens, xd.q, xd.k, xd.v, xd.a, xd.b, from_state=s0 is not None, chunk_states=cs)
    return cs


def _backward(x, ct, cs, want_d_state0=True, policy=None):
    cpr = lib()
    xd = x.to("cuda")
    d_state = None if ct["d_state"] is None else ct["d_state"].to("cuda")
    g = cpr.gdn_backward(policy or policy_of(x), x.cu_seqlens, xd.q, xd.k, xd.v, xd.a, xd.b, cs, ct["d_o"].to("cuda"),
                         d_state=d_state, want_d_state0=want_d_state0)
    torch.cuda.synchronize()
    return g


def _oracle(x, ct, starts=None):
    """The adjoint oracle; `starts` (the forward's stash) pins it to the trajectory the GPU forward
    took from its chunk-start states."""
    cpu = x.to("cpu")
    dO = ct["d_o"].cpu().double().numpy()
    dS = None if ct["d_state"] is None else ct["d_state"].cpu().double().numpy().transpose(0, 1, 3, 2)
    S0 = None if ct["s0"] is None else ct["s0"].cpu().double().numpy().transpose(0, 1, 3, 2)
    kw = {}
    if starts is not None:
        kw = dict(chunk=x.chunk, chunk_states=starts.cpu().double().numpy().transpose(0, 1, 3, 2),
                  row0=lib().gdn_chunk_rows(x.cu_seqlens, x.chunk).numpy())
    return gdn_varlen_backward(cpu.widen("q"), cpu.widen("k"), cpu.widen("v"), cpu.widen("a"), cpu.widen("b"),
                               dO, x.cu_seqlens, x.h_k, x.h_v, S0=S0, dS_T=dS, **kw)


def _compare_all(x, g, ref):
    names = GRADS + ("dS0",)
    for i in range(x.num_seqs):
        t0, t1 = int(x.cu_seqlens[i]), int(x.cu_seqlens[i + 1])
        for n, r in zip(names, ref):
            if n == "dS0":
                got = g["d_state0"][i].cpu().double().numpy().transpose(0, 2, 1)
                _close(got, r[i], f"seq {i} dS0")
            else:
                got = g[n][t0:t1].cpu().double().numpy()
                _close(got, r[t0:t1], f"seq {i} {n}")


CASES = [
    # dim, io, chunk, with d_state, with S0
    (16, "f32", 16, True, True),
    (16, "f32", 64, False, False),
    (32, "f32", 8, True, False),
    (64, "bf16", 32, True, True),
    (128, "bf16", 64, True, True),
    (128, "f32", 20, False, True),
]


@pytest.mark.parametrize("dim,io,chunk,with_ds,with_s0", CASES)
def test_backward_matches_oracle(dim, io, chunk, with_ds, with_s0):
    lens = [1, 64, 65, 200, 0, 33]
    x = gi.make_inputs(61, lens, h_k=2, h_v=4, dk=dim, dv=dim, chunk=chunk, io=io)
    ct = gi.make_cotangents(x, 62, with_d_state=with_ds, with_s0=with_s0)
    say(f"backward vs oracle dim={dim} io={io} C={chunk} dS={with_ds} S0={with_s0}")
    cs = _forward(x, None if ct["s0"] is None else ct["s0"].to("cuda"))
    g = _backward(x, ct, cs)
    _compare_all(x, g, _oracle(x, ct))


@pytest.mark.parametrize("dim,io,chunk", [(16, "f32", 8), (128, "bf16", 64)])
def test_backward_bf16_boundaries_straight_through(dim, io, chunk):
    """bf16 boundary dtype: the forward rounds the state at every chunk start and the backward
    reads the rounding as the identity.  Against the adjoint oracle run on the GPU forward's own
    chunk-start states (the trajectory the forward took), at the fp32 tolerances; the stash rows
    are bf16 values, so the rounding did happen."""
    lens = [1, 64, 65, 200, 0, 33]
    x = gi.make_inputs(65, lens, h_k=2, h_v=4, dk=dim, dv=dim, chunk=chunk, io=io)
    ct = gi.make_cotangents(x, 66, with_d_state=True, with_s0=True)
    pol = lib().Policy(x.h_k, x.h_v, x.dk, x.dv, chunk, io, boundary="bf16")
    say(f"backward, bf16 boundaries, dim={dim} io={io} C={chunk}")
    cs = _forward(x, ct["s0"].to("cuda"), policy=pol)
    n = int(lib().gdn_chunk_rows(x.cu_seqlens, chunk)[-1])
    rows = cs[:n].cpu()
    assert torch.equal(rows, rows.to(torch.bfloat16).to(torch.float32))
    g = _backward(x, ct, cs, policy=pol)
    _compare_all(x, g, _oracle(x, ct, starts=cs[:n]))


@pytest.mark.parametrize("dim,io,chunk", [(16, "f32", 100), (32, "f32", 128), (128, "bf16", 256)])
def test_backward_chunk_above_64_equals_chunk_64(dim, io, chunk):
    """A chunk above the gradient kernel's 64-token tile: the backward first rebuilds a 64-token
    stash from each sequence's row 0 of the forward's stash.  With fp32 boundaries that is the
    stash a 64-token forward keeps, so the gradients match the oracle and equal the chunk-64
    backward bit for bit; with the trainer forward's c and w they are the same bits again."""
    cpr = lib()
    lens = [0, 1, 64, 65, 200, 0, 33, 300, 0]
    x = gi.make_inputs(72, lens, h_k=2, h_v=4, dk=dim, dv=dim, chunk=chunk, io=io)
    x64 = dataclasses.replace(x, chunk=64)
    ct = gi.make_cotangents(x, 73, with_d_state=True, with_s0=True)
    say(f"backward, chunk {chunk} > 64, dim={dim} io={io}")
    s0 = ct["s0"].to("cuda")
    g = _backward(x, ct, _forward(x, s0))
    _compare_all(x, g, _oracle(x, ct))
    g64 = _backward(x64, ct, _forward(x64, s0))
    for n in GRADS + ("d_state0",):
        assert sha(g[n]) == sha(g64[n]), n
    # from zero states, with the kept c and w of the trainer forward at this chunk
    xd = x.to("cuda")
    pool = cpr.StatePool(policy_of(x), x.num_seqs)
    _, cs, cw = cpr.gdn_trainer_forward(pool, x.cu_seqlens, xd.q, xd.k, xd.v, xd.a, xd.b)
    d_state = ct["d_state"].to("cuda")
    g1 = cpr.gdn_backward(policy_of(x), x.cu_seqlens, xd.q, xd.k, xd.v, xd.a, xd.b, cs, ct["d_o"].to("cuda"),
                          d_state=d_state, want_d_state0=True, cw=cw)
    g2 = _backward(x64, ct, _forward(x64))
    for n in GRADS + ("d_state0",):
        assert sha(g1[n]) == sha(g2[n]), n


def test_backward_gqa_ratio_four():
    x = gi.make_inputs(63, [150, 64, 9], h_k=2, h_v=8, dk=64, dv=64, chunk=64, io="bf16")
    ct = gi.make_cotangents(x, 64)
    say("backward vs oracle GQA 4:1")
    g = _backward(x, ct, _forward(x))
    _compare_all(x, g, _oracle(x, ct))


def test_backward_deterministic_and_packing_invariant():
    lens = [300, 1, 128, 77, 0, 190]
    x = gi.make_inputs(65, lens, h_k=2, h_v=4, dk=128, dv=128, chunk=64, io="bf16")
    ct = gi.make_cotangents(x, 66, with_s0=True)
    say("backward determinism and packing")
    s0 = ct["s0"].to("cuda")
    cs = _forward(x, s0)
    g1 = _backward(x, ct, cs)
    g2 = _backward(x, ct, _forward(x, s0, fused=True))     # stash of the one-pass forward
    for n in GRADS + ("d_state0",):
        assert sha(g1[n]) == sha(g2[n]), n
    for i, L in enumerate(lens):
        t0, t1 = int(x.cu_seqlens[i]), int(x.cu_seqlens[i + 1])
        xi = x.select([i])
        cti = {"d_o": ct["d_o"][t0:t1].contiguous(), "d_state": ct["d_state"][i:i + 1].contiguous(),
               "s0": ct["s0"][i:i + 1].contiguous()}
        gi_ = _backward(xi, cti, _forward(xi, cti["s0"].to("cuda")))
        for n in GRADS:
            assert sha(gi_[n]) == sha(g1[n][t0:t1]), (i, n)
        assert sha(gi_["d_state0"][0]) == sha(g1["d_state0"][i]), i


@pytest.mark.parametrize("dim,io", [(32, "f32"), (128, "bf16")])
def test_backward_bits_do_not_depend_on_the_chunk(dim, io):
    """With fp32 boundaries the chunk size is a deployment setting (it is left out of the policy
    digest): the forward's bits do not depend on it, and neither do the gradients', because the
    backward always differentiates at chunk 64 on a 64-token stash rebuilt from each sequence's
    first row.  Every gradient is the same bits for C in {8, 20, 32, 64, 100}, from the forward's
    stash and from the trainer forward's kept c and w, and matches the oracle."""
    cpr = lib()
    x = gi.make_inputs(67, [257, 0, 64, 1, 130], h_k=2, h_v=4, dk=dim, dv=dim, chunk=64, io=io)
    ct = gi.make_cotangents(x, 68, with_s0=True)
    s0 = ct["s0"].to("cuda")
    ref = _oracle(x, ct)
    digests = []
    for C in (8, 20, 32, 64, 100):
        say(f"backward bits at chunk {C} dim={dim} io={io}")
        xc = dataclasses.replace(x, chunk=C)
        pol = policy_of(xc)
        assert cpr.gdn_policy_digest(pol) == cpr.gdn_policy_digest(policy_of(x))
        g = _backward(xc, ct, _forward(xc, s0))
        _compare_all(xc, g, ref)
        digests.append(tuple(sha(g[n]) for n in GRADS + ("d_state0",)))
        # the trainer forward's c and w at this chunk, from zero states
        xd = xc.to("cuda")
        pool = cpr.StatePool(pol, xc.num_seqs)
        _, cs, cw = cpr.gdn_trainer_forward(pool, xc.cu_seqlens, xd.q, xd.k, xd.v, xd.a, xd.b)
        g1 = cpr.gdn_backward(pol, xc.cu_seqlens, xd.q, xd.k, xd.v, xd.a, xd.b, cs, ct["d_o"].to("cuda"),
                              d_state=ct["d_state"].to("cuda"), cw=cw)
        torch.cuda.synchronize()
        digests.append(tuple(sha(g1[n]) for n in GRADS) + ("zero-start",))
    assert len(set(d for d in digests if d[-1] != "zero-start")) == 1
    assert len(set(d for d in digests if d[-1] == "zero-start")) == 1


def test_backward_bf16_boundaries_depend_on_the_chunk():
    """With bf16 boundaries the chunk is numerical policy: the rounded trajectory moves with C, so
    do the gradients, and the policy digests differ."""
    cpr = lib()
    x = gi.make_inputs(75, [200, 77], h_k=1, h_v=2, dk=32, dv=32, chunk=32, io="f32")
    ct = gi.make_cotangents(x, 76)
    say("backward, bf16 boundaries at chunks 16 and 32")
    out = []
    for C in (16, 32):
        xc = dataclasses.replace(x, chunk=C)
        pol = cpr.Policy(x.h_k, x.h_v, x.dk, x.dv, C, "f32", boundary="bf16")
        g = _backward(xc, ct, _forward(xc, policy=pol), policy=pol)
        out.append((cpr.gdn_policy_digest(pol), sha(g["dk"])))
    assert out[0][0] != out[1][0] and out[0][1] != out[1][1]


def test_backward_trainer_10240_varlen():
    """The trainer workload (10240 tokens packed varlen, 32 value heads over 16 key heads,
    d = 128, chunk 64, bf16): sampled oracle parity on every sequence for key head 5 (value
    heads 10 and 11), finite gradients everywhere, and packing invariance for one sequence."""
    cpr = lib()
    x = gi.trainer_10240(device="cuda")
    ct = gi.make_cotangents(x, 69, device="cuda")
    say(f"backward trainer 10240 lengths={x.lengths.tolist()}")
    cs = _forward(x)
    g = _backward(x, ct, cs)
    for n in GRADS + ("d_state0",):
        assert bool(torch.isfinite(g[n]).all()), n
    cpu = x.to("cpu")
    dO = ct["d_o"].cpu().double().numpy()
    dS = ct["d_state"].cpu().double().numpy()
    kh = 5
    for i in range(x.num_seqs):
        t0, t1 = int(x.cu_seqlens[i]), int(x.cu_seqlens[i + 1])
        rows = slice(t0, t1)
        dq = dk = 0
        for h in (2 * kh, 2 * kh + 1):
            r = recurrence_backward(cpu.widen("q", rows)[:, kh], cpu.widen("k", rows)[:, kh],
                                    cpu.widen("v", rows)[:, h], cpu.widen("a", rows)[:, h],
                                    cpu.widen("b", rows)[:, h], dO[t0:t1, h], None, dS[i, h].T)
            dq, dk = dq + r[0], dk + r[1]
            _close(g["dv"][t0:t1, h].cpu().double().numpy(), r[2], f"seq {i} dv h{h}")
            _close(g["da"][t0:t1, h].cpu().double().numpy(), r[3], f"seq {i} da h{h}")
            _close(g["db"][t0:t1, h].cpu().double().numpy(), r[4], f"seq {i} db h{h}")
            _close(g["d_state0"][i, h].cpu().double().numpy().T, r[5], f"seq {i} dS0 h{h}")
        _close(g["dq"][t0:t1, kh].cpu().double().numpy(), dq, f"seq {i} dq")
        _close(g["dk"][t0:t1, kh].cpu().double().numpy(), dk, f"seq {i} dk")
    # packing: the last sequence alone gives the same bits
    i = x.num_seqs - 1
    t0, t1 = int(x.cu_seqlens[i]), int(x.cu_seqlens[i + 1])
    xi = x.select([i])
    cti = {"d_o": ct["d_o"][t0:t1].contiguous(), "d_state": ct["d_state"][i:i + 1].contiguous(), "s0": None}
    gi_ = _backward(xi, cti, _forward(xi))
    for n in GRADS:
        assert sha(gi_[n]) == sha(g[n][t0:t1]), n
    assert cpr.gdn_backward_workspace_bytes(policy_of(x), x.total_tokens, x.num_seqs) > 0


@pytest.mark.parametrize("dim,io", [(16, "f32"), (128, "bf16")])
def test_trainer_forward_stash_gives_the_same_gradients(dim, io):
    """gdn_trainer_forward equals gdn_prefill bit for bit (o, final states, chunk states), and the
    c and w it keeps are the bits the backward's replay recomputes: the gradients with and
    without the kept values are identical."""
    cpr = lib()
    x = gi.make_inputs(70, [1, 64, 65, 200, 0, 33], h_k=2, h_v=4, dk=dim, dv=dim, chunk=32, io=io)
    ct = gi.make_cotangents(x, 71)
    say(f"trainer forward stash dim={dim} io={io}")
    xd = x.to("cuda")
    p1 = cpr.StatePool(policy_of(x), x.num_seqs)
    p2 = cpr.StatePool(policy_of(x), x.num_seqs)
    o1, cs1 = cpr.gdn_prefill(p1, x.cu_seqlens, xd.q, xd.k, xd.v, xd.a, xd.b)
    o2, cs2, cw = cpr.gdn_trainer_forward(p2, x.cu_seqlens, xd.q, xd.k, xd.v, xd.a, xd.b)
    torch.cuda.synchronize()
    n = int(cpr.gdn_chunk_rows(x.cu_seqlens, x.chunk)[-1])
    assert sha(o1) == sha(o2) and sha(p1.state) == sha(p2.state) and sha(cs1[:n]) == sha(cs2[:n])
    d_state = ct["d_state"].to("cuda")
    g1 = cpr.gdn_backward(policy_of(x), x.cu_seqlens, xd.q, xd.k, xd.v, xd.a, xd.b, cs1, ct["d_o"].to("cuda"),
                          d_state=d_state, want_d_state0=True)
    g2 = cpr.gdn_backward(policy_of(x), x.cu_seqlens, xd.q, xd.k, xd.v, xd.a, xd.b, cs2, ct["d_o"].to("cuda"),
                          d_state=d_state, want_d_state0=True, cw=cw)
    torch.cuda.synchronize()
    for name in GRADS + ("d_state0",):
        assert sha(g1[name]) == sha(g2[name]), name


@pytest.mark.parametrize("lens,chunk", [([0, 3, 0], 16), ([0, 0], 16), ([0, 0], 100)])
def test_backward_empty_sequences(lens, chunk):
    """Empty sequences: a sequence with no token passes dL/dS_T through to dL/dS_0 unchanged and its
    neighbours are unaffected; a batch of empty sequences alone (also where C > 64 makes the
    backward rebuild a 64-token stash) gives just that."""
    x = gi.make_inputs(79, lens, h_k=2, h_v=4, dk=16, dv=16, chunk=chunk, io="f32")
    ct = gi.make_cotangents(x, 80, with_d_state=True, with_s0=True)
    say(f"backward, empty sequences {lens} C={chunk}")
    cs = _forward(x, ct["s0"].to("cuda"))
    g = _backward(x, ct, cs)
    _compare_all(x, g, _oracle(x, ct))
    for i, n in enumerate(lens):
        if n == 0:
            assert sha(g["d_state0"][i]) == sha(ct["d_state"][i].to("cuda")), i
