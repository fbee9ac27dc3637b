"""Seeded random configurations of the whole forward path: head dim, io dtype, GQA ratio, chunk size,
boundary dtype, ragged lengths (empty sequences included) and a given initial state drawn together,
so that combinations the targeted tests do not enumerate are exercised too.  For each one:

- the two-pass prefill, the one-pass prefill and the overlapped prefill give the same bits (o, final
  states, chunk-start rows);
- every (sequence, value head) matches the fp64 oracle (section "Solving the linear-attention
  headache": the recurrence; "The execution contract": the boundary dtype) at the io dtype's bound.
  With bf16 boundaries the oracle runs chunk by chunk from the GPU's own chunk-start rows: the
  state is rounded to bf16 at every chunk start, and fp64 and fp32 can round an element to
  different bf16 neighbours, so a whole-sequence reference would drift from the path the GPU took.
  The first row is the rounded initial state bit for bit, and every later row lies within bf16
  rounding of the oracle's state at the end of the chunk before it;
- decoding the first non-empty sequence token by token from the same initial state gives the
  prefill's bits, outputs and final state.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
from oracle import recurrence, round_to_bf16
from tests.gpu_util import check_close, lib, say, sha

pytestmark = pytest.mark.gpu


def _cases(n=16, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        d = int(rng.choice([16, 32, 64, 128]))
        io = str(rng.choice(["f32", "bf16"]))
        h_k = int(rng.choice([1, 2]))
        ratio = int(rng.choice([1, 2, 4]))
        chunk = int(rng.choice([1, 5, 16, 64, 100]))
        boundary = str(rng.choice(["f32", "bf16"]))
        lens = [int(t) for t in rng.integers(0, 160, size=int(rng.integers(1, 6)))]
        from_state = bool(rng.integers(0, 2))
        out.append((c, d, io, h_k, ratio, chunk, boundary, lens, from_state))
    return out


def _state0(seed, B, h_v, d):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn((B, h_v, d, d), generator=g, dtype=torch.float64) / d ** 0.5).to(torch.float32)


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"case{c[0]}-d{c[1]}-{c[2]}-r{c[4]}-C{c[5]}-{c[6]}")
def test_random_configuration(case):
    c, d, io, h_k, ratio, chunk, boundary, lens, from_state = case
    cpr = lib()
    h_v = h_k * ratio
    say(f"random config {case}")
    x = gi.make_inputs(2000 + c, lens, h_k=h_k, h_v=h_v, dk=d, dv=d, chunk=chunk, io=io)
    xd = x.to("cuda")
    B = x.num_seqs
    pol = cpr.Policy(h_k, h_v, d, d, chunk, io, boundary=boundary)
    S0 = _state0(3000 + c, B, h_v, d) if from_state else None
    rows = cpr.gdn_chunk_rows_bound(x.total_tokens, B, chunk)
    used = int(cpr.gdn_chunk_rows(x.cu_seqlens, chunk)[-1])

    def run(fn):
        pool = cpr.StatePool(pol, B)
        if S0 is not None:
            pool.state[:B].copy_(S0.to("cuda"))
        cs = torch.empty((max(rows, 1), h_v, d, d), dtype=torch.float32, device="cuda")
        o, _ = fn(pool, x.cu_seqlens, xd.q, xd.k, xd.v, xd.a, xd.b, from_state=from_state, chunk_states=cs)
        torch.cuda.synchronize()
        return o, pool, cs

    o2, p2, cs2 = run(cpr.gdn_prefill)
    o1, p1, cs1 = run(cpr.gdn_prefill_fused)
    o3, p3, cs3 = run(cpr.gdn_prefill_overlapped)
    assert sha(o1) == sha(o2) == sha(o3), "o differs between the prefill paths"
    assert sha(p1.state[:B]) == sha(p2.state[:B]) == sha(p3.state[:B]), "final states differ"
    assert sha(cs1[:used]) == sha(cs2[:used]) == sha(cs3[:used]), "chunk-start rows differ"
    cpr.gdn_device_status()                                   # raises if an overlapped wait gave up

    o_np = o2.float().cpu().double().numpy()
    st = p2.state[:B].cpu().double().numpy()
    cs_np = cs2.cpu().double().numpy()
    row0 = cpr.gdn_chunk_rows(x.cu_seqlens, chunk).numpy()
    for i in range(B):
        t0, t1 = int(x.cu_seqlens[i]), int(x.cu_seqlens[i + 1])
        L = t1 - t0
        for h in range(h_v):
            g = h // ratio
            what = f"case {c} seq {i} head {h}"
            ins = [x.widen("q", slice(t0, t1))[:, g], x.widen("k", slice(t0, t1))[:, g],
                   x.widen("v", slice(t0, t1))[:, h], x.widen("a", slice(t0, t1))[:, h],
                   x.widen("b", slice(t0, t1))[:, h]]
            s0 = np.zeros((d, d)) if S0 is None else S0[i, h].double().numpy().T
            if boundary == "f32" or L == 0:
                ref_o, ref_S, _ = recurrence(*ins, S0=s0, chunk=chunk, boundary=boundary)
            else:                                             # chunk by chunk from the GPU's rows
                parts = []
                assert np.array_equal(cs_np[row0[i], h].T, round_to_bf16(s0)), what + " row 0"
                for cc in range((L + chunk - 1) // chunk):
                    a0, a1 = cc * chunk, min(L, (cc + 1) * chunk)
                    start = cs_np[row0[i] + cc, h].T
                    if cc:                                    # within bf16 rounding of the oracle's
                        err = np.abs(start - ref_S)           # chunk-end state from the previous row
                        assert np.all(err <= 2.0 ** -8 * np.abs(ref_S) + 1e-5), f"{what} row {cc}"
                    oc, ref_S, _ = recurrence(*[t[a0:a1] for t in ins], S0=start, pos0=a0, chunk=chunk,
                                              boundary=boundary)
                    parts.append(oc)
                ref_o = np.concatenate(parts, 0)
            if L > 0:
                check_close(io, o_np[t0:t1, h], ref_o, what + " o")
            check_close(io, st[i, h].T, ref_S, what + " S")

    # decode the first non-empty sequence from the same initial state: the prefill's bits
    nz = [i for i in range(B) if lens[i] > 0]
    if nz:
        i = nz[0]
        t0, t1 = int(x.cu_seqlens[i]), int(x.cu_seqlens[i + 1])
        pool = cpr.StatePool(pol, 1)
        if S0 is not None:
            pool.state[0].copy_(S0[i].to("cuda"))
        ids = torch.zeros(1, dtype=torch.int32, device="cuda")
        outs = [cpr.gdn_decode_step(pool, xd.q[t:t + 1], xd.k[t:t + 1], xd.v[t:t + 1], xd.a[t:t + 1],
                                    xd.b[t:t + 1], slot_ids=ids) for t in range(t0, t1)]
        torch.cuda.synchronize()
        assert sha(torch.cat(outs, 0)) == sha(o2[t0:t1]), f"case {c}: decode o differs from prefill"
        assert sha(pool.state[0]) == sha(p2.state[i]), f"case {c}: decode state differs from prefill"
