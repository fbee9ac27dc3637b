"""bf16 boundary dtype on the GPU: the state is resynchronised (rounded to bf16) at every chunk
start, by every path at the same positions ("The execution contract": boundary dtypes are pinned
constants).  Parity against the oracle's rounding model; bitwise identity across two-pass
prefill, one-pass prefill, decode, continuation and packing.

Tolerance: normwise 3e-3 per (sequence, value head) for both io dtypes.  A rounding decision the
GPU takes on its fp32 state can differ from the oracle's (taken on the fp32 rounding of its fp64
state) when the two values straddle a bf16 rounding point; that element then differs by one bf16
ulp, which an elementwise 1e-4 bound would flag although both sides followed the rule.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
from oracle import round_to_bf16
from tests.gpu_util import gpu_state_math, lib, normwise, oracle_seq_head, prefill, say, sha

pytestmark = pytest.mark.gpu


def _policy(x, chunk=None):
    cpr = lib()
    return cpr.Policy(x.h_k, x.h_v, x.dk, x.dv, chunk or x.chunk, x.io, boundary="bf16")


def _prefill(x, pool=None, from_state=False, fused=False, chunk=None):
    cpr = lib()
    xd = x.to("cuda")
    pool = pool or cpr.StatePool(_policy(x, chunk), max(x.num_seqs, 1), boundary=True)
    rows = cpr.gdn_chunk_rows_bound(x.total_tokens, x.num_seqs, pool.policy.chunk)
    cs = torch.zeros((max(rows, 1), x.h_v, x.dv, x.dk), device="cuda")
    fn = cpr.gdn_prefill_fused if fused else cpr.gdn_prefill
    o, cs = fn(pool, x.cu_seqlens, xd.q, xd.k, xd.v, xd.a, xd.b, from_state=from_state, chunk_states=cs)
    torch.cuda.synchronize()
    return o, pool, cs


def _decode(x, pool, slot=0):
    cpr = lib()
    xd = x.to("cuda")
    ids = torch.tensor([slot], dtype=torch.int32, device="cuda")
    out = [cpr.gdn_decode_step(pool, xd.q[t:t + 1], xd.k[t:t + 1], xd.v[t:t + 1], xd.a[t:t + 1], xd.b[t:t + 1],
                               slot_ids=ids) for t in range(x.total_tokens)]
    torch.cuda.synchronize()
    return torch.cat(out)


@pytest.mark.parametrize("dim,io", [(16, "f32"), (64, "bf16"), (128, "bf16")])
def test_bf16_boundaries_match_oracle(dim, io):
    cpr = lib()
    lens = [1, 64, 65, 200, 0, 33]
    x = gi.make_inputs(41, lens, h_k=2, h_v=4, dk=dim, dv=dim, chunk=32, io=io)
    say(f"bf16 boundaries vs oracle dim={dim} io={io}")
    o, pool, cs = _prefill(x)
    rows = cpr.gdn_chunk_rows(x.cu_seqlens, 32).numpy()
    o_np = o.float().cpu().double().numpy()
    for i, L in enumerate(lens):
        t0, t1 = int(x.cu_seqlens[i]), int(x.cu_seqlens[i + 1])
        for h in range(x.h_v):
            ref_o, ref_S, ref_R = oracle_seq_head(x, i, h)
            ref_o_b, ref_S_b, ref_R_b = _oracle_bf16(x, i, h)
            if L:
                assert normwise(o_np[t0:t1, h], ref_o_b) <= 3e-3
            assert normwise(gpu_state_math(pool, i, h), ref_S_b) <= 3e-3
            for r in range(len(ref_R_b)):
                got = cs[rows[i] + r, h].cpu().double().numpy().T
                assert normwise(got, ref_R_b[r]) <= 3e-3
                if r > 0:                                       # a chunk start: bf16-representable
                    assert np.array_equal(round_to_bf16(got), got)
            if L > 32 and h == 0:
                # the rounding is real: the f32-boundary result differs from the bf16 one
                assert not np.array_equal(ref_o, ref_o_b)


def _oracle_bf16(x, i, h):
    from oracle import recurrence
    t0, t1 = int(x.cu_seqlens[i]), int(x.cu_seqlens[i + 1])
    g = h // (x.h_v // x.h_k)
    rows = slice(t0, t1)
    return recurrence(x.widen("q", rows)[:, g], x.widen("k", rows)[:, g], x.widen("v", rows)[:, h],
                      x.widen("a", rows)[:, h], x.widen("b", rows)[:, h], chunk=x.chunk, boundary="bf16")


@pytest.mark.parametrize("chunk", [16, 64])
def test_bf16_boundaries_identical_across_paths(chunk):
    cpr = lib()
    x = gi.make_inputs(42, [300], h_k=2, h_v=4, dk=128, dv=128, chunk=chunk, io="bf16")
    say(f"bf16 boundaries: paths C={chunk}")
    o2, pool2, cs2 = _prefill(x)
    o1, pool1, cs1 = _prefill(x, fused=True)
    assert sha(o1) == sha(o2) and sha(pool1.state) == sha(pool2.state)
    n = int(cpr.gdn_chunk_rows([0, 300], chunk)[-1])
    assert sha(cs1[:n]) == sha(cs2[:n])
    pool_d = cpr.StatePool(_policy(x), 1, boundary=True)
    od = _decode(x, pool_d)
    assert sha(od) == sha(o2) and sha(pool_d.state) == sha(pool2.state)
    last = (299 // chunk) * chunk
    assert int(pool_d.boundary_pos[0]) == last and sha(pool_d.boundary[0]) == sha(cs2[last // chunk])
    # split: a prefill ending mid-chunk, a continuation ending on a chunk start, then decode
    cut1, cut2 = chunk + 5, 3 * chunk
    pool_s = cpr.StatePool(_policy(x), 1)
    oa, _, _ = _prefill(x.token_slice(0, cut1), pool=pool_s)
    ob, _, _ = _prefill(x.token_slice(cut1, cut2), pool=pool_s, from_state=True, fused=True)
    oc = _decode(x.token_slice(cut2, 300), pool_s)
    assert sha(torch.cat([oa, ob, oc])) == sha(o2) and sha(pool_s.state) == sha(pool2.state)
    # and the result is not the fp32-boundary one
    o32, _, _ = prefill(x)
    assert sha(o32) != sha(o2)


def test_bf16_boundaries_packing_invariance():
    x = gi.make_inputs(43, [70, 129, 1, 64], h_k=2, h_v=4, dk=64, dv=64, chunk=32, io="bf16")
    say("bf16 boundaries: packing")
    o, pool, _ = _prefill(x)
    for i in range(x.num_seqs):
        t0, t1 = int(x.cu_seqlens[i]), int(x.cu_seqlens[i + 1])
        oi, pi, _ = _prefill(x.select([i]))
        assert sha(oi) == sha(o[t0:t1]) and sha(pi.state[0]) == sha(pool.state[i])


def test_explicit_resync_rounds_in_place():
    cpr = lib()
    x = gi.make_inputs(44, [128, 100], h_k=1, h_v=2, dk=32, dv=32, chunk=64, io="f32")
    say("bf16 boundaries: explicit resync")
    o, pool, _ = _prefill(x)
    before = pool.state.clone()
    cpr.gdn_state_resync(pool, [0, 1])
    torch.cuda.synchronize()
    s0 = pool.state[0].cpu().double().numpy()
    assert np.array_equal(round_to_bf16(before[0].cpu().double().numpy()), s0)   # 128: rounded
    assert sha(pool.state[1]) == sha(before[1])                                   # 100: untouched
    assert pool.boundary_pos.tolist() == [128, -1]
