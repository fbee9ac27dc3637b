"""The chunkwise (WY/UT) evaluation on matrix cores (gdn_prefill_chunked), both output modes,
against the fp64 oracle; and the R2 reading's defining properties.

Tolerance: the bf16-io bound, normwise 3e-3 per (sequence, value head) block, on o, the final
state and every chunk-start state.  The chunk form is not bit-identical to the recurrence: its
products run on bf16 matrix cores with split (high + low bf16) operands and fp32 accumulation,
so it agrees to fp32-level rounding before o is rounded to bf16.

R2: the chunk form gives the states at chunk starts, the pinned per-token step gives everything
in between.  So (1) R2's o for a chunk is bit for bit what the CPR path produces when started
from R2's state at that chunk start, which is what a decode produces between chunk starts;
(2) at a chunk start such a decode resynchronises by re-running the chunk form over the chunk it
just finished, from the previous chunk-start state (the native mode's final state), and lands
exactly on R2's next chunk-start state; (3) R2's chunk-start states differ from the per-token
ones (the resynchronisation changes values), while both stay within tolerance of the oracle.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
from tests.gpu_util import gpu_state_math, lib, normwise, oracle_seq_head, policy_of, say, sha

pytestmark = pytest.mark.gpu
TOL = 3e-3


def _chunked(x, outputs, pool=None, from_state=False):
    cpr = lib()
    xd = x.to("cuda")
    pool = pool or cpr.StatePool(policy_of(x), max(x.num_seqs, 1))
    o, cs = cpr.gdn_prefill_chunked(pool, x.cu_seqlens, xd.q, xd.k, xd.v, xd.a, xd.b, from_state=from_state,
                                    outputs=outputs)
    torch.cuda.synchronize()
    return o, pool, cs


def _check_vs_oracle(x, o, pool, cs, S0=None, pos0=None):
    cpr = lib()
    rows = cpr.gdn_chunk_rows(x.cu_seqlens, x.chunk, pos0).numpy()
    o_np = o.float().cpu().double().numpy()
    for i in range(x.num_seqs):
        t0, t1 = int(x.cu_seqlens[i]), int(x.cu_seqlens[i + 1])
        for h in range(x.h_v):
            ref_o, ref_S, ref_R = oracle_seq_head(x, i, h, S0=None if S0 is None else S0[i, h].T,
                                                  pos0=0 if pos0 is None else int(pos0[i]))
            if t1 > t0:
                assert normwise(o_np[t0:t1, h], ref_o) <= TOL, (i, h, "o")
            assert normwise(gpu_state_math(pool, i, h), ref_S) <= TOL, (i, h, "S")
            for r in range(len(ref_R)):
                got = cs[rows[i] + r, h].cpu().double().numpy().T
                assert normwise(got, ref_R[r]) <= TOL, (i, h, "row", r)


@pytest.mark.parametrize("dim,chunk", [(32, 64), (64, 32), (128, 64), (128, 20)])
@pytest.mark.parametrize("mode", ["native", "r2"])
def test_chunked_matches_oracle(dim, chunk, mode):
    cpr = lib()
    outputs = cpr.GDN_CHUNKED_NATIVE if mode == "native" else cpr.GDN_CHUNKED_R2
    lens = [1, 64, 65, 200, 0, 33]
    x = gi.make_inputs(81, lens, h_k=2, h_v=4, dk=dim, dv=dim, chunk=chunk, io="bf16")
    say(f"chunked {mode} vs oracle dim={dim} C={chunk}")
    o, pool, cs = _chunked(x, outputs)
    _check_vs_oracle(x, o, pool, cs)


@pytest.mark.parametrize("mode", ["native", "r2"])
def test_chunked_continuation_from_state(mode):
    cpr = lib()
    outputs = cpr.GDN_CHUNKED_NATIVE if mode == "native" else cpr.GDN_CHUNKED_R2
    x = gi.make_inputs(82, [150, 64, 7], h_k=2, h_v=4, dk=64, dv=64, chunk=64, io="bf16")
    ct = gi.make_cotangents(x, 83, with_d_state=False, with_s0=True)
    pos0 = [37, 64, 0]
    say(f"chunked {mode} continuation")
    pool = cpr.StatePool(policy_of(x), x.num_seqs)
    pool.state.copy_(ct["s0"].to("cuda"))
    pool.pos.copy_(torch.tensor(pos0, dtype=torch.int64))
    o, pool, cs = _chunked(x, outputs, pool=pool, from_state=True)
    _check_vs_oracle(x, o, pool, cs, S0=ct["s0"].double().numpy(), pos0=pos0)
    assert pool.pos.tolist() == [p + int(n) for p, n in zip(pos0, x.lengths)]


@pytest.mark.parametrize("mode", ["native", "r2"])
def test_chunked_packing_invariance(mode):
    cpr = lib()
    outputs = cpr.GDN_CHUNKED_NATIVE if mode == "native" else cpr.GDN_CHUNKED_R2
    x = gi.make_inputs(84, [130, 1, 64, 77], h_k=2, h_v=4, dk=128, dv=128, chunk=64, io="bf16")
    say(f"chunked {mode} packing")
    o, pool, cs = _chunked(x, outputs)
    for i in range(x.num_seqs):
        t0, t1 = int(x.cu_seqlens[i]), int(x.cu_seqlens[i + 1])
        oi, pi, _ = _chunked(x.select([i]), outputs)
        assert sha(oi) == sha(o[t0:t1]) and sha(pi.state[0]) == sha(pool.state[i]), i


def test_r2_outputs_are_the_per_token_step_from_chunk_form_states():
    """(1), (2) and (3) of the module docstring on one 300-token sequence."""
    cpr = lib()
    x = gi.make_inputs(85, [300], h_k=2, h_v=4, dk=128, dv=128, chunk=64, io="bf16")
    say("R2 structure")
    o, pool, cs = _chunked(x, cpr.GDN_CHUNKED_R2)
    C = x.chunk
    # per-token prefill started from R2's chunk-start state reproduces R2's o and final state
    for c in range(300 // C + 1):
        t0, t1 = c * C, min(300, (c + 1) * C)
        part = x.token_slice(t0, t1)
        pc = cpr.StatePool(policy_of(x), 1)
        pc.state[0].copy_(cs[c])
        pc.pos.fill_(t0)
        pd = part.to("cuda")
        oc, _ = cpr.gdn_prefill(pc, part.cu_seqlens, pd.q, pd.k, pd.v, pd.a, pd.b, from_state=True)
        torch.cuda.synchronize()
        assert sha(oc) == sha(o[t0:t1]), c
        if t1 == 300:
            assert sha(pc.state[0]) == sha(pool.state[0])
    # the resynchronisation a decode performs at a chunk start: the chunk form re-run over the
    # chunk just finished, from the previous chunk-start state, lands exactly on R2's state
    for c in range(300 // C):
        part = x.token_slice(c * C, (c + 1) * C)
        pc = cpr.StatePool(policy_of(x), 1)
        pc.state[0].copy_(cs[c])
        pc.pos.fill_(c * C)
        pd = part.to("cuda")
        cpr.gdn_prefill_chunked(pc, part.cu_seqlens, pd.q, pd.k, pd.v, pd.a, pd.b, from_state=True,
                                outputs=cpr.GDN_CHUNKED_NATIVE)
        torch.cuda.synchronize()
        assert sha(pc.state[0]) == sha(cs[c + 1]), c
    # the chunk-form states differ from the per-token (CPR) states at every chunk start after 0
    ref_pool = cpr.StatePool(policy_of(x), 1)
    xd = x.to("cuda")
    _, cs_cpr = cpr.gdn_prefill(ref_pool, x.cu_seqlens, xd.q, xd.k, xd.v, xd.a, xd.b)
    torch.cuda.synchronize()
    assert sha(cs[0]) == sha(cs_cpr[0])
    for c in range(1, 300 // C + 1):
        assert sha(cs[c]) != sha(cs_cpr[c]), c
        assert normwise(cs[c].cpu().double().numpy(), cs_cpr[c].cpu().double().numpy()) <= TOL


def test_chunked_prefill_5x2048_sampled():
    """The 5 x 2048 rollout workload through both modes: oracle samples on two (sequence, value
    head) pairs per sequence, finite everywhere."""
    cpr = lib()
    x = gi.prefill_5x2048(device="cuda")
    for mode, outputs in (("native", cpr.GDN_CHUNKED_NATIVE), ("r2", cpr.GDN_CHUNKED_R2)):
        say(f"chunked {mode} 5x2048")
        o, pool, cs = _chunked(x, outputs)
        assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(pool.state).all())
        o_np = None
        for i in range(x.num_seqs):
            t0, t1 = int(x.cu_seqlens[i]), int(x.cu_seqlens[i + 1])
            for h in (3 * i % 32, (7 * i + 19) % 32):
                ref_o, ref_S, _ = oracle_seq_head(x, i, h)
                o_np = o[t0:t1, h].float().cpu().double().numpy()
                assert normwise(o_np, ref_o) <= TOL, (mode, i, h)
                assert normwise(gpu_state_math(pool, i, h), ref_S) <= TOL, (mode, i, h)


def test_chunked_rejects_unsupported_policies():
    cpr = lib()
    x = gi.make_inputs(86, [10], h_k=1, h_v=1, dk=32, dv=32, chunk=64, io="f32")
    pool = cpr.StatePool(policy_of(x), 1)
    xd = x.to("cuda")
    with pytest.raises(cpr.GdnError) as e:
        cpr.gdn_prefill_chunked(pool, x.cu_seqlens, xd.q, xd.k, xd.v, xd.a, xd.b)
    assert e.value.code == cpr.GDN_EUNSUPPORTED


def _prompt_plus_generated(prompts: gi.GdnInputs, steps, order):
    """Each sequence's prompt followed by its generated tokens; steps[s] holds the token of slot
    order[s][j] in row j."""
    n, T = prompts.num_seqs, len(steps)
    L = prompts.lengths
    cu = gi.cu_from_lengths(L + T)
    parts = {}
    for name in ("q", "k", "v", "a", "b"):
        p = getattr(prompts, name)
        out = torch.empty((int(cu[-1]),) + tuple(p.shape[1:]), dtype=p.dtype, device=p.device)
        for i in range(n):
            o0, p0 = int(cu[i]), int(prompts.cu_seqlens[i])
            out[o0:o0 + L[i]] = p[p0:p0 + L[i]]
        for s, st in enumerate(steps):
            rows = getattr(st, name)
            for j, i in enumerate(order[s]):
                out[int(cu[i]) + L[i] + s] = rows[j]
        parts[name] = out
    return gi.GdnInputs("prompt+generated", prompts.h_k, prompts.h_v, prompts.dk, prompts.dv, prompts.chunk,
                        prompts.io, cu, *(parts[nm] for nm in ("q", "k", "v", "a", "b")))


@pytest.mark.parametrize("dim,chunk,cap", [(32, 16, 0), (128, 64, 0), (128, 64, 7)])
def test_r2_decode_equals_one_chunked_r2_prefill(dim, chunk, cap):
    """R2 inside gdn_decode_step: prompts prefilled with gdn_prefill_chunked(R2) into a pool with R2
    attached, then decode steps that cross several chunk starts (slots listed in a different order
    every step): every decode output and the final states equal, bit for bit, one chunked R2
    prefill over prompt and generated tokens; the boundary record holds R2's last chunk-start state.
    The resynchronisation changes values (an R1 decode of the same tokens differs), and the
    outputs stay within the bf16 tolerance of the oracle.  With cap > 0 the decode steps run under
    that workgroup cap (the listed slots' step and the others' step then take their items in
    turn), with the same bits."""
    cpr = lib()
    lens = [chunk, 1, 100, 2 * chunk, 37, 3 * chunk + 5]
    T = 2 * chunk + 11
    prompts = gi.make_inputs(41, lens, h_k=2, h_v=4, dk=dim, dv=dim, chunk=chunk, io="bf16", device="cuda")
    steps = [gi.make_inputs(41, [1] * len(lens), h_k=2, h_v=4, dk=dim, dv=dim, chunk=chunk, io="bf16",
                            sub=300 + s, device="cuda") for s in range(T)]
    rng = np.random.default_rng(41)
    order = [rng.permutation(len(lens)).tolist() for _ in range(T)]
    P = policy_of(prompts)
    say(f"R2 decode dim={dim} C={chunk} cap={cap}: prompts {lens}, {T} steps")
    pool = cpr.StatePool(P, len(lens), boundary=True)
    pool.attach_r2()
    cpr.gdn_prefill_chunked(pool, prompts.cu_seqlens, prompts.q, prompts.k, prompts.v, prompts.a, prompts.b,
                            outputs=cpr.GDN_CHUNKED_R2)
    r1 = cpr.StatePool(P, len(lens), boundary=True)
    cpr.gdn_prefill_chunked(r1, prompts.cu_seqlens, prompts.q, prompts.k, prompts.v, prompts.a, prompts.b,
                            outputs=cpr.GDN_CHUNKED_R2)
    if cap:
        pool.set_max_workgroups(cap)
    outs = torch.empty((len(lens), T, P.h_v, P.dv), dtype=torch.bfloat16, device="cuda")
    outs_r1 = torch.empty_like(outs)
    for s, st in enumerate(steps):
        ids = torch.tensor(order[s], dtype=torch.int32, device="cuda")
        o = cpr.gdn_decode_step(pool, st.q, st.k, st.v, st.a, st.b, slot_ids=ids)
        o1 = cpr.gdn_decode_step(r1, st.q, st.k, st.v, st.a, st.b, slot_ids=ids)
        outs[ids.long(), s] = o
        outs_r1[ids.long(), s] = o1
    torch.cuda.synchronize()
    assert pool.pos.tolist() == [L + T for L in lens]
    say(f"R2 decode dim={dim} C={chunk}: one chunked R2 prefill over prompt and generated tokens")
    full = _prompt_plus_generated(prompts, steps, order)
    ref = cpr.StatePool(P, len(lens))
    o_full, _ = cpr.gdn_prefill_chunked(ref, full.cu_seqlens, full.q, full.k, full.v, full.a, full.b,
                                        outputs=cpr.GDN_CHUNKED_R2)
    torch.cuda.synchronize()
    for i in range(len(lens)):
        t1 = int(full.cu_seqlens[i + 1])
        assert sha(outs[i]) == sha(o_full[t1 - T:t1]), f"slot {i}"
    assert sha(pool.state) == sha(ref.state)
    bpos = pool.boundary_pos.tolist()
    assert bpos == [(L + T - 1) // chunk * chunk for L in lens]
    assert sha(outs_r1) != sha(outs)                    # R1's per-token chunk starts differ from R2's
    for i in (0, 5):
        for h in (0, 3):
            ref_o, ref_S, _ = oracle_seq_head(full, i, h)
            assert normwise(outs[i, :, h].float().cpu().double().numpy(), ref_o[-T:]) <= TOL
            assert normwise(gpu_state_math(pool, i, h), ref_S) <= TOL
