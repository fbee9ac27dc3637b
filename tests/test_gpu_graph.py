"""Graph capture ("What it actually costs": the method keeps working under graph capture): the
library's calls allocate nothing, never synchronise and record no memset, so a decode step (also
under the R2 reading), a continuation prefill and a trainer step (CPR and chunkwise) captured in a
HIP graph replay to exactly the bytes of eager calls.

Each test replays its graph several times, with eager work and synchronisations between the
replays, and compares every replay with the eager result bit for bit.  The replays cross chunk
starts, so the resynchronisation commit runs inside the graph too.
"""
import pytest
import torch

import gdn_inputs as gi
from tests.gpu_util import lib, policy_of, say, sha

pytestmark = pytest.mark.gpu


def _pools(x, n_slots, boundary):
    cpr = lib()
    pol = policy_of(x)
    return cpr.StatePool(pol, n_slots, boundary=boundary), cpr.StatePool(pol, n_slots, boundary=boundary)


@pytest.mark.parametrize("boundary,record", [("f32", True), ("bf16", True), ("f32", False)])
def test_decode_step_graph_replays_match_eager(boundary, record):
    """One decode step captured and replayed 70 times against eager steps.  fp32 boundaries with
    no boundary record take the uncounted launch shape; the other cases count workgroups."""
    cpr = lib()
    B, steps = 8, 70
    prompts = gi.make_inputs(91, [5, 60, 63, 64, 1, 100, 127, 33], h_k=2, h_v=4, dk=128, dv=128, chunk=64,
                             io="bf16")
    toks = gi.make_inputs(92, [steps] * B, h_k=2, h_v=4, dk=128, dv=128, chunk=64, io="bf16").to("cuda")
    say(f"graph: decode, boundary={boundary}, record={record}")
    pol = cpr.Policy(2, 4, 128, 128, 64, "bf16", boundary=boundary)
    eager = cpr.StatePool(pol, B, boundary=record)
    graphed = cpr.StatePool(pol, B, boundary=record)
    pd = prompts.to("cuda")
    for pool in (eager, graphed):
        cpr.gdn_prefill(pool, prompts.cu_seqlens, pd.q, pd.k, pd.v, pd.a, pd.b)
    torch.cuda.synchronize()
    # step t of slot i is token i * steps + t of the packed decode batch
    idx = lambda t: torch.arange(B, device="cuda") * steps + t
    sq, sk, sv = toks.q[idx(0)].clone(), toks.k[idx(0)].clone(), toks.v[idx(0)].clone()
    sa, sb = toks.a[idx(0)].clone(), toks.b[idx(0)].clone()
    so = torch.empty((B, 4, 128), dtype=torch.bfloat16, device="cuda")
    ids = torch.arange(B, dtype=torch.int32, device="cuda")
    # warm up the capture stream on a throwaway pool, then capture one step on the graphed pool
    scratch = cpr.StatePool(pol, B, boundary=record)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        cpr.gdn_decode_step(scratch, sq, sk, sv, sa, sb, slot_ids=ids, o=so)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cpr.gdn_decode_step(graphed, sq, sk, sv, sa, sb, slot_ids=ids, o=so)
    torch.cuda.synchronize()
    for t in range(steps):
        sq.copy_(toks.q[idx(t)]); sk.copy_(toks.k[idx(t)]); sv.copy_(toks.v[idx(t)])
        sa.copy_(toks.a[idx(t)]); sb.copy_(toks.b[idx(t)])
        g.replay()
        oe = cpr.gdn_decode_step(eager, toks.q[idx(t)], toks.k[idx(t)], toks.v[idx(t)], toks.a[idx(t)],
                                 toks.b[idx(t)], slot_ids=ids)
        torch.cuda.synchronize()
        assert sha(so) == sha(oe), t
        assert sha(graphed.state) == sha(eager.state) and graphed.pos.tolist() == eager.pos.tolist(), t
    if record:
        assert sha(graphed.boundary) == sha(eager.boundary)
        assert graphed.boundary_pos.tolist() == eager.boundary_pos.tolist()


@pytest.mark.parametrize("entry", ["gdn_prefill", "gdn_prefill_fused", "gdn_prefill_overlapped"])
def test_continuation_prefill_graph_replays_match_eager(entry):
    cpr = lib()
    run = getattr(cpr, entry)
    n, reps = 3, 4
    x = gi.make_inputs(93, [40] * n * reps, h_k=2, h_v=4, dk=64, dv=64, chunk=32, io="bf16").to("cuda")
    say(f"graph: continuation prefill ({entry})")
    eager, graphed = _pools(x, n, boundary=False)
    ids = torch.arange(n, dtype=torch.int32, device="cuda")
    cu = torch.tensor([0, 40, 80, 120], dtype=torch.int32, device="cuda")
    part = lambda r: slice(r * n * 40, (r + 1) * n * 40)
    sq, sk, sv = x.q[part(0)].clone(), x.k[part(0)].clone(), x.v[part(0)].clone()
    sa, sb = x.a[part(0)].clone(), x.b[part(0)].clone()
    so = torch.empty((n * 40, 4, 64), dtype=torch.bfloat16, device="cuda")
    rows = cpr.gdn_chunk_rows_bound(n * 40, n, 32)
    cs = torch.empty((rows, 4, 64, 64), device="cuda")
    scratch = cpr.StatePool(policy_of(x), n)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run(scratch, cu, sq, sk, sv, sa, sb, slot_ids=ids, from_state=True, o=so, chunk_states=cs)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(graphed, cu, sq, sk, sv, sa, sb, slot_ids=ids, from_state=True, o=so, chunk_states=cs)
    torch.cuda.synchronize()
    for r in range(reps):
        sq.copy_(x.q[part(r)]); sk.copy_(x.k[part(r)]); sv.copy_(x.v[part(r)])
        sa.copy_(x.a[part(r)]); sb.copy_(x.b[part(r)])
        g.replay()
        oe, _ = cpr.gdn_prefill(eager, cu, x.q[part(r)], x.k[part(r)], x.v[part(r)], x.a[part(r)], x.b[part(r)],
                                slot_ids=ids, from_state=True)
        torch.cuda.synchronize()
        assert sha(so) == sha(oe), r
        assert sha(graphed.state) == sha(eager.state) and graphed.pos.tolist() == eager.pos.tolist() == [40 * (r + 1)] * n


def _capture(fn):
    """fn() once on a side stream (warm-up), then captured into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("evaluation", ["cpr", "native"])
def test_trainer_step_graph_replays_match_eager(evaluation):
    """A trainer step (forward keeping its stash, then the backward) captured once and replayed on
    four batches, each replay against eager calls bit for bit (o and every gradient)."""
    cpr = lib()
    lens, reps = [70, 1, 128, 33], 4
    n = sum(lens)
    batches = [gi.make_inputs(95 + r, lens, h_k=2, h_v=4, dk=64, dv=64, chunk=32, io="bf16").to("cuda")
               for r in range(reps)]
    cts = [gi.make_cotangents(x, 99 + r, device="cuda") for r, x in enumerate(batches)]
    say(f"graph: trainer step ({evaluation})")
    x0 = batches[0]
    P = policy_of(x0)
    B = len(lens)
    cu = torch.from_numpy(x0.cu_seqlens).to("cuda")
    ids = torch.arange(B, dtype=torch.int32, device="cuda")
    st = {k: getattr(x0, k).clone() for k in ("q", "k", "v", "a", "b")}
    sdo, sds = cts[0]["d_o"].clone(), cts[0]["d_state"].clone()
    so = torch.empty((n, 4, 64), dtype=torch.bfloat16, device="cuda")
    cs = torch.empty((cpr.gdn_chunk_rows_bound(n, B, 32), 4, 64, 64), device="cuda")
    grads = {"dq": torch.empty((n, 2, 64), device="cuda"), "dk": torch.empty((n, 2, 64), device="cuda"),
             "dv": torch.empty((n, 4, 64), device="cuda"), "da": torch.empty((n, 4), device="cuda"),
             "db": torch.empty((n, 4), device="cuda")}
    pool = cpr.StatePool(P, B)
    if evaluation == "cpr":
        cw = torch.empty((2, n, 4, 64), device="cuda")
        ws = torch.empty(cpr.gdn_backward_workspace_bytes(P, n, B), dtype=torch.uint8, device="cuda")

        def step():
            cpr.gdn_trainer_forward(pool, cu, st["q"], st["k"], st["v"], st["a"], st["b"], slot_ids=ids, o=so,
                                    chunk_states=cs, cw=cw)
            cpr.gdn_backward(P, cu, st["q"], st["k"], st["v"], st["a"], st["b"], cs, sdo, d_state=sds,
                             workspace=ws, out=grads, cw=cw)
    else:
        stash = torch.empty(cpr.gdn_trainer_forward_chunked_stash_bytes(P, n, B), dtype=torch.uint8, device="cuda")
        ws = torch.empty(cpr.gdn_backward_chunked_workspace_bytes(P, n, B), dtype=torch.uint8, device="cuda")

        def step():
            cpr.gdn_trainer_forward_chunked(pool, cu, st["q"], st["k"], st["v"], st["a"], st["b"], slot_ids=ids,
                                            o=so, chunk_states=cs, stash=stash)
            cpr.gdn_backward_chunked(P, cu, st["q"], st["k"], st["v"], st["a"], st["b"], cs, stash, sdo,
                                     d_state=sds, workspace=ws, out=grads)
    g = _capture(step)
    for r, (x, ct) in enumerate(zip(batches, cts)):
        for k in st:
            st[k].copy_(getattr(x, k))
        sdo.copy_(ct["d_o"]); sds.copy_(ct["d_state"])
        g.replay()
        torch.cuda.synchronize()
        got = {k: sha(v) for k, v in grads.items()}
        got_o = sha(so)
        ep = cpr.StatePool(P, B)
        if evaluation == "cpr":
            o, ecs, ecw = cpr.gdn_trainer_forward(ep, x.cu_seqlens, x.q, x.k, x.v, x.a, x.b)
            ref = cpr.gdn_backward(P, x.cu_seqlens, x.q, x.k, x.v, x.a, x.b, ecs, ct["d_o"], d_state=ct["d_state"],
                                   cw=ecw)
        else:
            o, ecs, estash = cpr.gdn_trainer_forward_chunked(ep, x.cu_seqlens, x.q, x.k, x.v, x.a, x.b)
            ref = cpr.gdn_backward_chunked(P, x.cu_seqlens, x.q, x.k, x.v, x.a, x.b, ecs, estash, ct["d_o"],
                                           d_state=ct["d_state"])
        torch.cuda.synchronize()
        assert got_o == sha(o), r
        for k in grads:
            assert got[k] == sha(ref[k]), (r, k)


def test_r2_decode_step_graph_replays_match_eager():
    """An R2 decode step (chunk-form resynchronisation over the listed slots at a chunk start, the
    pinned step, the ring append) captured once and replayed across chunk starts against eager
    steps on a twin pool, bit for bit."""
    cpr = lib()
    B, steps, C = 6, 40, 16
    prompts = gi.make_inputs(101, [16, 1, 30, 32, 5, 47], h_k=2, h_v=4, dk=32, dv=32, chunk=C, io="bf16")
    toks = gi.make_inputs(102, [steps] * B, h_k=2, h_v=4, dk=32, dv=32, chunk=C, io="bf16").to("cuda")
    say("graph: R2 decode step")
    P = policy_of(prompts)
    pools = []
    pd = prompts.to("cuda")
    for _ in range(2):
        pool = cpr.StatePool(P, B, boundary=True)
        pool.attach_r2()
        cpr.gdn_prefill_chunked(pool, prompts.cu_seqlens, pd.q, pd.k, pd.v, pd.a, pd.b,
                                outputs=cpr.GDN_CHUNKED_R2)
        pools.append(pool)
    eager, graphed = pools
    torch.cuda.synchronize()
    idx = lambda t: torch.arange(B, device="cuda") * steps + t
    sq, sk, sv = toks.q[idx(0)].clone(), toks.k[idx(0)].clone(), toks.v[idx(0)].clone()
    sa, sb = toks.a[idx(0)].clone(), toks.b[idx(0)].clone()
    so = torch.empty((B, 4, 32), dtype=torch.bfloat16, device="cuda")
    ids = torch.arange(B, dtype=torch.int32, device="cuda")
    scratch = cpr.StatePool(P, B, boundary=True)
    scratch.attach_r2()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        cpr.gdn_decode_step(scratch, sq, sk, sv, sa, sb, slot_ids=ids, o=so)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cpr.gdn_decode_step(graphed, sq, sk, sv, sa, sb, slot_ids=ids, o=so)
    torch.cuda.synchronize()
    for t in range(steps):
        sq.copy_(toks.q[idx(t)]); sk.copy_(toks.k[idx(t)]); sv.copy_(toks.v[idx(t)])
        sa.copy_(toks.a[idx(t)]); sb.copy_(toks.b[idx(t)])
        g.replay()
        oe = cpr.gdn_decode_step(eager, toks.q[idx(t)], toks.k[idx(t)], toks.v[idx(t)], toks.a[idx(t)],
                                 toks.b[idx(t)], slot_ids=ids)
        torch.cuda.synchronize()
        assert sha(so) == sha(oe), t
        assert sha(graphed.state) == sha(eager.state) and graphed.pos.tolist() == eager.pos.tolist(), t
    assert sha(graphed.boundary) == sha(eager.boundary)
