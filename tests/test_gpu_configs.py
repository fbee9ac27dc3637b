"""GPU parity and identity at the workloads' full sizes, in the launch configuration the
benchmark times.  The oracle checks every (sequence, value head) pair of the prefill, decode,
trainer and long workloads (in a host process pool), element by element against a forward error
bound of the fp32 arithmetic (tests/bf16_check.py) besides the normwise tolerance; identity is
checked on every output byte with SHA-256.

  prefill   5 x 2048 tokens, 32 value heads over 16 key heads, d = 128, chunk 64, bf16
  decode    256 slots seeded by ragged prompts (1..2048 tokens), 128 steps, resync every 64
  trainer   10240 tokens packed varlen (lengths 64..4096), boundary states stashed
  long      one 65536-token sequence alone, among neighbours, at other chunk sizes, and decoded
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
from tests.gpu_util import (check_close, gpu_state_math, lib, oracle_items, oracle_seq_head, policy_of, prefill,
                            run_oracle_checks, say, sha)

pytestmark = pytest.mark.gpu


def _decode_seq(pool, x, slot=0, on_step=None):
    """Decode the single sequence x token by token into `slot`; returns o [T, H_v, dv]."""
    cpr = lib()
    xd = x.to("cuda")
    ids = torch.tensor([slot], dtype=torch.int32, device="cuda")
    out = torch.empty((x.total_tokens, x.h_v, x.dv), dtype=xd.v.dtype, device="cuda")
    for t in range(x.total_tokens):
        cpr.gdn_decode_step(pool, xd.q[t:t + 1], xd.k[t:t + 1], xd.v[t:t + 1], xd.a[t:t + 1], xd.b[t:t + 1],
                            slot_ids=ids, o=out[t:t + 1])
        if on_step is not None:
            on_step(t)
    torch.cuda.synchronize()
    return out


def test_prefill_5x2048():
    cpr = lib()
    x = gi.prefill_5x2048(device="cuda")
    say("prefill 5x2048: packed run")
    o, pool, cs = prefill(x)
    rows = cpr.gdn_chunk_rows(x.cu_seqlens, 64).numpy()
    # every (sequence, value head): o element by element, the final state column by column, and
    # every chunk-start row
    tot = run_oracle_checks(oracle_items(x, o, pool.state, chunk_states=cs), "prefill 5x2048")
    assert tot["elements"] == x.total_tokens * x.h_v * x.dv
    assert tot["ulp0"] >= 0.999 * tot["elements"]       # round to nearest even: nearly all outputs exact
    say("prefill 5x2048: sequence 2 alone")
    o2, pool2, _ = prefill(x.select([2]))
    assert sha(o2) == sha(o[int(x.cu_seqlens[2]):int(x.cu_seqlens[3])])
    assert sha(pool2.state[0]) == sha(pool.state[2])
    say("prefill 5x2048: sequence 4 decoded token by token")
    dpool = cpr.StatePool(policy_of(x), 1, boundary=True)
    seen = []

    def check_boundary(t):
        if t % 64 == 0:                      # the step at a chunk start committed its state
            seen.append(sha(dpool.boundary[0]) == sha(cs[rows[4] + t // 64]))

    od = _decode_seq(dpool, x.select([4]), on_step=check_boundary)
    assert sha(od) == sha(o[int(x.cu_seqlens[4]):])
    assert sha(dpool.state[0]) == sha(pool.state[4])
    assert len(seen) == 32 and all(seen)


def _with_generated(prompts: gi.GdnInputs, steps):
    """Pack each sequence's prompt followed by its generated tokens (one per decode step)."""
    n = prompts.num_seqs
    L = prompts.lengths
    T = len(steps)
    dec = {name: torch.stack([getattr(s, name) for s in steps]) for name in ("q", "k", "v", "a", "b")}
    idx_p, idx_d = [], []
    out_len = L + T
    cu = gi.cu_from_lengths(out_len)
    total = int(cu[-1])
    src_prompt = torch.full((total,), -1, dtype=torch.int64)
    src_step = torch.full((total,), -1, dtype=torch.int64)
    for i in range(n):
        o0 = int(cu[i])
        p0 = int(prompts.cu_seqlens[i])
        src_prompt[o0:o0 + L[i]] = torch.arange(p0, p0 + L[i])
        src_step[o0 + L[i]:o0 + L[i] + T] = torch.arange(T) * n + i
    dev = prompts.device
    src_prompt, src_step = src_prompt.to(dev), src_step.to(dev)
    is_p = src_prompt >= 0

    def gather(name):
        p = getattr(prompts, name)
        d = dec[name].reshape((T * n,) + tuple(p.shape[1:]))
        out = torch.empty((total,) + tuple(p.shape[1:]), dtype=p.dtype, device=dev)
        out[is_p] = p[src_prompt[is_p]]
        out[~is_p] = d[src_step[~is_p]]
        return out

    return gi.GdnInputs("prompt+generated", prompts.h_k, prompts.h_v, prompts.dk, prompts.dv, prompts.chunk,
                        prompts.io, cu, gather("q"), gather("k"), gather("v"), gather("a"), gather("b"))


def test_decode_256x1_128_steps_equals_one_prefill():
    cpr = lib()
    prompts = gi.decode_prompts(device="cuda")
    n = prompts.num_seqs
    say(f"decode: prefill {n} prompts ({prompts.total_tokens} tokens)")
    P = policy_of(prompts)
    pool = cpr.StatePool(P, n, boundary=True)
    cpr.gdn_prefill(pool, prompts.cu_seqlens, prompts.q, prompts.k, prompts.v, prompts.a, prompts.b)
    start_state = pool.state.clone()
    steps = [gi.decode_tokens(s, n, device="cuda") for s in range(128)]
    say("decode: 128 steps")
    outs = []
    for s in steps:
        outs.append(cpr.gdn_decode_step(pool, s.q, s.k, s.v, s.a, s.b))
    torch.cuda.synchronize()
    L = prompts.lengths
    assert pool.pos.cpu().numpy().tolist() == (L + 128).tolist()
    # every slot resynchronised at its last chunk start inside the decoded range, if any
    bp = pool.boundary_pos.cpu().numpy()
    for i in range(n):
        starts = [p for p in range(int(L[i]), int(L[i]) + 128) if p % 64 == 0]
        assert bp[i] == (starts[-1] if starts else -1)
    say("decode: one packed prefill over prompt + generated tokens")
    full = _with_generated(prompts, steps)
    o_full, pool_full, cs_full = prefill(full)
    dec_o = torch.stack(outs, dim=1)                    # [n, 128, H_v, dv]
    for i in range(n):
        t1 = int(full.cu_seqlens[i + 1])
        assert sha(dec_o[i]) == sha(o_full[t1 - 128:t1]), f"slot {i}"
    assert sha(pool.state) == sha(pool_full.state)
    rows = cpr.gdn_chunk_rows(full.cu_seqlens, 64).numpy()
    for i in range(n):
        if bp[i] >= 0:
            assert sha(pool.boundary[i]) == sha(cs_full[rows[i] + bp[i] // 64]), f"boundary {i}"
    for (i, h) in [(int(np.argmin(L)), 3), (int(np.argmax(L)), 30)]:
        say(f"decode: oracle slot {i} head {h} over prompt and generated tokens")
        ref_o, ref_S, _ = oracle_seq_head(full, i, h)
        check_close("bf16", dec_o[i, :, h].float().cpu().numpy(), ref_o[-128:], f"decode o slot {i}")
        check_close("bf16", gpu_state_math(pool, i, h), ref_S, f"decode S slot {i}")
    # every (slot, value head): the oracle continues from the state the prefill left in the slot
    # (fp32, exact in fp64) over the 128 generated tokens, against every decode output
    gen = gi.GdnInputs("decode", P.h_k, P.h_v, P.dk, P.dv, 64, "bf16", gi.cu_from_lengths([128] * n),
                       *(torch.stack([getattr(s, f) for s in steps], dim=1).reshape(
                           (n * 128,) + tuple(getattr(steps[0], f).shape[1:])) for f in ("q", "k", "v", "a", "b")))
    tot = run_oracle_checks(oracle_items(gen, dec_o.reshape(n * 128, P.h_v, P.dv), pool.state, S0=start_state,
                                         pos0=L.tolist()), "decode 256x128")
    assert tot["elements"] == n * 128 * P.h_v * P.dv


def test_trainer_forward_10240_varlen_with_stash():
    cpr = lib()
    x = gi.trainer_10240(device="cuda")
    say(f"trainer: lengths {list(x.lengths)}")
    rows = cpr.gdn_chunk_rows(x.cu_seqlens, 64).numpy()
    stash = torch.empty((int(rows[-1]) + 2 * x.num_seqs + x.total_tokens // 64, x.h_v, x.dv, x.dk),
                        dtype=torch.float32, device="cuda")
    o, pool, cs = prefill(x, chunk_states=stash)
    assert cs is stash
    tot = run_oracle_checks(oracle_items(x, o, pool.state, chunk_states=stash), "trainer 10240")
    assert tot["elements"] == x.total_tokens * x.h_v * x.dv
    for i in range(x.num_seqs):
        say(f"trainer: sequence {i} alone")
        oi, pi, ci = prefill(x.select([i]))
        t0, t1 = int(x.cu_seqlens[i]), int(x.cu_seqlens[i + 1])
        assert sha(oi) == sha(o[t0:t1])
        assert sha(ci[:rows[i + 1] - rows[i]]) == sha(stash[rows[i]:rows[i + 1]])
    i = int(np.argmin(x.lengths))
    say(f"trainer: sequence {i} replayed by decode")
    dpool = cpr.StatePool(policy_of(x), 1, boundary=True)
    ok = []
    _decode_seq(dpool, x.select([i]),
                on_step=lambda t: ok.append(sha(dpool.boundary[0]) == sha(stash[rows[i] + t // 64]))
                if t % 64 == 0 else None)
    assert ok and all(ok)
    assert sha(dpool.state[0]) == sha(pool.state[i])


@pytest.fixture(scope="module")
def long_x():
    x = gi.long_sequence(device="cuda")
    say("long: X alone")
    o, pool, _ = prefill(x)
    return x, sha(o), sha(pool.state), o


def test_long_sequence_matches_oracle(long_x):
    """Every value head of the 65536-token sequence against the oracle, element by element."""
    x, _, _, o = long_x
    pool = lib().StatePool(policy_of(x), 1)
    o2, pool, _ = prefill(x, pool=pool)
    assert sha(o2) == sha(o)
    tot = run_oracle_checks(oracle_items(x, o, pool.state), "long 65536")
    assert tot["elements"] == x.total_tokens * x.h_v * x.dv


@pytest.mark.parametrize("cap", [1, 7, 64, 4096])
def test_long_sequence_among_neighbours_under_a_grid_cap(long_x, cap):
    """X packed among 7 random neighbours with every compute kernel capped at `cap` workgroups
    ("Making kernels parallelism-invariant": identical bits however the work is split and whatever
    shares the launch): X's o and final state equal those of X alone, bit for bit, and the
    neighbours' equal their uncapped run."""
    x, so, sS, _ = long_x
    y, pos = gi.long_in_batch(x, 8, sub=100 + cap)
    say(f"long: X among 7 neighbours at position {pos} under a grid cap of {cap}")
    ref_o, ref_pool, _ = prefill(y)
    pool = lib().StatePool(policy_of(y), y.num_seqs)
    pool.set_max_workgroups(cap)
    o, pool, _ = prefill(y, pool=pool)
    t0 = int(y.cu_seqlens[pos])
    assert sha(o[t0:t0 + x.total_tokens]) == so
    assert sha(pool.state[pos:pos + 1]) == sS
    assert sha(o) == sha(ref_o) and sha(pool.state) == sha(ref_pool.state)


@pytest.mark.parametrize("batch", [2, 4, 8, 16, 32, 64])
def test_long_sequence_invariant_to_neighbours(long_x, batch):
    x, so, sS, _ = long_x
    y, pos = gi.long_in_batch(x, batch, sub=batch)
    say(f"long: X among {batch - 1} neighbours at position {pos} ({y.total_tokens} tokens)")
    o, pool, _ = prefill(y)
    t0 = int(y.cu_seqlens[pos])
    assert sha(o[t0:t0 + x.total_tokens]) == so
    assert sha(pool.state[pos:pos + 1]) == sS


@pytest.mark.parametrize("chunk", [16, 32, 128, 1024])
def test_long_sequence_invariant_to_chunk(long_x, chunk):
    x, so, sS, _ = long_x
    say(f"long: chunk {chunk}")
    o, pool, _ = prefill(x, chunk=chunk)
    assert sha(o) == so and sha(pool.state) == sS


def test_long_sequence_overlapped(long_x):
    x, so, sS, _ = long_x
    say("long: overlapped prefill")
    cpr = lib()
    pool = cpr.StatePool(policy_of(x), 1)
    xd = x.to("cuda")
    o, _ = cpr.gdn_prefill_overlapped(pool, x.cu_seqlens, xd.q, xd.k, xd.v, xd.a, xd.b)
    torch.cuda.synchronize()
    assert sha(o) == so and sha(pool.state) == sS


@pytest.mark.parametrize("cap", [1, 7, 64, 256, 1024, 4096])
def test_long_sequence_under_a_grid_cap(long_x, cap):
    """X through the two-pass prefill with the compute kernels capped at `cap` workgroups, each
    taking work items in turn ("Making kernels parallelism-invariant": identical bits however the
    work is split): the natural launch's o and final S, bit for bit."""
    x, so, sS, _ = long_x
    say(f"long: two-pass prefill under a grid cap of {cap}")
    pool = lib().StatePool(policy_of(x), 1)
    pool.set_max_workgroups(cap)
    o, pool, _ = prefill(x, pool=pool)
    assert sha(o) == so and sha(pool.state) == sS


@pytest.mark.parametrize("cap", [7, 100])
def test_long_sequence_one_pass_and_overlapped_under_a_grid_cap(long_x, cap):
    x, so, sS, _ = long_x
    cpr = lib()
    xd = x.to("cuda")
    for run in (cpr.gdn_prefill_fused, cpr.gdn_prefill_overlapped):
        say(f"long: {run.__name__} under a grid cap of {cap}")
        pool = cpr.StatePool(policy_of(x), 1)
        pool.set_max_workgroups(cap)
        o, _ = run(pool, x.cu_seqlens, xd.q, xd.k, xd.v, xd.a, xd.b)
        torch.cuda.synchronize()
        assert sha(o) == so and sha(pool.state) == sS


@pytest.mark.parametrize("record", [True, False])
@pytest.mark.parametrize("cap", [1, 7, 64])
def test_decode_under_a_grid_cap(cap, record):
    """Ragged prompts, then 70 decode steps that cross chunk starts, with the decode step capped
    at `cap` workgroups: every output, state, position and boundary record as in the natural
    launch.  With a boundary record every workgroup reads the slot's position and a second kernel
    advances it after the step; without one (fp32 boundaries) no workgroup reads the position and
    one workgroup per slot advances it.  The sequences live in a permuted subset of a larger pool,
    so three slots are never listed and must stay untouched."""
    cpr = lib()
    lens = [(53 * i) % 190 + 1 for i in range(16)]
    prompts = gi.make_inputs(31, lens, io="bf16", device="cuda", **gi.BIG)
    steps = [gi.make_inputs(31, [1] * len(lens), io="bf16", sub=500 + s, device="cuda", **gi.BIG) for s in range(70)]
    n_slots = len(lens) + 3
    ids = torch.tensor([(7 * i + 5) % n_slots for i in range(len(lens))], dtype=torch.int32, device="cuda")
    assert len(set(ids.tolist())) == len(lens)
    say(f"decode under a grid cap of {cap}, boundary record {record}")
    runs = []
    for c in (0, cap):
        pool = cpr.StatePool(policy_of(prompts), n_slots, boundary=record)
        cpr.gdn_prefill(pool, prompts.cu_seqlens, prompts.q, prompts.k, prompts.v, prompts.a, prompts.b,
                        slot_ids=ids)
        pool.set_max_workgroups(c)
        outs = [cpr.gdn_decode_step(pool, s.q, s.k, s.v, s.a, s.b, slot_ids=ids) for s in steps]
        torch.cuda.synchronize()
        pos = pool.pos.tolist()
        assert [pos[i] for i in ids.tolist()] == [L + len(steps) for L in lens]
        unlisted = sorted(set(range(n_slots)) - set(ids.tolist()))
        assert [pos[i] for i in unlisted] == [0] * 3
        assert not pool.state[unlisted].any()
        runs.append((sha(torch.stack(outs)), sha(pool.state), pos,
                     sha(pool.boundary) if record else None, pool.boundary_pos.tolist() if record else None))
    assert runs[0] == runs[1]


def test_decode_counted_and_uncounted_shapes_agree():
    """The same prompts and 70 decode steps through a pool with a boundary record (every workgroup
    reads the position; a second kernel advances it) and one without (no position read; one
    workgroup per slot advances it): outputs, states and positions are equal bit for bit, and the
    record holds each slot's last chunk-start state."""
    cpr = lib()
    lens = [(71 * i) % 300 + 1 for i in range(24)]
    prompts = gi.make_inputs(33, lens, io="bf16", device="cuda", **gi.BIG)
    steps = [gi.make_inputs(33, [1] * len(lens), io="bf16", sub=700 + s, device="cuda", **gi.BIG) for s in range(70)]
    say("decode: counted and uncounted launch shapes")
    runs = []
    for record in (True, False):
        pool = cpr.StatePool(policy_of(prompts), len(lens), boundary=record)
        cpr.gdn_prefill(pool, prompts.cu_seqlens, prompts.q, prompts.k, prompts.v, prompts.a, prompts.b)
        outs = [cpr.gdn_decode_step(pool, s.q, s.k, s.v, s.a, s.b) for s in steps]
        torch.cuda.synchronize()
        runs.append((sha(torch.stack(outs)), sha(pool.state), pool.pos.tolist()))
        if record:
            bpos = pool.boundary_pos.tolist()
            assert bpos == [(L + len(steps) - 1) // 64 * 64 for L in lens]
    assert runs[0] == runs[1]


def test_long_sequence_decoded_65536_steps(long_x):
    x, so, sS, _ = long_x
    say("long: 65536 decode steps")
    pool = lib().StatePool(policy_of(x), 1)
    od = _decode_seq(pool, x)
    assert sha(od) == so and sha(pool.state) == sS
