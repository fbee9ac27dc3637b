"""GPU parity and bitwise identity on small and medium inputs (through the C ABI binding).

Parity: the HIP path against the fp64 oracle on the same bytes (fp32 inputs: max-abs 1e-4;
bf16 inputs: normwise 3e-3 per (sequence, value head)).  Identity: SHA-256 of output bytes equal
across prefill, trainer forward (stash), decode, packing, order and chunk size -- the property
"Solving the linear-attention headache" (IsoExec articles) asks of CPR.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
from tests.gpu_util import (check_close, decode_all, gpu_state_math, lib, oracle_all, oracle_items,
                            oracle_seq_head, policy_of, prefill, run_oracle_checks, say, sha)

pytestmark = pytest.mark.gpu


def test_tiny_prefill_matches_oracle():
    x = gi.tiny_fp32()
    say("tiny fp32 prefill vs oracle")
    o, pool, cs = prefill(x)
    ref_o, ref_S, ref_R = oracle_all(x)
    check_close("f32", o.cpu().double().numpy(), ref_o, "o")
    for h in range(x.h_v):
        check_close("f32", gpu_state_math(pool, 0, h), ref_S[0, h], f"S head {h}")
        for r in range(len(ref_R)):
            check_close("f32", cs[r, h].cpu().double().numpy().T, ref_R[r, h], f"chunk state {r} head {h}")
    assert int(pool.pos[0]) == 256


def test_tiny_decode_bitwise_equals_prefill():
    cpr = lib()
    x = gi.tiny_fp32()
    say("tiny fp32 prefill vs 256 decode steps")
    o_p, pool_p, cs = prefill(x)
    pool_d = cpr.StatePool(policy_of(x), 1, boundary=True)
    o_d = decode_all(x, pool_d)
    assert sha(o_d) == sha(o_p)
    assert sha(pool_d.state) == sha(pool_p.state)
    assert int(pool_d.pos[0]) == 256
    # the last resynchronisation happened at position 192: the chunk-3 boundary state
    assert int(pool_d.boundary_pos[0]) == 192
    assert sha(pool_d.boundary[0]) == sha(cs[3])
    ref_o, _, _ = oracle_all(x)
    check_close("f32", o_d.cpu().double().numpy(), ref_o, "decode o")


def _exact_inputs(T=150, dk=16, hv=2, seed=3):
    """a = b = 1, one-hot keys, small integer values and queries: every fp32 operation of the
    step is exact, so any correct evaluation order gives the same bits as the oracle."""
    r = np.random.default_rng(seed)
    perm = r.integers(0, dk, (T, 1))
    k = np.eye(dk, dtype=np.float32)[perm]                     # [T, 1, dk]
    q = r.integers(-4, 5, (T, 1, dk)).astype(np.float32)
    v = r.integers(-8, 9, (T, hv, dk)).astype(np.float32)
    ones = np.ones((T, hv), np.float32)
    t = lambda z: torch.from_numpy(np.ascontiguousarray(z))
    return gi.GdnInputs("exact", 1, hv, dk, dk, 64, "f32", gi.cu_from_lengths([T]),
                        t(q), t(k), t(v), t(ones), t(ones.copy()))


@pytest.mark.parametrize("dk", [16, 128])
def test_exact_vector_is_bitwise_equal_to_oracle(dk):
    x = _exact_inputs(dk=dk)
    say(f"exact vector dk={dk}")
    o, pool, _ = prefill(x)
    ref_o, ref_S, _ = oracle_all(x)
    assert np.array_equal(o.cpu().double().numpy(), ref_o)
    for h in range(x.h_v):
        assert np.array_equal(gpu_state_math(pool, 0, h), ref_S[0, h])
    pool_d = lib().StatePool(policy_of(x), 1)
    o_d = decode_all(x, pool_d)
    assert np.array_equal(o_d.cpu().double().numpy(), ref_o)


def _tie_inputs(T=300, dk=16, hv=2, seed=5):
    """bf16 io with a = b = 1 and one-hot keys: the write makes row pi(t) of S equal v_t exactly,
    and with dyadic values (multiples of 2^-13 below 2) and queries in {-1, 0, 1} every fp32
    operation of the step and of the output dot is exact.  Many outputs then fall exactly halfway
    between two bf16 values (1 + 2^-8, for one), where round-to-nearest-even keeps the even one."""
    r = np.random.default_rng(seed)
    perm = r.integers(0, dk, (T, 1))
    k = np.eye(dk, dtype=np.float32)[perm]
    q = r.integers(-1, 2, (T, 1, dk)).astype(np.float32)
    vals = np.array([0.0, 1.0, -1.0, 2.0 ** -8, -(2.0 ** -8), 3 * 2.0 ** -8, -3 * 2.0 ** -8, 2.0 ** -7, 1.5,
                     -1.5, 2.0 ** -13, 0.5], np.float32)
    v = vals[r.integers(0, len(vals), (T, hv, dk))]
    ones = np.ones((T, hv), np.float32)
    t = lambda z: torch.from_numpy(np.ascontiguousarray(z))
    bf = lambda z: t(z).to(torch.bfloat16)
    x = gi.GdnInputs("ties", 1, hv, dk, dk, 64, "bf16", gi.cu_from_lengths([T]), bf(q), bf(k), bf(v), t(ones),
                     t(ones.copy()))
    assert torch.equal(x.v.float(), t(v)) and torch.equal(x.q.float(), t(q))      # exact in bf16
    return x


@pytest.mark.parametrize("dk", [16, 128])
def test_bf16_rounding_is_nearest_even_bit_for_bit(dk):
    """Exact fp32 outputs rounded to bf16 by every output path (pass 2, one-pass, overlapped,
    decode) equal the oracle's exact values rounded to nearest even, bit for bit, ties included."""
    from tests.bf16_check import bf16_bits_to_f64, rne_bf16_bits
    cpr = lib()
    x = _tie_inputs(dk=dk)
    ref_o, ref_S, _ = oracle_all(x)
    f32 = ref_o.astype(np.float32)
    assert np.array_equal(f32.astype(np.float64), ref_o)                # the outputs are exact in fp32
    u = f32.view(np.uint32)
    ties = int(((u & 0xFFFF) == 0x8000).sum())
    assert ties >= 0.03 * u.size                                         # many exact ties
    # compared as values, so that the sign of an exact zero (which the dot's order decides) is free
    want = bf16_bits_to_f64(rne_bf16_bits(ref_o))
    bits = lambda o: bf16_bits_to_f64(o.view(torch.int16).cpu().numpy().view(np.uint16))
    say(f"bf16 ties dk={dk}: two-pass ({ties} ties of {u.size})")
    o, pool, _ = prefill(x)
    assert np.array_equal(bits(o), want)
    for h in range(x.h_v):
        assert np.array_equal(gpu_state_math(pool, 0, h), ref_S[0, h])
    o_np, _, _ = prefill(x, c_stash=None)
    assert np.array_equal(bits(o_np), want)
    for overlapped in (False, True):
        say(f"bf16 ties dk={dk}: {'overlapped' if overlapped else 'one-pass'}")
        o1, _, _ = _fused(x, overlapped=overlapped)
        assert np.array_equal(bits(o1), want)
    say(f"bf16 ties dk={dk}: decode")
    o_d = decode_all(x, cpr.StatePool(policy_of(x), 1))
    assert np.array_equal(bits(o_d), want)


LENS = [1, 5, 64, 65, 130, 33, 0, 97]


@pytest.mark.parametrize("dim", [16, 32, 64, 128])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_varlen_gqa_matches_oracle(dim, io):
    """Ragged lengths (one token, a chunk and a token, several tiles, an empty sequence) with
    GQA 2:1; o, final S and every chunk-start state against the oracle."""
    cpr = lib()
    x = gi.make_inputs(11, LENS, h_k=2, h_v=4, dk=dim, dv=dim, chunk=32, io=io)
    say(f"varlen dim={dim} io={io}")
    o, pool, cs = prefill(x)
    rows = cpr.gdn_chunk_rows(x.cu_seqlens, 32).numpy()
    o_np = o.cpu().double().numpy()
    for i, L in enumerate(LENS):
        t0, t1 = int(x.cu_seqlens[i]), int(x.cu_seqlens[i + 1])
        for h in range(x.h_v):
            ref_o, ref_S, ref_R = oracle_seq_head(x, i, h)
            if L:
                check_close(io, o_np[t0:t1, h], ref_o, f"o seq {i} head {h}")
            check_close(io, gpu_state_math(pool, i, h), ref_S, f"S seq {i} head {h}")
            for r in range(len(ref_R)):
                got = cs[rows[i] + r, h].cpu().double().numpy().T
                check_close(io, got, ref_R[r], f"chunk state seq {i} row {r} head {h}")
        assert int(pool.pos[i]) == L


def test_packing_and_order_invariance():
    x = gi.make_inputs(12, [70, 200, 1, 129, 64], h_k=2, h_v=4, dk=128, dv=128, chunk=64, io="bf16")
    say("packing / order invariance")
    o_all, pool_all, _ = prefill(x)
    for i in range(x.num_seqs):
        t0, t1 = int(x.cu_seqlens[i]), int(x.cu_seqlens[i + 1])
        o_i, pool_i, _ = prefill(x.select([i]))
        assert sha(o_i) == sha(o_all[t0:t1]), f"seq {i}"
        assert sha(pool_i.state[0]) == sha(pool_all.state[i])
    order = [4, 2, 0, 3, 1]
    y = x.select(order)
    o_y, pool_y, _ = prefill(y)
    for j, i in enumerate(order):
        t0, t1 = int(x.cu_seqlens[i]), int(x.cu_seqlens[i + 1])
        s0, s1 = int(y.cu_seqlens[j]), int(y.cu_seqlens[j + 1])
        assert sha(o_y[s0:s1]) == sha(o_all[t0:t1])
        assert sha(pool_y.state[j]) == sha(pool_all.state[i])


def test_slot_mapping_is_respected():
    """Sequences land in the slots slot_ids names; untouched slots keep their contents."""
    cpr = lib()
    x = gi.make_inputs(13, [40, 90], h_k=1, h_v=2, dk=64, dv=64, chunk=16, io="bf16")
    say("slot mapping")
    o_ref, pool_ref, _ = prefill(x)
    pool = cpr.StatePool(policy_of(x), 5)
    pool.state[2].fill_(7.0)
    o, _ = cpr.gdn_prefill(pool, x.cu_seqlens, *[t.cuda() for t in (x.q, x.k, x.v, x.a, x.b)],
                           slot_ids=[4, 0])
    torch.cuda.synchronize()
    assert sha(o) == sha(o_ref)
    assert sha(pool.state[4]) == sha(pool_ref.state[0]) and sha(pool.state[0]) == sha(pool_ref.state[1])
    assert bool((pool.state[2] == 7.0).all()) and bool((pool.state[1] == 0).all())
    assert pool.pos.tolist() == [90, 0, 0, 0, 40]


@pytest.mark.parametrize("chunk", [1, 8, 16, 100, 1000])
def test_chunk_size_changes_no_bit(chunk):
    x = gi.make_inputs(14, [300, 77], h_k=2, h_v=4, dk=128, dv=128, chunk=64, io="bf16")
    say(f"chunk invariance C={chunk}")
    o64, pool64, _ = prefill(x)
    oc, poolc, _ = prefill(x, chunk=chunk)
    assert sha(oc) == sha(o64)
    assert sha(poolc.state) == sha(pool64.state)


def test_continue_from_state_then_decode_equals_one_prefill():
    cpr = lib()
    x = gi.make_inputs(15, [300], h_k=2, h_v=4, dk=128, dv=128, chunk=64, io="bf16")
    say("split prefill + decode vs one prefill")
    o_full, pool_full, cs_full = prefill(x)
    pool = cpr.StatePool(policy_of(x), 1, boundary=True)
    o1, _, _ = prefill(x.token_slice(0, 100), pool=pool)
    o2, _, cs2 = prefill(x.token_slice(100, 250), pool=pool, from_state=True)
    o3 = decode_all(x.token_slice(250, 300), pool)
    assert sha(torch.cat([o1, o2, o3])) == sha(o_full)
    assert sha(pool.state) == sha(pool_full.state)
    assert int(pool.pos[0]) == 300
    # continuation rows: the state entering 100, then the chunk starts 128 and 192
    assert sha(cs2[1]) == sha(cs_full[2]) and sha(cs2[2]) == sha(cs_full[3])
    ref = oracle_seq_head(x, 0, 3)[0]
    check_close("bf16", torch.cat([o1, o2, o3])[:, 3].cpu().double().numpy(), ref, "o head 3")
    # decode resynchronised at 256: its boundary record is chunk 4's entering state
    assert int(pool.boundary_pos[0]) == 256 and sha(pool.boundary[0]) == sha(cs_full[4])


def test_explicit_resync_commits_only_at_chunk_starts():
    cpr = lib()
    x = gi.make_inputs(16, [128, 100], h_k=1, h_v=2, dk=32, dv=32, chunk=64, io="f32")
    say("explicit resync")
    o, pool, cs = prefill(x, boundary=True)
    cpr.gdn_state_resync(pool, [0, 1])
    torch.cuda.synchronize()
    assert pool.boundary_pos.tolist() == [128, -1]         # 100 is not a chunk start
    assert sha(pool.boundary[0]) == sha(pool.state[0])
    assert bool((pool.boundary[1] == 0).all())


def test_repeat_runs_are_identical():
    x = gi.make_inputs(17, [333, 1000], h_k=2, h_v=4, dk=128, dv=128, chunk=64, io="bf16")
    say("repeat runs")
    first = [sha(t) for t in (prefill(x)[0],)]
    for _ in range(3):
        assert [sha(prefill(x)[0])] == first


@pytest.mark.parametrize("chunk", [1, 16])
def test_overlapped_repeat_runs_are_identical(chunk):
    """The overlapped kernel's waves meet through LDS counters; a missing or misplaced wait would
    show up as run-to-run differences.  Chunk 1 hands over a chunk at every token.  Five runs,
    each equal to gdn_prefill bit for bit."""
    x = gi.make_inputs(18, [700, 45, 1], h_k=2, h_v=4, dk=128, dv=128, chunk=chunk, io="bf16")
    say(f"overlapped repeat runs, chunk {chunk}")
    o_ref, pool_ref, _ = prefill(x, chunk=chunk)
    for _ in range(5):
        o, pool, _ = _fused(x, chunk=chunk, overlapped=True)
        assert sha(o) == sha(o_ref) and sha(pool.state) == sha(pool_ref.state)


def _fused(x, chunk=None, pool=None, from_state=False, stash=True, overlapped=False):
    cpr = lib()
    xd = x.to("cuda")
    if pool is None:
        pool = cpr.StatePool(policy_of(x, chunk), max(x.num_seqs, 1))
    cs = None
    if stash:
        rows = cpr.gdn_chunk_rows_bound(x.total_tokens, x.num_seqs, pool.policy.chunk)
        cs = torch.full((max(rows, 1), x.h_v, x.dv, x.dk), float("nan"), device="cuda")
    run = cpr.gdn_prefill_overlapped if overlapped else cpr.gdn_prefill_fused
    o, cs = run(pool, x.cu_seqlens, xd.q, xd.k, xd.v, xd.a, xd.b, from_state=from_state, chunk_states=cs)
    torch.cuda.synchronize()
    return o, pool, cs


@pytest.mark.parametrize("dim", [16, 32, 64, 128])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_fused_prefill_is_bitwise_equal_to_two_pass(dim, io):
    cpr = lib()
    x = gi.make_inputs(21, LENS, h_k=2, h_v=4, dk=dim, dv=dim, chunk=32, io=io)
    say(f"fused vs two-pass dim={dim} io={io}")
    o2, pool2, cs2 = prefill(x)
    o1, pool1, cs1 = _fused(x)
    assert sha(o1) == sha(o2)
    assert sha(pool1.state) == sha(pool2.state) and pool1.pos.tolist() == pool2.pos.tolist()
    n = int(cpr.gdn_chunk_rows(x.cu_seqlens, 32)[-1])
    assert sha(cs1[:n]) == sha(cs2[:n])
    assert bool(torch.isnan(cs1[n:]).all())              # nothing written past the last row
    o3, pool3, _ = _fused(x, stash=False)
    assert sha(o3) == sha(o2) and sha(pool3.state) == sha(pool2.state)
    # and directly against the oracle: o, final states and chunk-start rows of every pair
    run_oracle_checks(oracle_items(x, o1, pool1.state, chunk_states=cs1), f"fused dim={dim} io={io}")


@pytest.mark.parametrize("dim,io", [(16, "f32"), (128, "bf16")])
def test_degenerate_gates(dim, io):
    """The method's degenerate cases on the GPU.  a = 1, b = 0: the update writes nothing, so the
    final state is the initial one bit for bit (fma(k, 0, 1 * S) = S) and o_t = S_0^T q_t.  a = 0:
    the state forgets everything each token, S_t = b_t k_t v_t^T and o_t = b_t (k_t . q_t) v_t.
    Outputs against the oracle at the usual tolerances."""
    import dataclasses
    cpr = lib()
    x = gi.make_inputs(37, [50, 1, 77], h_k=2, h_v=4, dk=dim, dv=dim, chunk=32, io=io)
    s0 = torch.randn((x.num_seqs, x.h_v, dim, dim), generator=torch.Generator().manual_seed(7)) * 0.1
    for case, (av, bv) in {"keep": (1.0, 0.0), "forget": (0.0, None)}.items():
        say(f"degenerate gates {case} dim={dim} io={io}")
        xa = dataclasses.replace(x, a=torch.full_like(x.a, av), b=x.b if bv is None else torch.full_like(x.b, bv))
        pool = cpr.StatePool(policy_of(xa), xa.num_seqs)
        pool.state.copy_(s0.cuda())
        o, pool, _ = prefill(xa, pool=pool, from_state=True)
        if case == "keep":
            assert torch.equal(pool.state.cpu(), s0)
        for i in range(xa.num_seqs):
            t0, t1 = int(xa.cu_seqlens[i]), int(xa.cu_seqlens[i + 1])
            for h in (0, 3):
                S0_math = s0[i, h].double().numpy().T
                ref_o, ref_S, _ = oracle_seq_head(xa, i, h, S0=S0_math)
                check_close(io, o[t0:t1, h].float().cpu().numpy(), ref_o, f"{case} o seq {i} head {h}")
                check_close(io, gpu_state_math(pool, i, h), ref_S, f"{case} S seq {i} head {h}")


def test_many_sequences_beyond_one_scan_block():
    """700 ragged sequences (0..40 tokens, empty ones included) are more than a workgroup has
    threads, so the device-side varlen planners scan cu_seqlens in several blocks: the two-pass
    prefill with and without the c stash, the one-pass kernel and the overlapped kernel (under a
    cap that lets it run) agree bit for bit, and sampled sequences match the oracle."""
    cpr = lib()
    lens = [(37 * i) % 41 for i in range(700)]
    x = gi.make_inputs(36, lens, h_k=1, h_v=2, dk=16, dv=16, chunk=16, io="f32")
    say("700 ragged sequences")
    n = int(cpr.gdn_chunk_rows(x.cu_seqlens, 16)[-1])
    o0, pool0, cs0 = prefill(x)
    ref = (sha(o0), sha(pool0.state), pool0.pos.tolist(), sha(cs0[:n]))
    o1, pool1, cs1 = prefill(x, c_stash=False)
    assert (sha(o1), sha(pool1.state), pool1.pos.tolist(), sha(cs1[:n])) == ref
    o2, pool2, cs2 = _fused(x)
    assert (sha(o2), sha(pool2.state), pool2.pos.tolist(), sha(cs2[:n])) == ref
    pool3 = cpr.StatePool(policy_of(x), x.num_seqs)
    pool3.set_max_workgroups(200)
    o3, pool3, cs3 = _fused(x, pool=pool3, overlapped=True)
    assert (sha(o3), sha(pool3.state), pool3.pos.tolist(), sha(cs3[:n])) == ref
    for i in (3, 350, 699):
        for h in range(x.h_v):
            ref_o, ref_S, _ = oracle_seq_head(x, i, h)
            t0, t1 = int(x.cu_seqlens[i]), int(x.cu_seqlens[i + 1])
            check_close("f32", o0[t0:t1, h].float().cpu().numpy(), ref_o, f"o seq {i} head {h}")
            check_close("f32", gpu_state_math(pool0, i, h), ref_S, f"S seq {i} head {h}")


@pytest.mark.parametrize("dim,io", [(16, "f32"), (128, "bf16")])
def test_column_permutation_permutes_outputs_bitwise(dim, io):
    """Permuting the d_v columns of v and of the initial state permutes the columns of o and of the
    final state bit for bit: every column runs the same arithmetic on its own data, whichever lanes
    and workgroups hold it."""
    import dataclasses
    cpr = lib()
    x = gi.make_inputs(35, [70, 1, 130], h_k=2, h_v=4, dk=dim, dv=dim, chunk=32, io=io)
    perm = torch.from_numpy(np.random.default_rng(3).permutation(dim))
    s0 = torch.randn((x.num_seqs, x.h_v, dim, dim), generator=torch.Generator().manual_seed(5)) * 0.1
    say(f"column permutation dim={dim} io={io}")
    pool1 = cpr.StatePool(policy_of(x), x.num_seqs)
    pool1.state.copy_(s0.cuda())
    o1, pool1, _ = prefill(x, pool=pool1, from_state=True)
    xp = dataclasses.replace(x, v=x.v[:, :, perm].contiguous())
    pool2 = cpr.StatePool(policy_of(x), x.num_seqs)
    pool2.state.copy_(s0[:, :, perm, :].contiguous().cuda())      # state [slot][H_v][d_v][d_k]
    o2, pool2, _ = prefill(xp, pool=pool2, from_state=True)
    assert sha(o2) == sha(o1[:, :, perm.cuda()].contiguous())
    assert sha(pool2.state) == sha(pool1.state[:, :, perm.cuda(), :].contiguous())


@pytest.mark.parametrize("dim", [16, 32, 64, 128])
def test_prefill_under_a_grid_cap_matches_the_natural_launch(dim):
    """A ragged batch (empty, one-token and multi-chunk sequences) with every capped kernel limited
    to 1, 3 and 64 workgroups: two-pass with and without the c stash, one-pass and overlapped --
    o, final states, positions and chunk-start rows as in the natural launch, bit for bit."""
    cpr = lib()
    x = gi.make_inputs(29, LENS, h_k=2, h_v=4, dk=dim, dv=dim, chunk=32, io="bf16")
    n = int(cpr.gdn_chunk_rows(x.cu_seqlens, 32)[-1])
    o0, pool0, cs0 = prefill(x)
    ref = (sha(o0), sha(pool0.state), pool0.pos.tolist(), sha(cs0[:n]))
    for cap in (1, 3, 64):
        say(f"grid cap {cap} dim={dim}")
        for stash in (True, False):
            pool = cpr.StatePool(policy_of(x), x.num_seqs)
            pool.set_max_workgroups(cap)
            o, pool, cs = prefill(x, pool=pool, c_stash=stash)
            assert (sha(o), sha(pool.state), pool.pos.tolist(), sha(cs[:n])) == ref, (cap, stash)
        for overlapped in (False, True):
            pool = cpr.StatePool(policy_of(x), x.num_seqs)
            pool.set_max_workgroups(cap)
            o, pool, cs = _fused(x, pool=pool, overlapped=overlapped)
            assert (sha(o), sha(pool.state), pool.pos.tolist(), sha(cs[:n])) == ref, (cap, overlapped)


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("dim", [16, 32, 64, 128])
def test_c_stash_changes_no_bit(dim, io):
    """gdn_prefill with the c stash (pass 1 runs every token and keeps its c, pass 2 applies the
    kept c) against the same call without it: o, final states and chunk states bit for bit.  The
    stash then holds every token's c, exactly the block the trainer forward keeps."""
    cpr = lib()
    x = gi.make_inputs(23, LENS, h_k=2, h_v=4, dk=dim, dv=dim, chunk=32, io=io)
    say(f"c stash vs none dim={dim} io={io}")
    stash = torch.full((x.total_tokens, x.h_v, x.dv), float("nan"), device="cuda")
    o1, pool1, cs1 = prefill(x, c_stash=stash)
    o2, pool2, cs2 = prefill(x, c_stash=None)
    assert sha(o1) == sha(o2)
    assert sha(pool1.state) == sha(pool2.state) and pool1.pos.tolist() == pool2.pos.tolist()
    n = int(cpr.gdn_chunk_rows(x.cu_seqlens, 32)[-1])
    assert sha(cs1[:n]) == sha(cs2[:n])
    assert not bool(torch.isnan(stash).any())
    xd = x.to("cuda")
    pool3 = cpr.StatePool(policy_of(x), max(x.num_seqs, 1))
    o3, cs3, cw = cpr.gdn_trainer_forward(pool3, x.cu_seqlens, xd.q, xd.k, xd.v, xd.a, xd.b)
    torch.cuda.synchronize()
    assert sha(cw[0]) == sha(stash) and sha(o3) == sha(o1) and sha(cs3[:n]) == sha(cs1[:n])


@pytest.mark.parametrize("boundary", ["f32", "bf16"])
def test_c_stash_continuation_changes_no_bit(boundary):
    """The stash path continuing from a state (positions not on a chunk start), with both boundary
    dtypes: the same bits as the path without the stash and as one run over all tokens."""
    cpr = lib()
    x = gi.make_inputs(24, [300], h_k=2, h_v=4, dk=128, dv=128, chunk=64, io="bf16")
    say(f"c stash continuation boundary={boundary}")
    pol = cpr.Policy(2, 4, 128, 128, 64, "bf16", boundary=boundary)
    results = []
    for stash in (True, None):
        pool = cpr.StatePool(pol, 1)
        o1, _, _ = prefill(x.token_slice(0, 77), pool=pool, c_stash=stash)
        o2, _, cs2 = prefill(x.token_slice(77, 300), pool=pool, from_state=True, c_stash=stash)
        n = int(cpr.gdn_chunk_rows([0, 223], 64, [77])[-1])      # rows past n are never written
        results.append((sha(torch.cat([o1, o2])), sha(pool.state), sha(cs2[:n])))
    full = cpr.StatePool(pol, 1)
    o_full, _, _ = prefill(x, pool=full)
    assert results[0] == results[1]
    assert results[0][0] == sha(o_full) and results[0][1] == sha(full.state)


@pytest.mark.parametrize("chunk", [1, 16, 64, 1000])
def test_fused_continuation_matches(chunk):
    cpr = lib()
    x = gi.make_inputs(22, [300], h_k=2, h_v=4, dk=128, dv=128, chunk=chunk, io="bf16")
    say(f"fused continuation C={chunk}")
    o_full, pool_full, cs_full = prefill(x, chunk=chunk)
    pool = cpr.StatePool(policy_of(x, chunk), 1)
    o1, _, _ = _fused(x.token_slice(0, 77), pool=pool)
    o2, _, cs2 = _fused(x.token_slice(77, 300), pool=pool, from_state=True)
    assert sha(torch.cat([o1, o2])) == sha(o_full)
    assert sha(pool.state) == sha(pool_full.state) and int(pool.pos[0]) == 300
    rows = cpr.gdn_chunk_rows([0, 223], chunk, [77]).numpy()
    full_rows = cpr.gdn_chunk_rows([0, 300], chunk).numpy()
    # rows after the hand-over state are the same chunk-start states as in one run
    k0 = int(full_rows[-1]) - (int(rows[-1]) - 1)
    assert sha(cs2[1:int(rows[-1])]) == sha(cs_full[k0:int(full_rows[-1])])


@pytest.mark.parametrize("io", ["f32", "bf16"])
@pytest.mark.parametrize("dim", [16, 32, 64, 128])
def test_overlapped_prefill_is_bitwise_equal_to_two_pass(dim, io):
    """The overlapped prefill (pass 1 and the chunk outputs in one workgroup) against gdn_prefill:
    o, final states, positions and chunk-start rows bit for bit, nothing written past the rows."""
    cpr = lib()
    x = gi.make_inputs(26, LENS, h_k=2, h_v=4, dk=dim, dv=dim, chunk=32, io=io)
    say(f"overlapped vs two-pass dim={dim} io={io}")
    o2, pool2, cs2 = prefill(x)
    o1, pool1, cs1 = _fused(x, overlapped=True)
    assert sha(o1) == sha(o2)
    assert sha(pool1.state) == sha(pool2.state) and pool1.pos.tolist() == pool2.pos.tolist()
    n = int(cpr.gdn_chunk_rows(x.cu_seqlens, 32)[-1])
    assert sha(cs1[:n]) == sha(cs2[:n])
    assert bool(torch.isnan(cs1[n:]).all())
    o3, pool3, _ = _fused(x, stash=False, overlapped=True)
    assert sha(o3) == sha(o2) and sha(pool3.state) == sha(pool2.state)
    lib().gdn_device_status()                               # no wait gave up
    run_oracle_checks(oracle_items(x, o1, pool1.state, chunk_states=cs1), f"overlapped dim={dim} io={io}")


def test_overlapped_wait_give_up_is_reported():
    """With the overlapped kernel's wait bound set to one poll from the host, its waves give up
    waiting for each other (the staging wave cannot be a tile ahead, pass 2 cannot see a chunk
    handed over); every wave still leaves its work item normally, and gdn_device_status reports
    GDN_EHIP.  The status is cleared by the check: the same call with the default bound then
    reports nothing and gives gdn_prefill's bits."""
    cpr = lib()
    x = gi.make_inputs(29, [1000], h_k=2, h_v=4, dk=128, dv=128, chunk=64, io="bf16")
    xd = x.to("cuda")
    say("overlapped prefill with a one-poll wait bound")
    cpr.gdn_device_status()
    pool = cpr.StatePool(policy_of(x), 1)
    pool.set_wait_limit(1)
    cpr.gdn_prefill_overlapped(pool, x.cu_seqlens, xd.q, xd.k, xd.v, xd.a, xd.b)
    with pytest.raises(cpr.GdnError) as e:
        cpr.gdn_device_status()
    assert e.value.code == 3 and "gave up" in str(e.value)
    cpr.gdn_device_status()                                 # cleared by the check above
    say("overlapped prefill with the default wait bound")
    o_ref, pool_ref, _ = prefill(x)
    pool2 = cpr.StatePool(policy_of(x), 1)
    pool2.set_wait_limit(0)
    o, _ = cpr.gdn_prefill_overlapped(pool2, x.cu_seqlens, xd.q, xd.k, xd.v, xd.a, xd.b)
    cpr.gdn_device_status()
    assert sha(o) == sha(o_ref) and sha(pool2.state) == sha(pool_ref.state)


def test_side_stream_calls_match_the_current_stream():
    """Prefill (with the c stash the binding allocates), decode, the overlapped prefill and the
    backward called with a non-current stream: every tensor the binding allocates is allocated on
    that stream, and the results equal those of the same calls on the current stream bit for bit.
    Allocations on the current stream are made meanwhile, so memory the binding freed early would
    be reused under the kernels."""
    cpr = lib()
    x = gi.make_inputs(30, [300, 5, 129], h_k=2, h_v=4, dk=128, dv=128, chunk=64, io="bf16", device="cuda")
    steps = [gi.make_inputs(30, [1] * 3, h_k=2, h_v=4, dk=128, dv=128, io="bf16", sub=900 + s, device="cuda")
             for s in range(5)]
    ct = gi.make_cotangents(x, 31, device="cuda")

    def run(stream):
        pool = cpr.StatePool(policy_of(x), 3)
        o, cs = cpr.gdn_prefill(pool, x.cu_seqlens, x.q, x.k, x.v, x.a, x.b, stream=stream)
        junk = [torch.randn(1 << 20, device="cuda") for _ in range(4)]     # current-stream allocations
        outs = [cpr.gdn_decode_step(pool, s.q, s.k, s.v, s.a, s.b, stream=stream) for s in steps]
        g = cpr.gdn_backward(policy_of(x), x.cu_seqlens, x.q, x.k, x.v, x.a, x.b, cs, ct["d_o"],
                             d_state=ct["d_state"], stream=stream)
        p2 = cpr.StatePool(policy_of(x), 3)
        o2, _ = cpr.gdn_prefill_overlapped(p2, x.cu_seqlens, x.q, x.k, x.v, x.a, x.b, stream=stream)
        if stream is not None:
            stream.synchronize()
        torch.cuda.synchronize()
        del junk
        return [sha(o), sha(pool.state), sha(torch.stack(outs)), sha(o2)] + [sha(g[n]) for n in ("dq", "dk", "dv", "da", "db")]

    say("calls on the current stream")
    ref = run(None)
    say("the same calls on a side stream")
    side = torch.cuda.Stream()
    assert run(side) == ref


def test_overlapped_prefill_beyond_one_workgroup_per_cu():
    """A batch whose overlapped grid exceeds the CU count (40 sequences x 4 value heads x 8
    column groups) runs the one-pass kernel instead: still the same bits as gdn_prefill."""
    cpr = lib()
    lens = [(37 * i) % 150 + 1 for i in range(40)]
    x = gi.make_inputs(28, lens, h_k=2, h_v=4, dk=128, dv=128, chunk=32, io="bf16")
    say("overlapped beyond one workgroup per CU")
    o2, pool2, cs2 = prefill(x)
    o1, pool1, cs1 = _fused(x, overlapped=True)
    assert sha(o1) == sha(o2) and sha(pool1.state) == sha(pool2.state)
    n = int(cpr.gdn_chunk_rows(x.cu_seqlens, 32)[-1])
    assert sha(cs1[:n]) == sha(cs2[:n])


@pytest.mark.parametrize("boundary", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [1, 16, 64, 100])
def test_overlapped_continuation_matches(chunk, boundary):
    """Continuing from a state at a position off the chunk grid, both boundary dtypes; a chunk
    above 64 tokens takes the one-pass kernel and must give the same bits as well."""
    cpr = lib()
    x = gi.make_inputs(27, [300], h_k=2, h_v=4, dk=128, dv=128, chunk=chunk, io="bf16")
    say(f"overlapped continuation C={chunk} boundary={boundary}")
    pol = cpr.Policy(2, 4, 128, 128, chunk, "bf16", boundary=boundary)
    full = cpr.StatePool(pol, 1)
    o_full, _, cs_full = prefill(x, pool=full)
    pool = cpr.StatePool(pol, 1)
    o1, _, _ = _fused(x.token_slice(0, 77), pool=pool, overlapped=True)
    o2, _, cs2 = _fused(x.token_slice(77, 300), pool=pool, from_state=True, overlapped=True)
    assert sha(torch.cat([o1, o2])) == sha(o_full)
    assert sha(pool.state) == sha(full.state) and int(pool.pos[0]) == 300
    rows = cpr.gdn_chunk_rows([0, 223], chunk, [77]).numpy()
    full_rows = cpr.gdn_chunk_rows([0, 300], chunk).numpy()
    k0 = int(full_rows[-1]) - (int(rows[-1]) - 1)
    assert sha(cs2[1:int(rows[-1])]) == sha(cs_full[k0:int(full_rows[-1])])
