"""gdn_prefill_static, the prefill that allocates nothing (its scratch is a library-owned static
device buffer), against gdn_prefill with caller-owned chunk states, through the C ABI: the same
bits in o, final states and positions on consecutive calls of decreasing size (the buffer keeps the
previous call's contents), with and without room for the c stash, from zero and from a state; a
batch whose chunk-start rows exceed the buffer is refused before any launch."""
import pytest
import torch

import gdn_inputs as gi
from tests.gpu_util import lib, policy_of, say, sha

pytestmark = pytest.mark.gpu


def _reference(x, pool=None, from_state=False):
    cpr = lib()
    xd = x.to("cuda")
    pool = pool or cpr.StatePool(policy_of(x), x.num_seqs)
    o, _ = cpr.gdn_prefill(pool, x.cu_seqlens, xd.q, xd.k, xd.v, xd.a, xd.b, from_state=from_state)
    torch.cuda.synchronize()
    return o, pool


def _static(x, pool=None, from_state=False):
    cpr = lib()
    xd = x.to("cuda")
    pool = pool or cpr.StatePool(policy_of(x), x.num_seqs)
    cu = torch.from_numpy(x.cu_seqlens).to("cuda")
    ids = torch.arange(x.num_seqs, dtype=torch.int32, device="cuda")
    o = torch.empty((x.total_tokens, x.h_v, x.dv), dtype=xd.q.dtype, device="cuda")
    cpr.gdn_prefill_static(pool, cu, xd.q, xd.k, xd.v, xd.a, xd.b, slot_ids=ids, o=o, from_state=from_state)
    torch.cuda.synchronize()
    return o, pool


def _same(x, label):
    say(f"static prefill: {label} ({x.total_tokens} tokens in {x.num_seqs} sequences)")
    o_ref, p_ref = _reference(x)
    o, p = _static(x)
    assert sha(o) == sha(o_ref), label
    assert sha(p.state) == sha(p_ref.state) and p.pos.tolist() == p_ref.pos.tolist(), label


def test_static_prefill_equals_prefill_on_consecutive_calls():
    cpr = lib()
    big = dict(h_k=16, h_v=32, dk=128, dv=128, chunk=64, io="bf16", device="cuda")
    # 67 chunk-start rows (134 MiB) and a 58 MB c stash: both in the buffer
    _same(gi.make_inputs(81, [700, 1, 300, 2048, 0, 511], **big), "rows and c stash")
    # a second, smaller call: the buffer still holds the first call's rows and stash
    _same(gi.make_inputs(82, [100, 37], **big), "smaller, after a larger call")
    # 111 rows (222 MiB): the c stash no longer fits, the output pass recomputes c
    x = gi.make_inputs(83, [7000], **big)
    rows = cpr.gdn_chunk_rows_bound(x.total_tokens, x.num_seqs, 64)
    assert rows * 32 * 128 * 128 * 4 + x.total_tokens * 32 * 128 * 4 > cpr.GDN_STATIC_SCRATCH_BYTES
    _same(x, "rows only")
    # small heads, fp32 io, ragged
    _same(gi.make_inputs(84, [1, 64, 65, 0, 200], h_k=2, h_v=4, dk=16, dv=16, chunk=16, io="f32", device="cuda"),
          "d = 16, fp32")


def test_static_prefill_continues_from_slots():
    """Split prefill: the second half continues from the slots (from_state) at a position off the
    chunk grid; both halves through the static entry point equal both through gdn_prefill."""
    big = dict(h_k=16, h_v=32, dk=128, dv=128, chunk=64, io="bf16", device="cuda")
    say("static prefill: continuation")
    cpr = lib()
    a1 = gi.make_inputs(86, [77, 100, 5], **big)
    a2 = gi.make_inputs(87, [300, 1, 64], **big)
    o1r, pr = _reference(a1)
    o2r, pr = _reference(a2, pool=pr, from_state=True)
    o1, ps = _static(a1)
    o2, ps = _static(a2, pool=ps, from_state=True)
    assert sha(o1) == sha(o1r) and sha(o2) == sha(o2r)
    assert sha(ps.state) == sha(pr.state) and ps.pos.tolist() == pr.pos.tolist() == [377, 101, 69]
    assert cpr.GDN_STATIC_SCRATCH_BYTES == 256 << 20


def test_static_prefill_refuses_a_batch_above_the_buffer():
    """The 5 x 2048 workload needs 170 chunk-start rows (340 MiB): refused with GDN_EINVAL before any
    launch, o and the slots untouched."""
    cpr = lib()
    x = gi.prefill_5x2048(device="cuda")
    pool = cpr.StatePool(policy_of(x), x.num_seqs)
    cu = torch.from_numpy(x.cu_seqlens).to("cuda")
    ids = torch.arange(x.num_seqs, dtype=torch.int32, device="cuda")
    o = torch.zeros((x.total_tokens, x.h_v, x.dv), dtype=torch.bfloat16, device="cuda")
    say("static prefill: a batch above the buffer")
    with pytest.raises(cpr.GdnError) as e:
        cpr.gdn_prefill_static(pool, cu, x.q, x.k, x.v, x.a, x.b, slot_ids=ids, o=o)
    assert e.value.code == 1 and "static" in str(e.value)
    torch.cuda.synchronize()
    assert not o.any() and not pool.state.any() and not pool.pos.any()
