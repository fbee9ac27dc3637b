"""Helpers for the GPU tests: run the library through its binding, run the oracle on the same
bytes, compare with the stated tolerances, and digest outputs."""
import hashlib
import os
import sys

import numpy as np
import torch

import gdn_inputs as gi
from oracle import gdn_varlen, recurrence

# tolerance of the GPU path against the fp64 oracle
FP32_MAX_ABS = 1e-4          # fp32 inputs: elementwise max-abs on o and S
BF16_NORMWISE = 3e-3         # bf16 inputs: ||x - ref|| / ||ref|| per (sequence, value head)


def say(msg: str):
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def lib():
    import bitwise_aligned_gated_amd as cpr
    return cpr


def policy_of(x: gi.GdnInputs, chunk=None):
    cpr = lib()
    return cpr.Policy(x.h_k, x.h_v, x.dk, x.dv, chunk or x.chunk, x.io)


def sha(t: torch.Tensor) -> str:
    t = t.detach().to("cpu").contiguous()
    return hashlib.sha256(t.view(torch.uint8).numpy().tobytes() if t.numel() else b"").hexdigest()


def prefill(x: gi.GdnInputs, chunk=None, pool=None, slot_ids=None, from_state=False, boundary=False,
            chunk_states=None, c_stash=True):
    """Run gdn_prefill over x (tensors moved to the GPU). Returns (o, pool, chunk_states)."""
    cpr = lib()
    xd = x.to("cuda")
    if pool is None:
        pool = cpr.StatePool(policy_of(x, chunk), max(x.num_seqs, 1), boundary=boundary)
    o, cs = cpr.gdn_prefill(pool, x.cu_seqlens, xd.q, xd.k, xd.v, xd.a, xd.b, slot_ids=slot_ids,
                            from_state=from_state, chunk_states=chunk_states, c_stash=c_stash)
    torch.cuda.synchronize()
    return o, pool, cs


def decode_all(x: gi.GdnInputs, pool, slot_ids=None):
    """Feed the single sequence x token by token through gdn_decode_step into one slot of pool
    (slot 0 unless given).  Returns o [T, H_v, dv]."""
    cpr = lib()
    xd = x.to("cuda")
    T = x.total_tokens
    outs = []
    ids = torch.tensor([0] if slot_ids is None else slot_ids, dtype=torch.int32, device="cuda")
    for t in range(T):
        outs.append(cpr.gdn_decode_step(pool, xd.q[t:t + 1], xd.k[t:t + 1], xd.v[t:t + 1], xd.a[t:t + 1],
                                        xd.b[t:t + 1], slot_ids=ids))
    torch.cuda.synchronize()
    return torch.cat(outs, dim=0)


def oracle_seq_head(x: gi.GdnInputs, seq: int, h: int, S0=None, pos0=0, chunk=None):
    """Oracle for one (sequence, value head) of x on its exact bytes."""
    t0, t1 = int(x.cu_seqlens[seq]), int(x.cu_seqlens[seq + 1])
    g = h // (x.h_v // x.h_k)
    rows = slice(t0, t1)
    q = x.widen("q", rows)[:, g]
    k = x.widen("k", rows)[:, g]
    v = x.widen("v", rows)[:, h]
    a = x.widen("a", rows)[:, h]
    b = x.widen("b", rows)[:, h]
    return recurrence(q, k, v, a, b, S0=S0, pos0=pos0, chunk=chunk or x.chunk)


def oracle_all(x: gi.GdnInputs, chunk=None):
    cpu = x.to("cpu")
    return gdn_varlen(cpu.widen("q"), cpu.widen("k"), cpu.widen("v"), cpu.widen("a"), cpu.widen("b"),
                      x.cu_seqlens, x.h_k, x.h_v, chunk=chunk or x.chunk)


def gpu_state_math(pool, slot: int, h: int) -> np.ndarray:
    """State of (slot, value head) in math orientation S[d_k][d_v] as fp64."""
    return pool.state[slot, h].detach().to("cpu").to(torch.float64).numpy().T


def normwise(x: np.ndarray, ref: np.ndarray) -> float:
    d = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (d if d > 0 else 1.0))


def check_close(io: str, got: np.ndarray, ref: np.ndarray, what: str):
    if io == "f32":
        err = float(np.max(np.abs(got - ref))) if got.size else 0.0
        assert err <= FP32_MAX_ABS, f"{what}: max-abs {err:.3e} > {FP32_MAX_ABS}"
    else:
        err = normwise(got, ref)
        assert err <= BF16_NORMWISE, f"{what}: normwise {err:.3e} > {BF16_NORMWISE}"
    return err


def _raw(t: torch.Tensor) -> np.ndarray:
    """Host copy of a tensor's exact bytes: bf16 as uint16 bit patterns, fp32 as float32."""
    t = t.detach().to("cpu").contiguous()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


def oracle_items(x: gi.GdnInputs, o: torch.Tensor, state: torch.Tensor, pairs=None, slots=None,
                 chunk_states=None, S0=None, pos0=None, with_state=True):
    """Work items for tests.oracle_pool.check_pair, one per (sequence, value head) of `pairs`
    (default: every pair): the exact input bytes of x, the GPU's outputs o, its final states
    (state[slots[i], h], stored transposed), and, when chunk_states is given, the sequence's
    chunk-start rows (row offsets from gdn_chunk_rows).  S0 [B, H_v, d_v, d_k] (stored
    orientation) and pos0 [B] describe a continuation."""
    cpr = lib()
    q, k, v, a, b = (_raw(getattr(x, n)) for n in ("q", "k", "v", "a", "b"))
    go = _raw(o)
    st = state.detach().to("cpu").numpy() if with_state else None
    s0 = None if S0 is None else S0.detach().to("cpu").numpy()
    p0 = [0] * x.num_seqs if pos0 is None else [int(p) for p in pos0]
    cs = rows = None
    if chunk_states is not None:
        cs = chunk_states.detach().to("cpu").numpy()
        rows = cpr.gdn_chunk_rows(x.cu_seqlens, x.chunk, pos0=None if pos0 is None else p0).numpy()
    if pairs is None:
        pairs = [(i, h) for i in range(x.num_seqs) for h in range(x.h_v)]
    ratio = x.h_v // x.h_k
    items = []
    for i, h in pairs:
        t0, t1 = int(x.cu_seqlens[i]), int(x.cu_seqlens[i + 1])
        g = h // ratio
        slot = i if slots is None else int(slots[i])
        items.append(dict(
            label=f"{x.name} seq {i} head {h}", io=x.io, q=q[t0:t1, g], k=k[t0:t1, g], v=v[t0:t1, h],
            a=a[t0:t1, h], b=b[t0:t1, h], pos0=p0[i], chunk=x.chunk,
            S0=None if s0 is None else s0[i, h].T.astype(np.float64),
            got_o=go[t0:t1, h], got_S=None if st is None else st[slot, h].T.astype(np.float64),
            got_rows=None if cs is None else cs[rows[i]:rows[i + 1], h].transpose(0, 2, 1).astype(np.float64)))
    return items


def run_oracle_checks(items, what: str) -> dict:
    """Run tests.oracle_pool.check_pair over the items; fail with the first messages if any failed.
    Returns the totals of the elementwise counts."""
    from tests import oracle_pool
    say(f"{what}: {len(items)} oracle checks ({oracle_pool.WORKERS or 'no'} pool workers)")
    res = oracle_pool.run(items, progress=lambda n: say(f"{what}: {n}/{len(items)} checked"))
    bad = [r["msg"] for r in res if not r["ok"]]
    assert not bad, f"{len(bad)} failing pairs: {bad[:4]}"
    tot = oracle_pool.summarize(res)
    say(f"{what}: {tot}")
    return tot
