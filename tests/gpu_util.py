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
