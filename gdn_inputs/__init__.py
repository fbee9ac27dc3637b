"""Seeded synthetic inputs for the CPR gated-delta-rule workloads.

This module only draws and encodes numbers; it contains none of the recurrence's
arithmetic.  Both the CPU oracle (under ``oracle/``) and the GPU path consume the
exact bytes produced here, so the two sides never see different inputs.

Recipe (every workload):
  * one ``numpy.random.Generator(PCG64)`` per tensor, spawned from
    ``SeedSequence([seed, purpose])``;
  * q, v ~ N(0, 1) drawn in fp64;
  * k ~ N(0, 1) drawn in fp64, then L2-normalised per (token, key head) in fp64;
  * a = exp(-softplus(x)), b = sigmoid(y) with x, y ~ N(0, 1) in fp64, then cast to fp32;
  * fp64 -> fp32 is IEEE round-to-nearest-even (numpy ``astype``); fp32 -> bf16 is
    round-to-nearest-even on the bit pattern.  bf16 tensors are therefore the RNE
    bf16 of the RNE fp32 of the fp64 sample.

Layouts (row-major, tokens packed over sequences as given by ``cu_seqlens``):
  q, k ``[N, H_k, d_k]``; v ``[N, H_v, d_v]``; a, b ``[N, H_v]``.
bf16 tensors are held as ``numpy.uint16`` bit patterns.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "GdnInputs", "make_inputs", "f64_to_f32", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "config0", "config1", "config2_prompt_lengths", "config2_prompts", "config2_decode_tokens",
    "config3_lengths", "config3", "config4_x", "config4_lengths", "config4_batch", "cu_from_lengths",
]

# purposes used in SeedSequence([seed, purpose]) so that streams never collide
_P_Q, _P_K, _P_V, _P_A, _P_B, _P_LEN, _P_DECODE, _P_S0, _P_PACK = range(1, 10)


def f64_to_f32(x: np.ndarray) -> np.ndarray:
    """IEEE round-to-nearest-even fp64 -> fp32."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16, returned as uint16 bit patterns (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    # finite inputs only: the largest finite pattern plus the bias stays below 2**32
    r = (u + (np.uint32(0x7FFF) + lsb)) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, purpose: int, sub: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, purpose, sub])))


def cu_from_lengths(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=cu[1:])
    if cu[-1] >= 2**31:
        raise ValueError("total tokens exceed int32 cu_seqlens")
    return cu.astype(np.int32)


@dataclass
class GdnInputs:
    """One packed batch of tokens for the gated delta rule."""
    name: str
    h_k: int
    h_v: int
    dk: int
    dv: int
    chunk: int
    io: str                      # "f32" or "bf16"
    cu_seqlens: np.ndarray       # int32 [B+1]
    q: np.ndarray                # [N, H_k, dk] float32 or uint16 (bf16 bits)
    k: np.ndarray
    v: np.ndarray                # [N, H_v, dv]
    a: np.ndarray                # [N, H_v] float32
    b: np.ndarray
    meta: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return len(self.cu_seqlens) - 1

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.cu_seqlens.astype(np.int64))

    def widen(self, name: str) -> np.ndarray:
        """The tensor's exact value as fp64 (bf16/fp32 bits widened, no rounding)."""
        x = getattr(self, name)
        if x.dtype == np.uint16:
            x = bf16_bits_to_f32(x)
        return x.astype(np.float64)

    def digest(self) -> str:
        h = hashlib.sha256()
        for name in ("cu_seqlens", "q", "k", "v", "a", "b"):
            h.update(np.ascontiguousarray(getattr(self, name)).tobytes())
        return h.hexdigest()

    def select(self, seqs) -> "GdnInputs":
        """A new batch holding the listed sequences, in the listed order."""
        cu = self.cu_seqlens.astype(np.int64)
        idx = np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs]) if len(seqs) else np.zeros(0, np.int64)
        lengths = [int(cu[s + 1] - cu[s]) for s in seqs]
        return GdnInputs(self.name + f"[sel{len(seqs)}]", self.h_k, self.h_v, self.dk, self.dv, self.chunk,
                         self.io, cu_from_lengths(lengths), self.q[idx], self.k[idx], self.v[idx],
                         self.a[idx], self.b[idx], dict(self.meta))

    @staticmethod
    def concat(parts, name="concat") -> "GdnInputs":
        p0 = parts[0]
        lengths = np.concatenate([p.lengths for p in parts])
        cat = lambda n: np.concatenate([getattr(p, n) for p in parts], axis=0)
        return GdnInputs(name, p0.h_k, p0.h_v, p0.dk, p0.dv, p0.chunk, p0.io, cu_from_lengths(lengths),
                         cat("q"), cat("k"), cat("v"), cat("a"), cat("b"))

    def slice_tokens(self, t0: int, t1: int) -> "GdnInputs":
        """Tokens [t0, t1) of a single-sequence batch, as a single sequence."""
        assert self.num_seqs == 1
        return GdnInputs(self.name + f"[{t0}:{t1}]", self.h_k, self.h_v, self.dk, self.dv, self.chunk,
                         self.io, cu_from_lengths([t1 - t0]), self.q[t0:t1], self.k[t0:t1],
                         self.v[t0:t1], self.a[t0:t1], self.b[t0:t1])


def _encode(x64: np.ndarray, io: str) -> np.ndarray:
    x32 = f64_to_f32(x64)
    if io == "f32":
        return x32
    if io == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(io)


def make_inputs(seed: int, lengths, h_k: int, h_v: int, dk: int, dv: int, chunk: int = 64,
                io: str = "bf16", name: str = "custom", sub: int = 0) -> GdnInputs:
    """Draw q, k, v, a, b for a packed batch of sequences with the given lengths."""
    lengths = [int(x) for x in lengths]
    n = int(sum(lengths))
    q = _rng(seed, _P_Q, sub).standard_normal((n, h_k, dk))
    k = _rng(seed, _P_K, sub).standard_normal((n, h_k, dk))
    nrm = np.sqrt(np.sum(k * k, axis=-1, keepdims=True))
    k = k / nrm
    v = _rng(seed, _P_V, sub).standard_normal((n, h_v, dv))
    xa = _rng(seed, _P_A, sub).standard_normal((n, h_v))
    xb = _rng(seed, _P_B, sub).standard_normal((n, h_v))
    a = np.exp(-np.logaddexp(0.0, xa))          # exp(-softplus(x)), in (0, 1)
    b = 1.0 / (1.0 + np.exp(-xb))               # sigmoid, in (0, 1)
    return GdnInputs(name, h_k, h_v, dk, dv, chunk, io, cu_from_lengths(lengths),
                     _encode(q, io), _encode(k, io), _encode(v, io), f64_to_f32(a), f64_to_f32(b),
                     {"seed": seed, "sub": sub})


# ---------------------------------------------------------------------------------------------
# The five workloads.  Head layout for the large ones: 32 value heads over 16 key heads
# (value head h reads key head h // 2), d_k = d_v = 128, chunk 64.
# ---------------------------------------------------------------------------------------------
BIG = dict(h_k=16, h_v=32, dk=128, dv=128, chunk=64)


def config0() -> GdnInputs:
    """Tiny fp32 case: one 256-token sequence, 2 heads, d_k = d_v = 16, chunk 64."""
    return make_inputs(0, [256], h_k=2, h_v=2, dk=16, dv=16, chunk=64, io="f32", name="tiny-fp32-1x256")


def config1(num_seqs: int = 5, seqlen: int = 2048) -> GdnInputs:
    """Rollout prefill: 5 sequences x 2048 tokens, bf16 q/k/v."""
    return make_inputs(1, [seqlen] * num_seqs, io="bf16", name=f"prefill-{num_seqs}x{seqlen}", **BIG)


def config2_prompt_lengths(num_seqs: int = 256, max_len: int = 2048) -> np.ndarray:
    return _rng(2, _P_LEN).integers(1, max_len + 1, size=num_seqs)


def config2_prompts(num_seqs: int = 256, max_len: int = 2048) -> GdnInputs:
    """Ragged prompts that seed the decode states (lengths uniform in [1, max_len])."""
    return make_inputs(2, config2_prompt_lengths(num_seqs, max_len), io="bf16",
                       name=f"decode-prompts-{num_seqs}", **BIG)


def config2_decode_tokens(step: int, num_seqs: int = 256) -> GdnInputs:
    """The tokens of decode step ``step`` (one per sequence), drawn from their own stream."""
    return make_inputs(2, [1] * num_seqs, io="bf16", name=f"decode-step{step}", sub=1000 + step, **BIG)


def config3_lengths(total: int = 10240, lo: int = 64, hi: int = 4096, seed: int = 3) -> list:
    """Lengths in [lo, hi] summing exactly to ``total`` (draw while more than hi remains)."""
    rng = _rng(seed, _P_LEN)
    rem, out = total, []
    while rem > hi:
        L = int(rng.integers(lo, min(hi, rem - lo) + 1))
        out.append(L)
        rem -= L
    out.append(rem)
    rng.shuffle(out)
    return out


def config3() -> GdnInputs:
    """Trainer forward: 10240 tokens packed varlen, lengths in [64, 4096]."""
    return make_inputs(3, config3_lengths(), io="bf16", name="trainer-10240-varlen", **BIG)


def config4_x(seqlen: int = 65536) -> GdnInputs:
    """The long sequence X of the invariance sweep (large head layout, bf16)."""
    return make_inputs(4, [seqlen], io="bf16", name=f"long-{seqlen}", **BIG)


def config4_lengths(n_neighbours: int, sub: int, max_len: int = 8192) -> np.ndarray:
    return _rng(4, _P_LEN, sub).integers(1, max_len + 1, size=n_neighbours)


def config4_batch(x: GdnInputs, batch: int, sub: int, max_len: int = 8192):
    """Embed the single sequence ``x`` among ``batch - 1`` random neighbours.

    Returns (inputs, index of x in the batch)."""
    if batch == 1:
        return x, 0
    lens = config4_lengths(batch - 1, sub, max_len)
    nb = make_inputs(4, lens, io=x.io, name="neighbours", sub=100 + sub,
                     h_k=x.h_k, h_v=x.h_v, dk=x.dk, dv=x.dv, chunk=x.chunk)
    pos = int(_rng(4, _P_PACK, sub).integers(0, batch))
    order = list(range(batch - 1))
    parts = [nb.select(order[:pos]), x, nb.select(order[pos:])]
    parts = [p for p in parts if p.num_seqs > 0]
    return GdnInputs.concat(parts, name=f"x-in-batch{batch}"), pos
