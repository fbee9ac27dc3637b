"""Seeded synthetic inputs for the CPR gated-delta-rule workloads.

This module only draws and encodes numbers; it contains none of the recurrence's arithmetic.
Both the CPU oracle (under ``oracle/``) and the GPU path consume the exact bytes produced here:
tensors are drawn once, on the device where they will be used, and the oracle reads host copies
of those same bytes.

Recipe (every workload):
  * one seeded torch generator per tensor, seeded from (seed, purpose, sub) through SHA-256, on
    the chosen device (CPU: mt19937; GPU: Philox), so a (seed, device) pair fixes every byte;
  * q, v ~ N(0, 1) drawn in fp64;
  * k ~ N(0, 1) drawn in fp64, then L2-normalised per (token, key head) in fp64;
  * a = exp(-softplus(x)), b = sigmoid(y) with x, y ~ N(0, 1) in fp64, then rounded to fp32;
  * fp64 -> fp32 and fp32 -> bf16 are IEEE round-to-nearest-even, so a bf16 tensor holds the RNE
    bf16 of the RNE fp32 of the fp64 sample.
Sequence lengths (ragged workloads) come from numpy PCG64 streams seeded the same way.

Layouts (row-major, tokens packed over sequences as given by ``cu_seqlens``):
  q, k ``[N, H_k, d_k]``; v ``[N, H_v, d_v]``; a, b ``[N, H_v]`` (fp32).
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = [
    "GdnInputs", "make_inputs", "f32_to_bf16_bits", "bf16_bits_to_f32", "cu_from_lengths",
    "tiny_fp32", "prefill_5x2048", "decode_prompt_lengths", "decode_prompts", "decode_tokens",
    "trainer_lengths", "trainer_10240", "long_sequence", "neighbour_lengths", "long_in_batch",
]

# purposes, so that streams never collide
_P_Q, _P_K, _P_V, _P_A, _P_B, _P_LEN, _P_PACK = 1, 2, 3, 4, 5, 6, 7
_P_DO, _P_DS, _P_S0 = 8, 9, 10


def _seed_of(seed: int, purpose: int, sub: int) -> int:
    h = hashlib.sha256(f"gdn-inputs/{seed}/{purpose}/{sub}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(seed: int, purpose: int, sub: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed_of(seed, purpose, sub))
    return g


def _np_rng(seed: int, purpose: int, sub: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(_seed_of(seed, purpose, sub)))


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


def cu_from_lengths(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=cu[1:])
    if cu[-1] >= 2**31:
        raise ValueError("total tokens exceed int32 cu_seqlens")
    return cu.astype(np.int32)


@dataclass
class GdnInputs:
    """One packed batch of tokens for the gated delta rule (torch tensors on one device)."""
    name: str
    h_k: int
    h_v: int
    dk: int
    dv: int
    chunk: int
    io: str                      # "f32" or "bf16"
    cu_seqlens: np.ndarray       # int32 [B+1] (host)
    q: torch.Tensor              # [N, H_k, dk] float32 or bfloat16
    k: torch.Tensor
    v: torch.Tensor              # [N, H_v, dv]
    a: torch.Tensor              # [N, H_v] float32
    b: torch.Tensor
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

    @property
    def device(self) -> torch.device:
        return self.q.device

    def widen(self, name: str, rows=None) -> np.ndarray:
        """Host fp64 copy of a tensor (optionally of selected token rows): the exact values."""
        x = getattr(self, name)
        if rows is not None:
            x = x[rows]
        return x.detach().to("cpu").to(torch.float64).numpy()

    def to(self, device) -> "GdnInputs":
        mv = lambda t: t.to(device)
        return GdnInputs(self.name, self.h_k, self.h_v, self.dk, self.dv, self.chunk, self.io,
                         self.cu_seqlens.copy(), mv(self.q), mv(self.k), mv(self.v), mv(self.a),
                         mv(self.b), dict(self.meta))

    def digest(self) -> str:
        h = hashlib.sha256()
        h.update(self.cu_seqlens.tobytes())
        for name in ("q", "k", "v", "a", "b"):
            t = getattr(self, name).detach().to("cpu").contiguous()
            h.update(t.view(torch.uint8).numpy().tobytes() if t.numel() else b"")
        return h.hexdigest()

    def token_slice(self, t0: int, t1: int, name=None) -> "GdnInputs":
        """Packed tokens [t0, t1) as one sequence."""
        return GdnInputs(name or f"{self.name}[{t0}:{t1}]", self.h_k, self.h_v, self.dk, self.dv,
                         self.chunk, self.io, cu_from_lengths([t1 - t0]), self.q[t0:t1],
                         self.k[t0:t1], self.v[t0:t1], self.a[t0:t1], self.b[t0:t1])

    def select(self, seqs) -> "GdnInputs":
        """A new batch holding the listed sequences, in the listed order."""
        cu = self.cu_seqlens.astype(np.int64)
        if len(seqs):
            idx = torch.from_numpy(np.concatenate([np.arange(cu[s], cu[s + 1]) for s in seqs])).to(self.device)
        else:
            idx = torch.zeros(0, dtype=torch.int64, device=self.device)
        lengths = [int(cu[s + 1] - cu[s]) for s in seqs]
        return GdnInputs(self.name + f"[sel{len(seqs)}]", self.h_k, self.h_v, self.dk, self.dv, self.chunk,
                         self.io, cu_from_lengths(lengths), self.q[idx], self.k[idx], self.v[idx],
                         self.a[idx], self.b[idx], dict(self.meta))

    @staticmethod
    def concat(parts, name="concat") -> "GdnInputs":
        p0 = parts[0]
        lengths = np.concatenate([p.lengths for p in parts])
        cat = lambda n: torch.cat([getattr(p, n) for p in parts], dim=0)
        return GdnInputs(name, p0.h_k, p0.h_v, p0.dk, p0.dv, p0.chunk, p0.io, cu_from_lengths(lengths),
                         cat("q"), cat("k"), cat("v"), cat("a"), cat("b"))


def _io_dtype(io: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[io]


def make_inputs(seed: int, lengths, h_k: int, h_v: int, dk: int, dv: int, chunk: int = 64,
                io: str = "bf16", name: str = "custom", sub: int = 0, device="cpu") -> GdnInputs:
    """Draw q, k, v, a, b for a packed batch of sequences with the given lengths."""
    lengths = [int(x) for x in lengths]
    n = int(sum(lengths))
    dev = torch.device(device)
    f64 = torch.float64
    dt = _io_dtype(io)

    def normal(purpose, shape):
        return torch.randn(shape, generator=_gen(seed, purpose, sub, dev), device=dev, dtype=f64)

    q = normal(_P_Q, (n, h_k, dk)).to(torch.float32).to(dt)
    k = normal(_P_K, (n, h_k, dk))
    k = (k / torch.sqrt(torch.sum(k * k, dim=-1, keepdim=True))).to(torch.float32).to(dt)
    v = normal(_P_V, (n, h_v, dv)).to(torch.float32).to(dt)
    a = torch.exp(-torch.nn.functional.softplus(normal(_P_A, (n, h_v)))).to(torch.float32)
    b = torch.sigmoid(normal(_P_B, (n, h_v))).to(torch.float32)
    return GdnInputs(name, h_k, h_v, dk, dv, chunk, io, cu_from_lengths(lengths), q.contiguous(),
                     k.contiguous(), v.contiguous(), a.contiguous(), b.contiguous(),
                     {"seed": seed, "sub": sub, "device": str(dev)})


def make_cotangents(x: GdnInputs, seed: int, with_d_state: bool = True, with_s0: bool = False,
                    device=None) -> dict:
    """Upstream gradients for a backward over x: d_o ~ N(0, 1) in x's io dtype [N, H_v, d_v];
    d_state ~ N(0, 1) fp32 [B, H_v, d_v, d_k] (state layout, or None); and, for a forward that
    continues from given states, s0 ~ N(0, 1/d_k) fp32 in the same layout (or None)."""
    dev = torch.device(device) if device is not None else x.device
    f64 = torch.float64
    n, B = x.total_tokens, x.num_seqs

    def normal(purpose, shape):
        return torch.randn(shape, generator=_gen(seed, purpose, 0, dev), device=dev, dtype=f64)

    out = {"d_o": normal(_P_DO, (n, x.h_v, x.dv)).to(torch.float32).to(_io_dtype(x.io)).contiguous(),
           "d_state": None, "s0": None}
    if with_d_state:
        out["d_state"] = normal(_P_DS, (B, x.h_v, x.dv, x.dk)).to(torch.float32).contiguous()
    if with_s0:
        out["s0"] = (normal(_P_S0, (B, x.h_v, x.dv, x.dk)) / x.dk ** 0.5).to(torch.float32).contiguous()
    return out


# ---------------------------------------------------------------------------------------------
# The five workloads.  Head layout for the large ones: 32 value heads over 16 key heads
# (value head h reads key head h // 2), d_k = d_v = 128, chunk 64.
# ---------------------------------------------------------------------------------------------
BIG = dict(h_k=16, h_v=32, dk=128, dv=128, chunk=64)


def tiny_fp32(device="cpu") -> GdnInputs:
    """Tiny fp32 case: one 256-token sequence, 2 heads, d_k = d_v = 16, chunk 64."""
    return make_inputs(0, [256], h_k=2, h_v=2, dk=16, dv=16, chunk=64, io="f32",
                       name="tiny-fp32-1x256", device=device)


def prefill_5x2048(num_seqs: int = 5, seqlen: int = 2048, device="cpu") -> GdnInputs:
    """Rollout prefill: 5 sequences x 2048 tokens, bf16 q/k/v."""
    return make_inputs(1, [seqlen] * num_seqs, io="bf16", name=f"prefill-{num_seqs}x{seqlen}",
                       device=device, **BIG)


def decode_prompt_lengths(num_seqs: int = 256, max_len: int = 2048) -> np.ndarray:
    return _np_rng(2, _P_LEN).integers(1, max_len + 1, size=num_seqs)


def decode_prompts(num_seqs: int = 256, max_len: int = 2048, device="cpu") -> GdnInputs:
    """Ragged prompts that seed the decode states (lengths uniform in [1, max_len])."""
    return make_inputs(2, decode_prompt_lengths(num_seqs, max_len), io="bf16",
                       name=f"decode-prompts-{num_seqs}", device=device, **BIG)


def decode_tokens(step: int, num_seqs: int = 256, device="cpu") -> GdnInputs:
    """The tokens of decode step ``step`` (one per sequence), drawn from their own streams."""
    return make_inputs(2, [1] * num_seqs, io="bf16", name=f"decode-step{step}", sub=1000 + step,
                       device=device, **BIG)


def trainer_lengths(total: int = 10240, lo: int = 64, hi: int = 4096, seed: int = 3) -> list:
    """Lengths in [lo, hi] summing exactly to ``total`` (draw while more than hi remains)."""
    rng = _np_rng(seed, _P_LEN)
    rem, out = total, []
    while rem > hi:
        L = int(rng.integers(lo, min(hi, rem - lo) + 1))
        out.append(L)
        rem -= L
    out.append(rem)
    rng.shuffle(out)
    return out


def trainer_10240(device="cpu") -> GdnInputs:
    """Trainer forward: 10240 tokens packed varlen, lengths in [64, 4096]."""
    return make_inputs(3, trainer_lengths(), io="bf16", name="trainer-10240-varlen", device=device, **BIG)


def long_sequence(seqlen: int = 65536, device="cpu") -> GdnInputs:
    """The long sequence X of the invariance sweep (large head layout, bf16)."""
    return make_inputs(4, [seqlen], io="bf16", name=f"long-{seqlen}", device=device, **BIG)


def neighbour_lengths(n_neighbours: int, sub: int, max_len: int = 8192) -> np.ndarray:
    return _np_rng(4, _P_LEN, sub).integers(1, max_len + 1, size=n_neighbours)


def long_in_batch(x: GdnInputs, batch: int, sub: int, max_len: int = 8192):
    """Embed the single sequence ``x`` among ``batch - 1`` random neighbours.

    Returns (inputs, index of x in the batch)."""
    if batch == 1:
        return x, 0
    lens = neighbour_lengths(batch - 1, sub, max_len)
    nb = make_inputs(4, lens, io=x.io, name="neighbours", sub=100 + sub, h_k=x.h_k, h_v=x.h_v,
                     dk=x.dk, dv=x.dv, chunk=x.chunk, device=x.device)
    pos = int(_np_rng(4, _P_PACK, sub).integers(0, batch))
    order = list(range(batch - 1))
    parts = [nb.select(order[:pos]), x, nb.select(order[pos:])]
    parts = [p for p in parts if p.num_seqs > 0]
    return GdnInputs.concat(parts, name=f"x-in-batch{batch}"), pos
