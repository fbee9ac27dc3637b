"""Seeded random configurations of the chunkwise (WY/UT) evaluation on matrix cores
(gdn_prefill_chunked, native outputs and the R2 reading): head dim, GQA ratio, chunk size, ragged
lengths (empty sequences included) and a continuation from given states at given positions drawn
together, so that combinations the targeted tests do not list are exercised too.  For each one:

- o, the final states and every chunk-start state against the fp64 oracle at the bf16-io bound of
  tests/test_gpu_chunked.py (the chunk form is not bit-identical to the recurrence);
- every sequence run alone gives the bits it gets inside the packed batch.
"""
import numpy as np
import pytest
import torch

import gdn_inputs as gi
from tests.gpu_util import lib, policy_of, say, sha
from tests.test_gpu_chunked import _check_vs_oracle, _chunked

pytestmark = pytest.mark.gpu


def _cases(n=8, seed=20261205):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        d = int(rng.choice([32, 64, 128]))
        h_k = int(rng.choice([1, 2]))
        ratio = int(rng.choice([1, 2, 4]))
        chunk = int(rng.choice([16, 20, 32, 64]))
        lens = [int(t) for t in rng.integers(0, 160, size=int(rng.integers(1, 6)))]
        mode = str(rng.choice(["native", "r2"]))
        cont = bool(rng.integers(0, 2))
        pos0 = [int(p) for p in rng.integers(0, 100, size=len(lens))] if cont else None
        out.append((c, d, h_k, ratio, chunk, lens, mode, pos0))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"case{c[0]}-d{c[1]}-r{c[3]}-C{c[4]}-{c[6]}"
                         f"{'-cont' if c[7] else ''}")
def test_random_chunked_configuration(case):
    c, d, h_k, ratio, chunk, lens, mode, pos0 = case
    cpr = lib()
    outputs = cpr.GDN_CHUNKED_NATIVE if mode == "native" else cpr.GDN_CHUNKED_R2
    say(f"random chunked config {case}")
    x = gi.make_inputs(6000 + c, lens, h_k=h_k, h_v=h_k * ratio, dk=d, dv=d, chunk=chunk, io="bf16")
    B = x.num_seqs
    S0 = None
    if pos0 is not None:
        S0 = gi.make_cotangents(x, 7000 + c, with_d_state=False, with_s0=True)["s0"]

    def run(xs, idx):
        pool = cpr.StatePool(policy_of(xs), max(xs.num_seqs, 1))
        if pos0 is not None:
            pool.state[: xs.num_seqs].copy_(S0[idx].to("cuda"))
            pool.pos[: xs.num_seqs].copy_(torch.tensor([pos0[i] for i in idx], dtype=torch.int64))
        return _chunked(xs, outputs, pool=pool, from_state=pos0 is not None)

    o, pool, cs = run(x, list(range(B)))
    _check_vs_oracle(x, o, pool, cs, S0=None if S0 is None else S0.double().numpy(), pos0=pos0)
    if pos0 is not None:
        assert pool.pos[:B].tolist() == [p + int(n) for p, n in zip(pos0, x.lengths)]
    for i in range(B):                                        # packing invariance
        t0, t1 = int(x.cu_seqlens[i]), int(x.cu_seqlens[i + 1])
        oi, pi, _ = run(x.select([i]), [i])
        assert sha(oi) == sha(o[t0:t1]) and sha(pi.state[0]) == sha(pool.state[i]), f"case {c}: sequence {i}"
