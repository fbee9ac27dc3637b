"""Pins for the oracle's input widening and for the packed backward driver's chunk-state branch.

bf16_bits_to_f64 turns the bf16 bit patterns the GPU consumes into the fp64 values the oracle
computes with; every bf16 parity figure rests on it.  gdn_varlen_backward's chunk_states/row0
branch replaces the state at each chunk start with a row of a forward's stash (the trajectory a
forward actually took, needed for bf16 boundaries, section "The execution contract" of the
alphasignal.ai page on IsoExec: boundary dtypes are pinned constants).  Both are checked here
against facts that do not come from the oracle: the bf16 format itself, torch's own widening, and
the gradients the driver gives without the branch.
"""
import numpy as np
import pytest
import torch

import oracle.gdn_backward_oracle as gbo
from oracle import bf16_bits_to_f64, gdn_varlen, gdn_varlen_backward, num_boundary_rows


# --- bf16 widening ------------------------------------------------------------------------------

def test_bf16_widening_hand_values():
    """Values fixed by the bf16 format (sign, 8 exponent bits with bias 127, 7 fraction bits)."""
    cases = {
        0x0000: 0.0, 0x8000: -0.0, 0x3F80: 1.0, 0xBF80: -1.0, 0x4000: 2.0, 0xC040: -3.0,
        0x3F00: 0.5, 0x3FC0: 1.5, 0x4049: 3.140625, 0x0080: 2.0 ** -126, 0x0001: 2.0 ** -133,
        0x007F: 127 * 2.0 ** -133, 0x7F7F: (2 - 2.0 ** -7) * 2.0 ** 127, 0x7F80: np.inf, 0xFF80: -np.inf,
    }
    bits = np.array(list(cases), dtype=np.uint16)
    got = bf16_bits_to_f64(bits)
    want = np.array(list(cases.values()), dtype=np.float64)
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))      # -0.0 keeps its sign
    with np.errstate(invalid="ignore"):
        assert np.isnan(bf16_bits_to_f64(np.array([0x7FC0, 0xFFC1, 0x7F81], dtype=np.uint16))).all()


def test_bf16_widening_all_patterns_match_torch():
    """All 65,536 bit patterns: the oracle's widening equals torch's bf16 -> fp64 conversion,
    sign of zero included; NaN patterns widen to NaN.  A wrong shift or a dropped sign bit fails."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):          # NaN patterns pass through a float cast
        got = bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert nan.sum() == 2 * 127                       # exponent all ones with a nonzero fraction
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    # the widening is monotone on the non-negative patterns (value order = integer order)
    pos = got[: 0x7F81]
    assert np.all(np.diff(pos) > 0)


# --- the backward driver's chunk-state branch ----------------------------------------------------

def _packed(seed, lens, hk=1, hv=2, dk=4, dv=3):
    r = np.random.default_rng(seed)
    N = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    q, k = r.standard_normal((N, hk, dk)), r.standard_normal((N, hk, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v, dO = r.standard_normal((N, hv, dv)), r.standard_normal((N, hv, dv))
    a, b = r.uniform(0.3, 0.98, (N, hv)), r.uniform(0.2, 0.9, (N, hv))
    dST = r.standard_normal((len(lens), hv, dk, dv))
    return dict(q=q, k=k, v=v, a=a, b=b, dO=dO, cu=cu, hk=hk, hv=hv, dST=dST)


LENS = [9, 0, 13, 4, 1, 10]      # ragged: empty, exactly one chunk, one token, chunk + 1 ...
CHUNK = 4


def _rows(x, boundary):
    """The forward oracle's chunk-start rows and each sequence's first row."""
    _, _, R = gdn_varlen(x["q"], x["k"], x["v"], x["a"], x["b"], x["cu"], x["hk"], x["hv"], chunk=CHUNK,
                         boundary=boundary)
    n = [num_boundary_rows(0, L, CHUNK) for L in LENS]
    row0 = np.concatenate([[0], np.cumsum(n)[:-1]]).astype(np.int64)
    assert len(R) == sum(n)
    return R, row0


def _grads(x, fn=None, **kw):
    fn = fn or gdn_varlen_backward
    return fn(x["q"], x["k"], x["v"], x["a"], x["b"], x["dO"], x["cu"], x["hk"], x["hv"], dS_T=x["dST"],
              chunk=CHUNK, **kw)


def _assert_same(got, ref):
    for g, r, name in zip(got, ref, ("dq", "dk", "dv", "da", "db", "dS0")):
        scale = max(1.0, float(np.max(np.abs(r))))
        assert np.max(np.abs(g - r)) <= 1e-12 * scale, name


def test_chunk_states_of_the_fp32_forward_change_nothing(fn=None):
    """Fed the forward's own fp32 chunk-start rows, the driver restarts every chunk from the state
    the recurrence reaches there anyway, so the gradients are those of the call without rows (up
    to fp64 rounding: the forward forms b k w^T, the backward's replay k (b w)^T)."""
    x = _packed(0, LENS)
    R, row0 = _rows(x, "f32")
    _assert_same(_grads(x, fn, chunk_states=R, row0=row0), _grads(x))


def test_chunk_states_of_the_bf16_forward_give_the_bf16_gradients(fn=None):
    """Fed the rows of a bf16-boundary forward (rounded at every chunk start), the driver follows
    that trajectory: the gradients equal boundary="bf16", and differ from the fp32 ones."""
    x = _packed(1, LENS)
    R, row0 = _rows(x, "bf16")
    got = _grads(x, fn, chunk_states=R, row0=row0)
    _assert_same(got, _grads(x, boundary="bf16"))
    plain = _grads(x)
    assert not np.allclose(got[3], plain[3], rtol=1e-7, atol=0)


@pytest.mark.parametrize("pin", [test_chunk_states_of_the_fp32_forward_change_nothing,
                                 test_chunk_states_of_the_bf16_forward_give_the_bf16_gradients])
def test_row_offset_mutant_is_rejected(pin):
    """A driver that starts chunk c of sequence i from row row0[i] + c + 1 (an off-by-one row) must
    fail both pins.  The mutant is the real driver handed rows shifted by one, with one spare row
    so that the shift stays in bounds."""
    real = gbo.gdn_varlen_backward

    def off_by_one(*args, chunk_states=None, row0=None, **kw):
        if chunk_states is not None:
            spare = np.zeros((1,) + chunk_states.shape[1:])
            chunk_states = np.concatenate([chunk_states, spare])
            row0 = np.asarray(row0) + 1
        return real(*args, chunk_states=chunk_states, row0=row0, **kw)

    with pytest.raises(AssertionError):
        pin(fn=off_by_one)
