"""The pins must reject plausible mistakes: each mutant below is the oracle's recurrence with one
planted error (on the CPU); at least one pin in test_oracle_pins must fail for every mutant."""
import numpy as np
import pytest

import oracle.gdn_oracle as og
import tests.test_oracle_pins as pins


def _mutant(kind):
    def rec(q, k, v, a, b, S0=None, pos0=0, chunk=64):
        q, k, v, a, b = (np.asarray(x, np.float64) for x in (q, k, v, a, b))
        T, dk = k.shape
        dv = v.shape[1]
        S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64, copy=True)
        o = np.zeros((T, dv))
        rec_ = []
        for t in range(T):
            p = pos0 + t
            if kind != "record_late" and (t == 0 or p % chunk == 0):
                rec_.append(S.copy())
            u = (S @ k[t]) if kind == "transpose_u" else (S.T @ k[t])
            if kind == "drop_a_in_w":
                w = v[t] - u
            elif kind == "sign_w":
                w = v[t] + a[t] * u
            else:
                w = v[t] - a[t] * u
            Sold = S
            if kind == "drop_decay":
                S = S + b[t] * np.outer(k[t], w)
            elif kind == "drop_b":
                S = a[t] * S + np.outer(k[t], w)
            elif kind == "outer_swapped":
                S = a[t] * S + b[t] * np.outer(w[:dk], k[t][:dv]) if dk == dv else a[t] * S
            else:
                S = a[t] * S + b[t] * np.outer(k[t], w)
            if kind == "o_from_old_state":
                o[t] = Sold.T @ q[t]
            elif kind == "transpose_o":
                o[t] = S @ q[t]
            else:
                o[t] = S.T @ q[t]
            if kind == "record_late" and (t == 0 or p % chunk == 0):
                rec_.append(S.copy())
        R = np.stack(rec_) if rec_ else np.zeros((0, dk, dv))
        return o, S, R
    return rec


PIN_TESTS = [
    (pins.test_identity_gate_keeps_state, {}),
    (pins.test_delta_rule_projection_unit_key, {}),
    (pins.test_pure_decay, {}),
    (pins.test_zero_decay_rank_one, {}),
    (pins.test_exact_integer_vector, {}),
    (pins.test_unrolled_matrix_products, {}),
    (pins.test_exact_rational_dyadic, {}),
    (pins.test_boundary_rows_are_chunk_start_states, dict(pos0=5, length=60, chunk=64)),
    (pins.test_boundary_rows_are_chunk_start_states, dict(pos0=0, length=256, chunk=64)),
]


@pytest.mark.parametrize("kind", ["drop_a_in_w", "sign_w", "transpose_u", "drop_decay", "drop_b",
                                  "outer_swapped", "o_from_old_state", "transpose_o", "record_late"])
def test_some_pin_rejects_mutant(kind, monkeypatch):
    mutant = _mutant(kind)
    monkeypatch.setattr(pins, "recurrence", mutant)
    failed = []
    for fn, kw in PIN_TESTS:
        try:
            fn(**kw)
        except (AssertionError, ValueError):      # a shape error is a rejection too
            failed.append(fn.__name__)
    assert failed, f"mutant {kind} passed every pin"


def test_gqa_mutant_rejected(monkeypatch):
    """A driver that maps value head h to key head h % H_k must fail the packing/GQA pin."""
    real = og.recurrence

    def varlen_mod(q, k, v, a, b, cu_seqlens, h_k, h_v, S0=None, pos0=None, chunk=64):
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        B, N = len(cu) - 1, int(cu[-1])
        dk, dv = np.shape(k)[-1], np.shape(v)[-1]
        o = np.zeros((N, h_v, dv))
        S_fin = np.zeros((B, h_v, dk, dv))
        rows = []
        for i in range(B):
            t0, t1 = int(cu[i]), int(cu[i + 1])
            p0 = 0 if pos0 is None else int(pos0[i])
            per = []
            for h in range(h_v):
                g = h % h_k
                oh, sh, rh = real(q[t0:t1, g], k[t0:t1, g], v[t0:t1, h], a[t0:t1, h], b[t0:t1, h],
                                  S0=None if S0 is None else S0[i, h], pos0=p0, chunk=chunk)
                o[t0:t1, h], S_fin[i, h] = oh, sh
                per.append(rh)
            if t1 > t0:
                rows.append(np.stack(per, axis=1))
        return o, S_fin, (np.concatenate(rows) if rows else np.zeros((0, h_v, dk, dv)))

    monkeypatch.setattr(pins, "gdn_varlen", varlen_mod)
    with pytest.raises(AssertionError):
        pins.test_varlen_packing_and_gqa_mapping()
