"""Host process pool that runs the fp64 oracle and the elementwise checks for the full-size GPU
parity tests, one (sequence, value head) per work item.

The pool is started by conftest.py at the start of a GPU test session, before any test touches the
GPU (a process that has initialised the GPU must not start programs), and holds at most 16 worker
processes.  Workers import numpy and the oracle only, never torch or the HIP library.  Without a
pool (a session that was not started for GPU tests) the same work items run in this process.
"""
from __future__ import annotations

import os

import numpy as np

POOL = None
WORKERS = 0


_ONE_THREAD = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")


def start(workers: int | None = None) -> None:
    """Start the pool.  Each worker's BLAS runs one thread: the variables are set in the environment
    the workers inherit (numpy reads them when a worker imports it) and restored afterwards, so the
    test process itself keeps its own settings."""
    global POOL, WORKERS
    if POOL is not None:
        return
    import multiprocessing as mp
    WORKERS = workers or max(1, min(16, os.cpu_count() or 1))
    saved = {k: os.environ.get(k) for k in _ONE_THREAD}
    try:
        for k in _ONE_THREAD:
            os.environ[k] = "1"
        POOL = mp.get_context("spawn").Pool(WORKERS)
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


def stop() -> None:
    global POOL
    if POOL is not None:
        POOL.close()
        POOL.join()
        POOL = None


def run(items, progress=None):
    """check_pair over every item, in the pool when there is one; returns the results in order."""
    out = []
    chunk = max(1, len(items) // (8 * max(WORKERS, 1)))
    it = POOL.imap(check_pair, items, chunksize=chunk) if POOL is not None else map(check_pair, items)
    for n, r in enumerate(it, 1):
        out.append(r)
        if progress is not None and (n % 32 == 0 or n == len(items)):
            progress(n)
    return out


def _widen(x, io):
    from oracle import bf16_bits_to_f64
    if io == "bf16" and x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    return np.asarray(x, np.float64)


def check_pair(item: dict) -> dict:
    """The oracle on one (sequence, value head) and every comparison with the GPU's results.

    item: label; io ("f32" or "bf16"); q, k [T, d_k] and v [T, d_v] (bf16 bit patterns as uint16,
    or fp32); a, b [T] fp32; S0 [d_k, d_v] fp64 or None; pos0, chunk; got_o [T, d_v] (uint16 bits
    or fp32); got_S [d_k, d_v] fp64 (math orientation) or None; got_rows [R, d_k, d_v] or None.
    Tolerances: fp32 io max-abs 1e-4 on o and S; bf16 io normwise 3e-3 on o and S, plus every o
    element within half a bf16 spacing and the fp32 error bound, at most one ulp from the oracle
    where well conditioned, and every state column within its error bound.  Returns a dict with
    ok, msg and the elementwise counts."""
    from oracle import recurrence
    from tests.bf16_check import (check_bf16_outputs, check_state_columns, kernel_dot_depth,
                                  output_error_bounds)
    io = item["io"]
    q, k, v = (_widen(item[n], io) for n in ("q", "k", "v"))
    a, b = np.asarray(item["a"], np.float64), np.asarray(item["b"], np.float64)
    S0 = item.get("S0")
    res = {"label": item["label"], "ok": True, "msg": "", "stats": None, "normwise_o": 0.0, "normwise_S": 0.0}
    try:
        o, S, R = recurrence(q, k, v, a, b, S0=S0, pos0=item.get("pos0", 0), chunk=item.get("chunk", 64))
        got_o = item["got_o"]
        go = _widen(got_o, io)
        nrm = lambda x, r: float(np.linalg.norm(x - r) / max(np.linalg.norm(r), 1e-300))
        res["normwise_o"] = nrm(go, o) if o.size else 0.0
        if io == "f32":
            assert o.size == 0 or np.max(np.abs(go - o)) <= 1e-4, f"o max-abs {np.max(np.abs(go - o)):.3e}"
        else:
            assert res["normwise_o"] <= 3e-3, f"o normwise {res['normwise_o']:.3e}"
            n0 = None if S0 is None else np.linalg.norm(S0, axis=0)[None]
            E, D, _ = output_error_bounds(q[:, None], k[:, None], v[:, None], a[:, None], b[:, None],
                                          depth=kernel_dot_depth(k.shape[1]), N0=n0)
            res["stats"] = check_bf16_outputs(got_o, o, E[:, 0], item["label"])
        if item.get("got_S") is not None:
            gS = item["got_S"]
            res["normwise_S"] = nrm(gS, S)
            if io == "f32":
                assert np.max(np.abs(gS - S)) <= 1e-4, f"S max-abs {np.max(np.abs(gS - S)):.3e}"
            else:
                assert res["normwise_S"] <= 3e-3, f"S normwise {res['normwise_S']:.3e}"
                check_state_columns(gS, S, D[0], item["label"] + " final state")
        rows = item.get("got_rows")
        if rows is not None:
            assert len(rows) == len(R), f"{len(rows)} chunk-start rows, oracle has {len(R)}"
            for r in range(len(R)):
                if io == "f32":
                    assert np.max(np.abs(rows[r] - R[r])) <= 1e-4, f"row {r}"
                else:
                    assert nrm(rows[r], R[r]) <= 3e-3, f"row {r} normwise {nrm(rows[r], R[r]):.3e}"
    except AssertionError as e:
        res["ok"] = False
        res["msg"] = f"{item['label']}: {e}"
    return res


def summarize(results) -> dict:
    """Totals of the elementwise counts over many work items."""
    tot = {"elements": 0, "ulp0": 0, "ulp1": 0, "ulp_more": 0, "ill_conditioned": 0}
    worst = 0.0
    for r in results:
        if r["stats"]:
            for key in tot:
                tot[key] += r["stats"][key]
            worst = max(worst, r["stats"]["max_err_over_bound"])
    tot["max_err_over_bound"] = worst
    tot["max_normwise_o"] = max((r["normwise_o"] for r in results), default=0.0)
    tot["max_normwise_S"] = max((r["normwise_S"] for r in results), default=0.0)
    return tot
