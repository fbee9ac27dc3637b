#!/usr/bin/env python3
"""Benchmark of CPR Gated DeltaNet on one MI355X.

Step = one gdn_prefill over the rollout-prefill workload: 5 sequences x 2048 tokens, 32 value
heads over 16 key heads, d_k = d_v = 128, chunk 64, bf16 q/k/v/o, fp32 a/b/state (both passes
plus the position update).  value = tokens per second of that step.  Alongside: the rollout
decode workload (256 slots seeded by prefilling ragged prompts of 1..2048 tokens, then 128 timed
decode steps of one token each), reported as microseconds per step.

Timing: W untimed warm-up steps, then K steps bracketed by torch.cuda.synchronize(); per-kernel
durations come from HIP events the library records on the launch stream around each pass.
Inputs are seeded synthetic tensors already resident in HBM.  The fp64 oracle is timed on the
host over the same prefill workload (a process pool started before the GPU is touched).
Prints one JSON line.
"""
import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "CPR-GDN prefill tok/s (5×2048) + decode µs/step (256×1), % HBM peak"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector (256 CU x 2.4 GHz x 256 FLOP/clk/CU)
FP32_UNPACKED_PEAK_TFLOPS = 78.6  # the same without packed fp32 (the kernels are compiled without it)
FP32_MFMA_PEAK_TFLOPS = 157.3    # MI355X dense fp32 matrix-core peak


# ------------------------------------------------------------------ CPU baseline (oracle) worker
def _oracle_item(item):
    """Run the oracle on one (sequence, value head); inputs are bf16 bit patterns (uint16) or fp32,
    then an optional initial state (fp64, math orientation) and start position."""
    import numpy as np
    from oracle import bf16_bits_to_f64, recurrence
    q, k, v, a, b = item[:5]
    S0, pos0 = (item[5], item[6]) if len(item) > 5 else (None, 0)
    w = lambda x: bf16_bits_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)
    t = time.perf_counter()
    o, S, _ = recurrence(w(q), w(k), w(v), w(a), w(b), S0=S0, pos0=pos0, chunk=64)
    return o, S, time.perf_counter() - t


def _parity(groups, tol=3e-3):
    """Compare the oracle's (o, S) with the GPU's bf16 outputs and fp32 states, one group per
    sequence (or slot) with all its value heads: normwise per (sequence, head) (the tolerance), and
    element by element against the fp32 forward error bound of tests/bf16_check.py (every output
    within half a bf16 spacing plus the bound; well-conditioned outputs at most one ulp from the
    oracle; each final-state column within its bound).  A group is (oracle results per head,
    got_bits [T, H, d_v] uint16, got_S [H, d_k, d_v], inputs (q, k [T, H, d_k], v [T, H, d_v],
    a, b [T, H]) as fp64, S0 [H, d_k, d_v] or None)."""
    import numpy as np
    from tests.bf16_check import check_bf16_outputs, check_state_columns, kernel_dot_depth, output_error_bounds
    worst_o = worst_S = 0.0
    tot = {"elements": 0, "ulp0": 0, "ulp1": 0, "ulp_more": 0, "ill_conditioned": 0}
    failures = []
    nrm = lambda x, r: float(np.linalg.norm(x - r) / max(np.linalg.norm(r), 1e-300))
    for res, gb, gS, (q, k, v, a, b), S0 in groups:
        ro = np.stack([r[0] for r in res], axis=1)                     # [T, H, d_v]
        go = (np.asarray(gb, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        n0 = None if S0 is None else np.linalg.norm(S0, axis=1)
        E, D, _ = output_error_bounds(q, k, v, a, b, depth=kernel_dot_depth(k.shape[-1]), N0=n0)
        for h, r in enumerate(res):
            worst_o, worst_S = max(worst_o, nrm(go[:, h], r[0])), max(worst_S, nrm(gS[h], r[1]))
        try:
            st = check_bf16_outputs(gb, ro, E, "o")
            for h, r in enumerate(res):
                check_state_columns(gS[h], r[1], D[h], f"final state head {h}")
            for key in tot:
                tot[key] += st[key]
        except AssertionError as e:
            failures.append(str(e)[:200])
    ok = worst_o <= tol and worst_S <= tol and not failures
    return {"ok": ok, "max_normwise_o": worst_o, "max_normwise_S": worst_S, "tolerance": tol,
            "elementwise": tot, "elementwise_failures": failures[:3],
            "elementwise_note": "every output within half a bf16 spacing plus a forward error bound of the fp32 "
                                "arithmetic; well-conditioned outputs (2^-9 |o| above the bound) at most one bf16 "
                                "ulp from the oracle rounded to fp32 and then bf16; each final-state column within "
                                "its error bound"}


def _start_pool(workers):
    import multiprocessing as mp
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    os.environ["OPENBLAS_NUM_THREADS"] = "1"
    os.environ["MKL_NUM_THREADS"] = "1"
    return mp.get_context("spawn").Pool(workers)


# ------------------------------------------------------------------ HIP events via the runtime
class Hip:
    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        ev = ctypes.c_void_p()
        rc = self.lib.hipEventCreate(ctypes.byref(ev))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return ev

    def record(self, ev, stream_ptr):
        rc = self.lib.hipEventRecord(ev, ctypes.c_void_p(stream_ptr))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def ms(self, e0, e1) -> float:
        out = ctypes.c_float()
        rc = self.lib.hipEventElapsedTime(ctypes.byref(out), e0, e1)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(out.value)


# Sources the profiled forward kernels (prefill passes and decode step) are built from.
FORWARD_SOURCES = ("cpr_args.hpp", "cpr_common.hpp", "cpr_decode.hip", "cpr_prefill.hip", "cpr_schedule.hpp",
                   "cpr_step.hpp")


def kernel_source_digest() -> str:
    """SHA-256 over the forward kernels' sources (name + bytes, sorted), to tie stored counters to
    the code they were taken on."""
    import hashlib
    csrc = os.path.join(ROOT, "bitwise_aligned_gated_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(FORWARD_SOURCES):
        h.update(name.encode())
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch from the committed FETCH_SIZE/WRITE_SIZE counters, or {} when the
    kernel sources changed since they were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as fh:
            tr = json.load(fh)
    except (OSError, ValueError):
        return {}
    if tr.get("fingerprint") != kernel_source_digest():
        return {}
    return {k: v["bytes"] for k, v in tr.get("kernels", {}).items()}


def prefill_flops(lengths, h_v, dk, dv, chunk, stash=True):
    """Algorithmic FLOPs of the two passes.  Per token-head, the step is u = S^T k (2 dk dv), a*S
    (dk dv) and k c^T added (2 dk dv); the output o = S^T q adds 2 dk dv.
    With the c stash: pass 1 runs every token without output (5 dk dv) and pass 2 applies the kept
    c with output (a*S, k c^T, o: 5 dk dv).  Without it: pass 1 runs the tokens up to each
    sequence's last chunk start (5 dk dv) and pass 2 the whole step with output (7 dk dv)."""
    p2_tokens = sum(lengths)
    if stash:
        return p2_tokens * h_v * 5 * dk * dv, p2_tokens * h_v * 5 * dk * dv, p2_tokens
    p1_tokens = sum(max(0, ((L - 1) // chunk) * chunk) for L in lengths if L > 0)
    return p1_tokens * h_v * 5 * dk * dv, p2_tokens * h_v * 7 * dk * dv, p1_tokens


def backward_flops(lengths, h_v, dk, dv, chunk):
    """Algorithmic FLOPs of the trainer backward's kernels, per value head and token:
    adjoint  G + q dO^T (2), dc = (.)^T k (2) and a G + k du^T (3): 7 dk dv over every token;
    replay   the forward step without output: 5 dk dv;
    chunk gradients (matrix cores), per chunk of L tokens: three L x d x d products
             (dO S0^T, dU S0^T, C G_L^T) and five L x L x d products (dO C^T, dU C^T and the three
             decay-masked products with K, Q, K): 6 L d^2 + 10 L^2 d."""
    n = sum(lengths)
    chunks = []
    for L in lengths:
        chunks += [chunk] * (L // chunk) + ([L % chunk] if L % chunk else [])
    mfma = sum(6 * c * dk * dv + 10 * c * c * dk for c in chunks) * h_v
    return n * h_v * 7 * dk * dv, n * h_v * 5 * dk * dv, mfma


def normwise_t(got, ref) -> float:
    """||got - ref|| / ||ref|| of two device tensors, in fp64."""
    import torch
    g, r = got.double(), ref.double()
    den = float(torch.linalg.vector_norm(r))
    return float(torch.linalg.vector_norm(g - r)) / den if den > 0 else float(torch.linalg.vector_norm(g))


def prefill_bytes(lengths, h_k, h_v, dk, dv, chunk, io=2):
    """HBM bytes of a two-pass prefill from zero states over sequences of the given lengths.
    Returns (algorithmic, c stash one way, pass 1 as built, pass 2 as built):
      algorithmic  the I/O (q, k per key head, v, a, b read; o and the final states written), pass
                   1's second read of k, v, a, b for the tokens before each sequence's last chunk
                   start, and every chunk-start state after a sequence's first written once and read
                   once;
      c stash      every token's c (fp32), written by pass 1 and read by pass 2 in this build;
      pass 1 / 2   what each kernel moves as built: pass 1 reads k, v, a, b of every token and writes
                   every chunk-start row and the c stash; pass 2 reads q, k, a, every row and the
                   stash and writes o and the final states."""
    n, B = sum(lengths), len(lengths)
    n_rows = sum(0 if L == 0 else 1 + (L - 1) // chunk for L in lengths)
    plane = h_v * dk * dv * 4
    tok_kvab = h_k * dk * io + h_v * dv * io + 2 * h_v * 4
    io_bytes = n * (2 * h_k * dk * io + 2 * h_v * dv * io + 2 * h_v * 4) + B * plane
    p1_tokens = sum(max(0, ((L - 1) // chunk) * chunk) for L in lengths if L > 0)
    alg = io_bytes + p1_tokens * tok_kvab + 2 * (n_rows - B) * plane
    c_bytes = n * h_v * dv * 4
    pass1 = n * tok_kvab + n_rows * plane + c_bytes
    pass2 = n * (2 * h_k * dk * io + h_v * 4) + n_rows * plane + c_bytes + n * h_v * dv * io + B * plane
    return alg, c_bytes, pass1, pass2


def decode_bytes(batch, h_k, h_v, dk, dv, io_bytes=2):
    """Algorithmic HBM bytes of one decode step: the state read and written once, the token's
    q, k (per key head), v, a, b read and o written."""
    state = 2 * batch * h_v * dk * dv * 4
    tokens = batch * (2 * h_k * dk * io_bytes + 2 * h_v * dv * io_bytes + 2 * h_v * 4)
    return state + tokens


def host_environment():
    """Host-side facts for the record, gathered before anything touches the GPU: the CPU model,
    the numpy version and the GPU clocks rocm-smi reports before the run, i.e. at idle (None where
    a tool is missing)."""
    import subprocess
    env = {"cpu_model": None, "host_cpus": os.cpu_count(), "numpy": None, "gpu_clocks_idle": None}
    try:
        with open("/proc/cpuinfo") as fh:
            env["cpu_model"] = next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")), None)
    except OSError:
        pass
    try:
        import numpy
        env["numpy"] = numpy.__version__
    except ImportError:
        pass
    try:
        # under a profiler that loads its tool library into this process, the GPU is initialised
        # before main() runs, and a child started from here may not replace itself by exec
        with open("/proc/self/maps") as fh:
            if "rocprofiler" in fh.read():
                return env
    except OSError:
        pass
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=20)
        if r.returncode == 0:
            card = next(iter(json.loads(r.stdout).values()), {})
            env["gpu_clocks_idle"] = {k: v for k, v in card.items() if "clock" in k.lower() or k.lower().startswith(("sclk", "mclk", "fclk", "socclk"))} or card
    except (OSError, ValueError, subprocess.SubprocessError, StopIteration, AttributeError):
        pass
    return env


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # 20 warm-up calls: the first ~20 prefill calls of a process run up to ~30% slower than the steady
    # state, because the GPU lowers its clocks while idle (here while the first call loads the code
    # object) and raises them over ~20 ms of load; fewer warm-up calls time part of that ramp
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--decode-steps", type=int, default=128)
    ap.add_argument("--no-decode", action="store_true", help="skip the decode workload")
    ap.add_argument("--no-trainer", action="store_true", help="skip the trainer forward+backward workload")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip timing the oracle")
    ap.add_argument("--no-long", action="store_true", help="skip the single 65536-token sequence")
    ap.add_argument("--cpu-workers", type=int, default=min(16, os.cpu_count() or 1))
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 256 MiB fp32 copy kernel (torch.neg) 3 times, a known-size "
                         "reference for HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the CPR kernels are "
              "benchmarked on a single MI355X", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        sys.exit("--steps must be >= 1 and --warmup >= 0")

    host_env = host_environment()
    pool = None if args.no_cpu_baseline else _start_pool(args.cpu_workers)

    import numpy as np
    import torch

    import bitwise_aligned_gated_amd as cpr
    import gdn_inputs as gi

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    hip = Hip()
    stream = torch.cuda.current_stream().cuda_stream

    if args.copy_calibration:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)        # 256 MiB
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    # ---------------------------------------------------------------- prefill (the timed step)
    x = gi.prefill_5x2048(device=dev)
    P = cpr.Policy(x.h_k, x.h_v, x.dk, x.dv, x.chunk, x.io)
    N, B = x.total_tokens, x.num_seqs
    spool = cpr.StatePool(P, B, device=dev)
    rows = cpr.gdn_chunk_rows_bound(N, B, P.chunk)
    cs = torch.empty((rows, P.h_v, P.dv, P.dk), dtype=torch.float32, device=dev)
    o = torch.empty((N, P.h_v, P.dv), dtype=torch.bfloat16, device=dev)
    cu = torch.from_numpy(x.cu_seqlens).to(dev)
    ids = torch.arange(B, dtype=torch.int32, device=dev)
    stash = torch.empty((N, P.h_v, P.dv), dtype=torch.float32, device=dev)   # every token's c

    def step(events=None, c_stash=stash, pool=spool, out=o):
        cpr.gdn_prefill(pool, cu, x.q, x.k, x.v, x.a, x.b, slot_ids=ids, o=out, chunk_states=cs, c_stash=c_stash,
                        events=events)

    def timed(call, n_events):
        """args.warmup untimed calls, then args.steps timed ones: (ms per call, events per call)."""
        for _ in range(args.warmup):
            call(None)
        evs_ = [[hip.event() for _ in range(n_events)] for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0_ = time.perf_counter()
        for i_ in range(args.steps):
            call(evs_[i_])
        torch.cuda.synchronize()
        return (time.perf_counter() - t0_) * 1e3 / args.steps, evs_

    # The context legs of this workload run first, back to back on the GPU, and their host-side
    # checks wait until after the timed step: the timed step then runs at the clocks a busy GPU
    # holds (they drop while it idles and take ~20 ms of load to come back), whatever the warm-up
    # count.  Its own warm-up calls still precede it.
    # the same call without the c stash (pass 2 predicts every c again): context, same bits
    npool = cpr.StatePool(P, B, device=dev)
    on = torch.empty_like(o)
    n_ms, nevs = timed(lambda ev: step(ev, c_stash=None, pool=npool, out=on), 3)
    # the one-pass variant ("recurrent everywhere" in the pages' table); context only
    fpool = cpr.StatePool(P, B, device=dev)
    of = torch.empty_like(o)
    fused_ms, fevs = timed(lambda ev: cpr.gdn_prefill_fused(fpool, cu, x.q, x.k, x.v, x.a, x.b, slot_ids=ids, o=of,
                                                            events=ev), 2)
    # the chunkwise evaluation on matrix cores, both output modes ("native" in the pages' table,
    # and the R2 reading); context only, not bit-identical to CPR
    chunk_runs = {}
    cws = torch.empty(cpr.gdn_prefill_chunked_workspace_bytes(P, N, B), dtype=torch.uint8, device=dev)
    for label, mode in (("native", cpr.GDN_CHUNKED_NATIVE), ("r2", cpr.GDN_CHUNKED_R2)):
        cpool = cpr.StatePool(P, B, device=dev)
        oc = torch.empty_like(o)
        c_ms, cevs = timed(lambda ev, cpool=cpool, oc=oc, mode=mode: cpr.gdn_prefill_chunked(
            cpool, cu, x.q, x.k, x.v, x.a, x.b, slot_ids=ids, outputs=mode, o=oc, chunk_states=cs, workspace=cws,
            events=ev), 4)
        chunk_runs[label] = (c_ms, cevs, oc)
        del cpool
    del cws

    # the timed step
    ms_step, evs = timed(lambda ev: step(ev), 3)
    p1_ms = statistics.mean(hip.ms(e[0], e[1]) for e in evs)
    p2_ms = statistics.mean(hip.ms(e[1], e[2]) for e in evs)
    f1, f2, p1_tokens = prefill_flops([int(l) for l in x.lengths], P.h_v, P.dk, P.dv, P.chunk)
    kernels = {
        "boundary_pass": {"avg_ms": p1_ms, "tflops": f1 / (p1_ms * 1e-3) / 1e12, "flop": f1},
        "output_pass": {"avg_ms": p2_ms, "tflops": f2 / (p2_ms * 1e-3) / 1e12, "flop": f2},
    }
    dom = max(kernels, key=lambda k: kernels[k]["avg_ms"])
    traffic = measured_traffic()
    roofline = {"bound": "alu", "kernel": dom, "achieved": round(kernels[dom]["tflops"], 3),
                "peak": FP32_VECTOR_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(kernels[dom]["tflops"] / FP32_VECTOR_PEAK_TFLOPS, 4),
                "traffic": traffic.get(dom),
                "peak_unpacked": FP32_UNPACKED_PEAK_TFLOPS,
                "frac_unpacked": round(kernels[dom]["tflops"] / FP32_UNPACKED_PEAK_TFLOPS, 4)}
    # prefill HBM fraction (the metric's "% HBM peak"), on the method's algorithmic bytes: the I/O
    # (q, k per key head, v, a, b, o, final states), pass 1's second read of k, v, a, b up to each
    # sequence's last chunk start, and every chunk-start state after the first written once and read
    # once.  The c stash this build adds (each token's c written by pass 1 and read by pass 2) is a
    # trade of bytes for pass-2 arithmetic, not algorithmic traffic: its bytes are reported apart.
    alg_bytes, c_bytes, pass1_bytes, pass2_bytes = prefill_bytes([int(l) for l in x.lengths], P.h_k, P.h_v,
                                                                  P.dk, P.dv, P.chunk)
    kernels["boundary_pass"]["bytes"] = int(pass1_bytes)
    kernels["output_pass"]["bytes"] = int(pass2_bytes)
    prefill_gbs = alg_bytes / (ms_step * 1e-3) / 1e9

    # parity of the timed prefill output against the oracle (computed in the CPU leg below)
    o_bits = o.view(torch.int16).cpu().numpy().view(np.uint16)
    S_host = spool.state.cpu().numpy()
    digest_two_pass = hashlib.sha256(o.view(torch.int16).cpu().numpy().tobytes()).hexdigest()
    # SHA-256 identity digests of the timed call (the execution contract's admission check):
    # inputs (q, k, v, a, b bytes in that order), o, and the final states
    hin = hashlib.sha256()
    for t in (x.q, x.k, x.v, x.a, x.b):
        hin.update(t.contiguous().view(torch.uint8).cpu().numpy().tobytes())
    identity = {"inputs": hin.hexdigest(), "o": digest_two_pass,
                "final_state": hashlib.sha256(spool.state.view(torch.uint8).cpu().numpy().tobytes()).hexdigest()}

    # the context legs' results, checked against the timed step's
    nf1, nf2, _ = prefill_flops([int(l) for l in x.lengths], P.h_v, P.dk, P.dv, P.chunk, stash=False)
    n1 = statistics.mean(hip.ms(e[0], e[1]) for e in nevs)
    n2 = statistics.mean(hip.ms(e[1], e[2]) for e in nevs)
    no_stash = {"ms_per_step": round(n_ms, 4), "tok_s": round(N / (n_ms * 1e-3), 1),
                "boundary_pass_ms": round(n1, 4), "output_pass_ms": round(n2, 4),
                "boundary_pass_tflops": round(nf1 / (n1 * 1e-3) / 1e12, 3),
                "output_pass_tflops": round(nf2 / (n2 * 1e-3) / 1e12, 3),
                "bitwise_equal_to_stash": hashlib.sha256(on.view(torch.int16).cpu().numpy().tobytes()).hexdigest()
                == digest_two_pass and bool(torch.equal(npool.state, spool.state))}
    del npool, on
    fused_kernel_ms = statistics.mean(hip.ms(e[0], e[1]) for e in fevs)
    fused = {"ms_per_step": round(fused_ms, 4), "kernel_ms": round(fused_kernel_ms, 4),
             "tok_s": round(N / (fused_ms * 1e-3), 1),
             "bitwise_equal_to_two_pass": hashlib.sha256(of.view(torch.int16).cpu().numpy().tobytes()).hexdigest()
             == digest_two_pass}
    del fpool, of
    chunked = {}
    for label, (c_ms, cevs, oc) in chunk_runs.items():
        stage = [statistics.mean(hip.ms(e[j], e[j + 1]) for e in cevs) for j in range(3)]
        d_o = (oc.float() - o.float()).norm() / o.float().norm()
        chunked[label] = {"ms_per_step": round(c_ms, 4), "tok_s": round(N / (c_ms * 1e-3), 1),
                          "stages_ms": {"prep": round(stage[0], 4), "state": round(stage[1], 4),
                                        "output": round(stage[2], 4)},
                          "normwise_o_vs_cpr": float(d_o), "cpr_over_this": round(ms_step / c_ms, 3)}
    del chunk_runs

    # one 65536-token sequence (the invariance workload's X): where pass 1's chain of sequential
    # steps is the critical path, the two-pass prefill against the one-pass and overlapped
    # variants; context only
    long_seq = None
    if not args.no_long:
        xl = gi.long_sequence(device=dev)
        NL = xl.total_tokens
        cul = torch.from_numpy(xl.cu_seqlens).to(dev)
        idl = torch.zeros(1, dtype=torch.int32, device=dev)
        ol = torch.empty((NL, P.h_v, P.dv), dtype=torch.bfloat16, device=dev)
        csl = torch.empty((cpr.gdn_chunk_rows_bound(NL, 1, P.chunk), P.h_v, P.dv, P.dk), dtype=torch.float32,
                          device=dev)
        stl = torch.empty((NL, P.h_v, P.dv), dtype=torch.float32, device=dev)
        lpool = cpr.StatePool(P, 1, device=dev)
        runs = {"two_pass": lambda ev: cpr.gdn_prefill(lpool, cul, xl.q, xl.k, xl.v, xl.a, xl.b, slot_ids=idl, o=ol,
                                                       chunk_states=csl, c_stash=stl, events=ev),
                "one_pass": lambda ev: cpr.gdn_prefill_fused(lpool, cul, xl.q, xl.k, xl.v, xl.a, xl.b, slot_ids=idl,
                                                             o=ol, events=ev),
                "overlapped": lambda ev: cpr.gdn_prefill_overlapped(lpool, cul, xl.q, xl.k, xl.v, xl.a, xl.b,
                                                                    slot_ids=idl, o=ol, events=ev)}
        long_seq = {"workload": f"one sequence of {NL} tokens, the prefill head layout"}
        digests = {}
        for label, run in runs.items():
            nev = 3 if label == "two_pass" else 2
            run(None)
            lev = [[hip.event() for _ in range(nev)] for _ in range(3)]
            torch.cuda.synchronize()
            for e in lev:
                run(e)
            torch.cuda.synchronize()
            k_ms = [hip.ms(e[0], e[-1]) for e in lev]
            entry = {"ms": round(statistics.median(k_ms), 4), "tok_s": round(NL / (statistics.median(k_ms) * 1e-3), 1)}
            if label == "two_pass":
                entry["boundary_pass_ms"] = round(statistics.median(hip.ms(e[0], e[1]) for e in lev), 4)
                entry["output_pass_ms"] = round(statistics.median(hip.ms(e[1], e[2]) for e in lev), 4)
            long_seq[label] = entry
            digests[label] = hashlib.sha256(ol.view(torch.int16).cpu().numpy().tobytes()).hexdigest()
        long_seq["bitwise_equal"] = digests["two_pass"] == digests["one_pass"] == digests["overlapped"]
        del xl, ol, csl, stl, lpool

    # ---------------------------------------------------------------- decode workload
    decode = None
    dec_host = None
    if not args.no_decode:
        prompts = gi.decode_prompts(device=dev)
        nb = prompts.num_seqs
        dpool = cpr.StatePool(P, nb, device=dev)
        cpr.gdn_prefill(dpool, prompts.cu_seqlens, prompts.q, prompts.k, prompts.v, prompts.a, prompts.b)
        del prompts
        toks = [gi.decode_tokens(s, nb, device=dev) for s in range(args.decode_steps)]
        od = torch.empty((nb, P.h_v, P.dv), dtype=torch.bfloat16, device=dev)
        dids = torch.arange(nb, dtype=torch.int32, device=dev)
        wpool = cpr.StatePool(P, nb, device=dev)          # warm-up on a copy; the real states stay put
        wpool.state.copy_(dpool.state)
        wpool.pos.copy_(dpool.pos)
        for s in range(args.warmup):
            t = toks[s % len(toks)]
            cpr.gdn_decode_step(wpool, t.q, t.k, t.v, t.a, t.b, slot_ids=dids, o=od)
        del wpool
        snap_state, snap_pos = dpool.state.clone(), dpool.pos.clone()   # for the boundary-record run
        dec_lens = [int(p) for p in snap_pos.tolist()]
        start_host = snap_state.cpu().numpy() if pool is not None else None   # for the oracle leg
        torch.cuda.synchronize()
        devs = [[hip.event() for _ in range(3)] for _ in range(args.decode_steps)]
        t0 = time.perf_counter()
        dec_outs = [torch.empty_like(od) for _ in range(args.decode_steps)]   # every step's outputs
        for s in range(args.decode_steps):
            t = toks[s]
            cpr.gdn_decode_step(dpool, t.q, t.k, t.v, t.a, t.b, slot_ids=dids, o=dec_outs[s], events=devs[s][:2])
            hip.record(devs[s][2], stream)
        torch.cuda.synchronize()
        od = dec_outs[-1]
        dwall = time.perf_counter() - t0
        k_us = sorted(hip.ms(e[0], e[1]) * 1e3 for e in devs)
        call_us = sorted(hip.ms(e[0], e[2]) * 1e3 for e in devs)
        med = statistics.median(k_us)
        dbytes = decode_bytes(nb, P.h_k, P.h_v, P.dk, P.dv)
        k_avg_us = statistics.mean(k_us)
        decode = {
            "workload": "decode 256x1, 128 steps, slots seeded by ragged prompts 1..2048",
            "us_per_step_median": round(statistics.median(call_us), 2),
            "us_per_step_p90": round(call_us[int(0.9 * (len(call_us) - 1))], 2),
            "kernel_us_median": round(med, 2),
            "wall_us_per_step": round(dwall * 1e6 / args.decode_steps, 2),
            "hbm_frac": round(dbytes / (statistics.median(call_us) * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "roofline": {"bound": "hbm", "kernel": "decode_step", "achieved": round(dbytes / (k_avg_us * 1e-6) / 1e9, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(dbytes / (k_avg_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                         "traffic": traffic.get("decode_step"), "bytes_per_step": dbytes},
        }
        # The same steps through a pool with a boundary record: every chunk start is committed to
        # the record and a second kernel advances the positions.  Same bits as the steps above.
        rpool = cpr.StatePool(P, nb, device=dev, boundary=True)
        rpool.state.copy_(snap_state)
        rpool.pos.copy_(snap_pos)
        del snap_state, snap_pos
        od_r = torch.empty_like(od)
        revs = [[hip.event() for _ in range(2)] for _ in range(args.decode_steps)]
        for s in range(args.decode_steps):
            t = toks[s]
            cpr.gdn_decode_step(rpool, t.q, t.k, t.v, t.a, t.b, slot_ids=dids, o=od_r, events=revs[s])
        torch.cuda.synchronize()
        r_us = statistics.median(hip.ms(e[0], e[1]) * 1e3 for e in revs)
        decode["with_boundary_record"] = {
            "us_per_step_median": round(r_us, 2),
            "bitwise_equal": bool(torch.equal(rpool.state, dpool.state) and torch.equal(rpool.pos, dpool.pos)
                                  and torch.equal(od_r.view(torch.int16), od.view(torch.int16))),
        }
        del rpool, od_r
        if pool is not None:
            # host copies for the oracle leg: the states the prompts left (fp32, exact in fp64), the
            # 128 tokens of every slot and every decode output of the timed steps
            u16 = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
            dec_host = {"S0": start_host, "final": dpool.state.cpu().numpy(), "lens": dec_lens,
                        "q": np.stack([u16(t.q) for t in toks], 1), "k": np.stack([u16(t.k) for t in toks], 1),
                        "v": np.stack([u16(t.v) for t in toks], 1),
                        "a": np.stack([t.a.cpu().numpy() for t in toks], 1),
                        "b": np.stack([t.b.cpu().numpy() for t in toks], 1),
                        "o": np.stack([u16(o_) for o_ in dec_outs], 1)}
        # the same workload under the R2 reading: prompts prefilled by the chunk form (GDN_CHUNKED_R2),
        # decode resynchronising with the chunk form at every chunk start (context; other values)
        prompts = gi.decode_prompts(device=dev)
        r2pool = cpr.StatePool(P, nb, device=dev, boundary=True)
        r2pool.attach_r2()
        cpr.gdn_prefill_chunked(r2pool, prompts.cu_seqlens, prompts.q, prompts.k, prompts.v, prompts.a, prompts.b,
                                outputs=cpr.GDN_CHUNKED_R2)
        del prompts
        torch.cuda.synchronize()
        r2evs = [[hip.event() for _ in range(2)] for _ in range(args.decode_steps)]
        od2 = torch.empty_like(od)
        for s in range(args.decode_steps):
            t = toks[s]
            cpr.gdn_decode_step(r2pool, t.q, t.k, t.v, t.a, t.b, slot_ids=dids, o=od2, events=r2evs[s])
        torch.cuda.synchronize()
        r2_us = sorted(hip.ms(e[0], e[1]) * 1e3 for e in r2evs)
        starts = sum(1 for s in range(args.decode_steps) for L in dec_lens if (L + s) % P.chunk == 0)
        decode["r2_reading"] = {
            "us_per_step_median": round(statistics.median(r2_us), 2),
            "us_per_step_max": round(r2_us[-1], 2),
            "resyncs": starts,
            "note": "prompts by gdn_prefill_chunked(R2); each step runs the chunk form over the token ring of "
                    "the slots at a chunk start (listed on the device; 512 workgroups take them in turn), then their "
                    "pinned step, on a second stream beside the other slots' step; ring and workspace "
                    f"{(r2pool.r2_ring.numel() + r2pool.r2_workspace.numel()) / 2**20:.0f} MiB"}
        del r2pool, od2

    # ---------------------------------------------------------------- trainer forward + backward
    trainer = None
    if not args.no_trainer:
        xt = gi.trainer_10240(device=dev)
        ct = gi.make_cotangents(xt, 69, device=dev)
        Nt, Bt = xt.total_tokens, xt.num_seqs
        tpool = cpr.StatePool(P, Bt, device=dev)
        tcs = torch.empty((cpr.gdn_chunk_rows_bound(Nt, Bt, P.chunk), P.h_v, P.dv, P.dk), dtype=torch.float32,
                          device=dev)
        to = torch.empty((Nt, P.h_v, P.dv), dtype=torch.bfloat16, device=dev)
        tcu = torch.from_numpy(xt.cu_seqlens).to(dev)
        tids = torch.arange(Bt, dtype=torch.int32, device=dev)
        ws = torch.empty(cpr.gdn_backward_workspace_bytes(P, Nt, Bt), dtype=torch.uint8, device=dev)
        grads = {"dq": torch.empty((Nt, P.h_k, P.dk), device=dev), "dk": torch.empty((Nt, P.h_k, P.dk), device=dev),
                 "dv": torch.empty((Nt, P.h_v, P.dv), device=dev), "da": torch.empty((Nt, P.h_v), device=dev),
                 "db": torch.empty((Nt, P.h_v), device=dev)}

        tcw = torch.empty((2, Nt, P.h_v, P.dv), dtype=torch.float32, device=dev)

        def train_step(fe=None, be=None):
            cpr.gdn_trainer_forward(tpool, tcu, xt.q, xt.k, xt.v, xt.a, xt.b, slot_ids=tids, o=to,
                                    chunk_states=tcs, cw=tcw, events=fe)
            cpr.gdn_backward(P, tcu, xt.q, xt.k, xt.v, xt.a, xt.b, tcs, ct["d_o"], d_state=ct["d_state"],
                             workspace=ws, out=grads, events=be, cw=tcw)

        for _ in range(args.warmup):
            train_step()
        tev = [([hip.event() for _ in range(3)], [hip.event() for _ in range(4)]) for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            train_step(*tev[i])
        torch.cuda.synchronize()
        t_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        avg = lambda pairs: statistics.mean(hip.ms(a, b) for a, b in pairs)
        fwd_ms = avg([(f[0], f[2]) for f, _ in tev])
        adj_ms = avg([(b[0], b[1]) for _, b in tev])
        rep_ms = avg([(b[1], b[2]) for _, b in tev])
        grad_ms = avg([(b[2], b[3]) for _, b in tev])
        fa, _, fg = backward_flops([int(l) for l in xt.lengths], P.h_v, P.dk, P.dv, P.chunk)
        # the per-token gradient kernel reads dc, w (fp32) and v (bf16) and writes dv (fp32)
        tok_bytes = Nt * P.h_v * P.dv * (4 + 4 + 2 + 4)
        trainer = {
            "workload": f"trainer forward+backward, {Nt} tokens packed varlen {xt.lengths.tolist()} (H_k=16, "
                        "H_v=32, dk=dv=128, chunk=64, bf16 io); the forward keeps its chunk states and every "
                        "token's c and w for the backward",
            "ms_per_step": round(t_ms, 4), "forward_ms": round(fwd_ms, 4),
            "backward_ms": round(adj_ms + rep_ms + grad_ms, 4),
            "kernels": {"adjoint": {"avg_ms": round(adj_ms, 4), "tflops": round(fa / (adj_ms * 1e-3) / 1e12, 3),
                                    "bound": "alu", "peak_unpacked": FP32_UNPACKED_PEAK_TFLOPS},
                        "token_grads": {"avg_ms": round(rep_ms, 4), "bound": "hbm",
                                        "bytes": int(tok_bytes), "gbs": round(tok_bytes / (rep_ms * 1e-3) / 1e9, 1),
                                        "note": "dv = b dc, db = dc . w and v . dv per token-head (the replay "
                                                "would run here too, but the trainer forward kept every token's "
                                                "c and w)"},
                        "grad_chunk": {"avg_ms": round(grad_ms, 4), "tflops": round(fg / (grad_ms * 1e-3) / 1e12, 3),
                                       "bound": "mfma", "peak": FP32_MFMA_PEAK_TFLOPS,
                                       "frac": round(fg / (grad_ms * 1e-3) / 1e12 / FP32_MFMA_PEAK_TFLOPS, 4)}},
            "workspace_bytes": int(ws.numel()),
            "h100_fwd_bwd_ms": 7.386,
        }

        # the native trainer: chunkwise forward on matrix cores and the chunk form of its backward
        npool = cpr.StatePool(P, Bt, device=dev)
        ncs = torch.empty_like(tcs)
        no = torch.empty_like(to)
        nstash = torch.empty(cpr.gdn_trainer_forward_chunked_stash_bytes(P, Nt, Bt), dtype=torch.uint8, device=dev)
        nws = torch.empty(cpr.gdn_backward_chunked_workspace_bytes(P, Nt, Bt), dtype=torch.uint8, device=dev)
        ngrads = {k: torch.empty_like(v) for k, v in grads.items()}

        def native_step(fe=None, be=None):
            cpr.gdn_trainer_forward_chunked(npool, tcu, xt.q, xt.k, xt.v, xt.a, xt.b, slot_ids=tids, o=no,
                                            chunk_states=ncs, stash=nstash, events=fe)
            cpr.gdn_backward_chunked(P, tcu, xt.q, xt.k, xt.v, xt.a, xt.b, ncs, nstash, ct["d_o"],
                                     d_state=ct["d_state"], workspace=nws, out=ngrads, events=be)

        for _ in range(args.warmup):
            native_step()
        nev = [([hip.event() for _ in range(4)], [hip.event() for _ in range(4)]) for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            native_step(*nev[i])
        torch.cuda.synchronize()
        n_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        nf_ms = avg([(f[0], f[3]) for f, _ in nev])
        nb = [avg([(b[j], b[j + 1]) for _, b in nev]) for j in range(3)]
        trainer["native_chunked"] = {
            "ms_per_step": round(n_ms, 4), "forward_ms": round(nf_ms, 4), "backward_ms": round(sum(nb), 4),
            "backward_stages_ms": {"chunk_form_adjoint": round(nb[0], 4), "token_grads": round(nb[1], 4),
                                   "grad_chunk": round(nb[2], 4)},
            "normwise_vs_cpr": {k: round(float(normwise_t(ngrads[k], grads[k])), 8) for k in grads},
            "cpr_over_native": round(t_ms / n_ms, 3),
            "h100_fwd_bwd_ms": 5.177,
            "note": "gdn_trainer_forward_chunked (prep, state, output on bf16 matrix cores, keeping T^T, W^T and "
                    "c) and gdn_backward_chunked (w and the intra-chunk part of dC, the chunk chain of the "
                    "adjoint last chunk first, then the same per-token and chunk-gradient kernels as CPR)",
        }
        del npool, ncs, no, nstash, nws, ngrads
        del tpool, tcs, tcw, to, ws, grads, xt, ct

    # ---------------------------------------------------------------- CPU baseline (oracle)
    cpu = None
    parity_ok = True
    if pool is not None:
        xh = x.to("cpu")
        u16 = lambda t: t.contiguous().view(torch.int16).numpy().view(np.uint16)
        w64 = lambda z: (z.astype(np.uint32) << 16).view(np.float32).astype(np.float64) if z.dtype == np.uint16 \
            else z.astype(np.float64)
        qh, kh, vh = u16(xh.q), u16(xh.k), u16(xh.v)
        ah, bh = xh.a.numpy(), xh.b.numpy()
        grp = P.h_v // P.h_k
        kv = np.arange(P.h_v) // grp                                    # key head of each value head
        items = []
        for i in range(B):
            s0, s1 = int(x.cu_seqlens[i]), int(x.cu_seqlens[i + 1])
            for h in range(P.h_v):
                items.append((qh[s0:s1, kv[h]], kh[s0:s1, kv[h]], vh[s0:s1, h], ah[s0:s1, h], bh[s0:s1, h]))
        t0 = time.perf_counter()
        res = pool.map(_oracle_item, items, chunksize=1)
        cpu_wall = time.perf_counter() - t0
        groups = []
        for i in range(B):
            s0, s1 = int(x.cu_seqlens[i]), int(x.cu_seqlens[i + 1])
            ins = (w64(qh[s0:s1][:, kv]), w64(kh[s0:s1][:, kv]), w64(vh[s0:s1]), ah[s0:s1].astype(np.float64),
                   bh[s0:s1].astype(np.float64))
            groups.append((res[i * P.h_v:(i + 1) * P.h_v], o_bits[s0:s1], S_host[i].transpose(0, 2, 1).astype(np.float64),
                           ins, None))
        par = _parity(groups)
        parity_ok = parity_ok and par["ok"]
        cpu = {"value": round(N / cpu_wall, 1), "unit": "tok/s", "cores": args.cpu_workers, "kind": "oracle",
               "sample": f"the whole prefill workload ({B}x{x.lengths[0]} tokens, {P.h_v} value heads): "
                         f"{len(items)} (sequence, head) recurrences over a {args.cpu_workers}-process pool, "
                         f"{cpu_wall:.1f} s wall, {sum(r[2] for r in res):.1f} s of oracle time in the workers",
               "parity_vs_gpu": par,
               "cpu_model": host_env["cpu_model"], "numpy": host_env["numpy"]}
        del res, items, groups
        if dec_host is not None:
            # the decode workload's steps: every (slot, value head) continued by the oracle from the
            # state the prompts left in the slot, over the slot's tokens
            d = dec_host
            nb = d["S0"].shape[0]
            steps = d["q"].shape[1]
            items = []
            for i in range(nb):
                for h in range(P.h_v):
                    items.append((d["q"][i, :, kv[h]], d["k"][i, :, kv[h]], d["v"][i, :, h], d["a"][i, :, h],
                                  d["b"][i, :, h], d["S0"][i, h].T.astype(np.float64), d["lens"][i]))
            t0 = time.perf_counter()
            res = pool.map(_oracle_item, items, chunksize=16)
            dec_wall = time.perf_counter() - t0
            groups = []
            for i in range(nb):
                ins = (w64(d["q"][i][:, kv]), w64(d["k"][i][:, kv]), w64(d["v"][i]), d["a"][i].astype(np.float64),
                       d["b"][i].astype(np.float64))
                groups.append((res[i * P.h_v:(i + 1) * P.h_v], d["o"][i], d["final"][i].transpose(0, 2, 1).astype(np.float64),
                               ins, d["S0"][i].transpose(0, 2, 1).astype(np.float64)))
            dpar = _parity(groups)
            parity_ok = parity_ok and dpar["ok"]
            cpu["decode"] = {"value": round(dec_wall * 1e6 / steps, 1), "unit": "us/step", "kind": "oracle",
                             "sample": f"the whole decode workload: {nb} slots x {P.h_v} value heads x {steps} "
                                       f"steps from the prompts' states, {len(items)} recurrences over the "
                                       f"{args.cpu_workers}-process pool, {dec_wall:.1f} s wall",
                             "parity_vs_gpu": dpar}
            del res, items, groups
        pool.close()
        pool.join()

    # The pages' per-layer table (native mixed / recurrent everywhere / CPR), measured here.
    def _pick(d, *keys):
        for key in keys:
            d = d.get(key) if isinstance(d, dict) else None
        return d

    def _row(native, recurrent, cpr_, unit):
        row = {"unit": unit, "native": native, "recurrent_everywhere": recurrent, "cpr": cpr_}
        for name, val in (("recurrent_over_native", recurrent), ("cpr_over_native", cpr_)):
            row[name] = round(val / native, 3) if native and val else None
        return row

    table = {
        "rollout_prefill_5x2048": _row(_pick(chunked, "native", "ms_per_step"), _pick(fused, "ms_per_step"),
                                       round(ms_step, 4), "ms"),
        "rollout_decode_256x1": _row(_pick(decode, "us_per_step_median"), _pick(decode, "us_per_step_median"),
                                     _pick(decode, "with_boundary_record", "us_per_step_median"), "us"),
        "trainer_fwd_bwd_10240": _row(_pick(trainer, "native_chunked", "ms_per_step"), None,
                                      _pick(trainer, "ms_per_step"), "ms"),
        "note": "native = the chunk form on matrix cores (prefill, trainer) and the plain recurrent step "
                "(decode); recurrent everywhere = the one-pass recurrent prefill (the same bits as CPR here) "
                "and the same decode step; CPR decode = the step committing every chunk start to the "
                "boundary record (reading R1; decode.r2_reading is R2's). No separate recurrent-everywhere "
                "trainer is built: CPR's backward already runs the adjoint token by token.",
    }

    out = {
        "metric": METRIC, "value": round(N / (ms_step * 1e-3), 1), "unit": "tok/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "prefill 5x2048: H_k=16, H_v=32, dk=dv=128, chunk=64, "
                               "bf16 q/k/v/o, fp32 a/b/state",
                   "global_batch": B, "seq_len": int(x.lengths[0]), "parallelism": "single-gpu"},
        "prefill": {"boundary_pass_ms": round(p1_ms, 4), "output_pass_ms": round(p2_ms, 4),
                    "algorithmic_bytes": int(alg_bytes), "hbm_frac": round(prefill_gbs / HBM_PEAK_GBS, 4),
                    "hbm_frac_note": "algorithmic bytes of CPR (I/O, pass 1's second read of k, v, a, b, each "
                                     "chunk-start state written and read once) over the step time",
                    "c_stash_bytes": int(2 * c_bytes),
                    "bytes_moved_with_stash": int(pass1_bytes + pass2_bytes),
                    "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                                for k, v in kernels.items()},
                    "sha256": identity,
                    "without_c_stash": no_stash, "one_pass_variant": fused, "chunked_matrix_core": chunked,
                    "long_sequence": long_seq},
        "roofline": roofline,
        "decode": decode,
        "trainer": trainer,
        "cpu_baseline": cpu,
        "environment": {"gpu": torch.cuda.get_device_name(0),
                        "compute_units": torch.cuda.get_device_properties(0).multi_processor_count,
                        "hip": torch.version.hip, "torch": torch.__version__, **host_env},
        "context": {"table_mi355x": table,
                    "h100_per_layer_ms": {"prefill_5x2048_cpr": 1.412, "prefill_5x2048_native": 0.844,
                                          "decode_256x1_cpr": 0.0846, "decode_256x1_native": 0.0612,
                                          "decode_256x1_recurrent": 0.0612, "prefill_5x2048_recurrent": 3.639,
                                          "trainer_fwd_bwd_10240_recurrent": 22.863,
                                          "trainer_fwd_bwd_10240_cpr": 7.386, "trainer_fwd_bwd_10240_native": 5.177},
                    "note": "pages' H100 figures; head layout not stated there"},
    }
    print(json.dumps(out, default=lambda v: v.item() if hasattr(v, "item") else str(v)), flush=True)
    if not parity_ok:
        print("bench: the GPU outputs breach the oracle tolerance (cpu_baseline.parity_vs_gpu)", file=sys.stderr)
        sys.exit(3)


if __name__ == "__main__":
    main()
