"""The benchmark's work and byte accounting (host logic, no GPU): the algorithmic bytes and FLOPs it
divides by measured times, checked against counts worked out independently from the layouts, and
its refusal of more than one GPU."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_decode_bytes_per_step():
    # 256 slots x 32 value heads x 128 x 128 fp32 state, read and written once: 1,073,741,824 B;
    # per slot q, k (16 key heads x 128 bf16 each), v and o (32 x 128 bf16 each), a and b (32 fp32)
    state = 2 * 256 * 32 * 128 * 128 * 4
    tokens = 256 * (2 * 16 * 128 * 2 + 2 * 32 * 128 * 2 + 2 * 32 * 4)
    assert state + tokens == 1_080_098_816
    assert bench.decode_bytes(256, 16, 32, 128, 128) == 1_080_098_816


def test_prefill_bytes_5x2048():
    alg, c, p1, p2 = bench.prefill_bytes([2048] * 5, 16, 32, 128, 128, 64)
    plane = 32 * 128 * 128 * 4                           # one state of all value heads, 2 MiB
    n = 10240
    qkvabo = n * (2 * 16 * 128 * 2 + 2 * 32 * 128 * 2 + 2 * 32 * 4)   # q, k, v, o (bf16), a, b (fp32)
    reread = 5 * 1984 * (16 * 128 * 2 + 32 * 128 * 2 + 2 * 32 * 4)   # k, v, a, b before each last chunk start
    rows = 5 * 32                                        # chunk starts 0, 64, ..., 1984 of each sequence
    assert alg == qkvabo + 5 * plane + reread + 2 * (rows - 5) * plane == 1_039_319_040
    assert c == n * 32 * 128 * 4 == 167_772_160
    assert p1 == 631_767_040 and p2 == 682_885_120


def test_prefill_bytes_ragged_and_empty():
    alg, c, p1, p2 = bench.prefill_bytes([0, 1, 64, 65], 1, 1, 16, 16, 64, io=4)
    plane = 16 * 16 * 4
    tok_kvab = 16 * 4 + 16 * 4 + 8
    io_bytes = 130 * (2 * 16 * 4 + 2 * 16 * 4 + 8) + 4 * plane
    # rows: 0, 1, 1, 2; pass 1 rereads only the 64 tokens of the last sequence before its second chunk
    assert alg == io_bytes + 64 * tok_kvab + 2 * (4 - 4) * plane
    assert p1 == 130 * tok_kvab + 4 * plane + c


def test_flop_counts():
    f1, f2, p1_tokens = bench.prefill_flops([2048] * 5, 32, 128, 128, 64)
    assert f1 == f2 == 10240 * 32 * 5 * 128 * 128 and p1_tokens == 10240
    g1, g2, _ = bench.prefill_flops([2048] * 5, 32, 128, 128, 64, stash=False)
    assert g1 == 5 * 1984 * 32 * 5 * 128 * 128 and g2 == 10240 * 32 * 7 * 128 * 128
    adj, rep, mfma = bench.backward_flops([64, 65], 2, 16, 16, 64)
    assert adj == 129 * 2 * 7 * 256 and rep == 129 * 2 * 5 * 256
    per_chunk = lambda L: 6 * L * 16 * 16 + 10 * L * L * 16
    assert mfma == 2 * (per_chunk(64) * 2 + per_chunk(1))


def test_bench_runs_on_one_gpu_only():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
