"""The C ABI without a GPU: the library loads, exports every declared symbol, and its host-only
logic (SHA-256, policy digest and check, validation, chunk-row planning, argument errors that are
raised before any launch) is correct."""
import ctypes
import hashlib
import os
import re
import struct
import subprocess

import numpy as np
import pytest

from oracle import num_boundary_rows

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cpr_gdn.h")


def _lib_module():
    """Load the binding, building the library first only if nothing is built."""
    lib = os.path.join(ROOT, "bitwise_aligned_gated_amd", "libcpr_gdn.so")
    if not os.path.exists(lib):
        import runpy
        runpy.run_path(os.path.join(ROOT, "bitwise_aligned_gated_amd", "build.py"))["build_library"]()
    import bitwise_aligned_gated_amd as cpr
    return cpr


cpr = _lib_module()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 15
    out = subprocess.run(["nm", "-D", "--defined-only", cpr.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (gdn_\w+)", out))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    lib = ctypes.CDLL(cpr.LIB_PATH)
    for n in names:
        assert getattr(lib, n) is not None
    assert set(cpr.EXPORTS) == set(names)


@pytest.mark.parametrize("n", [0, 1, 3, 55, 56, 57, 63, 64, 65, 119, 120, 1000, 4097])
def test_sha256_matches_hashlib(n):
    data = np.random.default_rng(n).integers(0, 256, n, dtype=np.uint8).tobytes()
    assert cpr.gdn_sha256(data) == hashlib.sha256(data).digest()


def test_policy_digest_is_sha256_of_canonical_bytes():
    p = cpr.Policy(16, 32, 128, 128, chunk=64, io="bf16")
    canon = b"cpr-gdn-policy-v1" + struct.pack("<10i", 16, 32, 128, 128, 1, 0, 1, 0, 8, 0)
    assert cpr.gdn_policy_digest(p) == hashlib.sha256(canon).digest()
    # with bf16 boundaries the chunk size moves bits and enters the digest
    pb = cpr.Policy(16, 32, 128, 128, chunk=64, io="bf16", boundary="bf16")
    canon_b = b"cpr-gdn-policy-v1" + struct.pack("<10i", 16, 32, 128, 128, 1, 1, 1, 64, 8, 0)
    assert cpr.gdn_policy_digest(pb) == hashlib.sha256(canon_b).digest()
    assert cpr.gdn_policy_digest(pb) != cpr.gdn_policy_digest(cpr.Policy(16, 32, 128, 128, chunk=32, boundary="bf16"))
    # chunk is a deployment setting and does not enter the digest; dtypes and shapes do
    assert cpr.gdn_policy_digest(cpr.Policy(16, 32, 128, 128, chunk=16)) == cpr.gdn_policy_digest(p)
    assert cpr.gdn_policy_digest(cpr.Policy(16, 32, 128, 128, io="f32")) != cpr.gdn_policy_digest(p)
    assert cpr.gdn_policy_digest(cpr.Policy(8, 32, 128, 128)) != cpr.gdn_policy_digest(p)


def test_semantic_and_deployment_digests():
    p = cpr.Policy(16, 32, 128, 128, chunk=64, io="bf16")
    sem = b"cpr-gdn-semantic-v1" + struct.pack("<6i", 1, 16, 32, 128, 128, 0)
    assert cpr.gdn_semantic_digest(p) == hashlib.sha256(sem).digest()
    # the semantic digest ignores everything that only affects rounding or deployment
    for other in (cpr.Policy(16, 32, 128, 128, chunk=16, io="f32"), cpr.Policy(16, 32, 128, 128, boundary="bf16")):
        assert cpr.gdn_semantic_digest(other) == cpr.gdn_semantic_digest(p)
    assert cpr.gdn_semantic_digest(cpr.Policy(16, 32, 64, 64)) != cpr.gdn_semantic_digest(p)
    dep = cpr.gdn_deployment_digest(p)
    # canonical bytes: the tag, chunk (fp32 boundaries) and the kernels' work-mapping version (6)
    assert dep == hashlib.sha256(b"cpr-gdn-deploy-v1" + struct.pack("<2i", 64, 6)).digest()
    assert cpr.gdn_deployment_digest(cpr.Policy(16, 32, 128, 128, chunk=64, boundary="bf16")) == \
        hashlib.sha256(b"cpr-gdn-deploy-v1" + struct.pack("<2i", 0, 6)).digest()
    # fp32 boundaries: chunk is a deployment setting (deployment digest moves, policy digest not)
    p16 = cpr.Policy(16, 32, 128, 128, chunk=16)
    assert cpr.gdn_deployment_digest(p16) != dep and cpr.gdn_policy_digest(p16) == cpr.gdn_policy_digest(p)
    # bf16 boundaries: chunk is numerical (policy digest moves, deployment digest not)
    b64, b16 = cpr.Policy(16, 32, 128, 128, chunk=64, boundary="bf16"), cpr.Policy(16, 32, 128, 128, chunk=16, boundary="bf16")
    assert cpr.gdn_deployment_digest(b64) == cpr.gdn_deployment_digest(b16)
    assert cpr.gdn_policy_digest(b64) != cpr.gdn_policy_digest(b16)


def test_policy_check_refuses_mismatch():
    d1 = cpr.gdn_policy_digest(cpr.Policy(16, 32, 128, 128))
    d2 = cpr.gdn_policy_digest(cpr.Policy(16, 32, 128, 128, io="f32"))
    cpr.gdn_policy_check(d1, d1)
    with pytest.raises(cpr.GdnError) as e:
        cpr.gdn_policy_check(d1, d2)
    assert e.value.code == 4


@pytest.mark.parametrize("args,code", [
    ((16, 32, 96, 96), 2), ((16, 32, 128, 64), 2), ((16, 30, 128, 128), 1), ((0, 32, 128, 128), 1),
    ((16, 32, 128, 128, 0), 1), ((16, 32, 128, 128, 64, "bf16", 2), 2),
])
def test_policy_validation(args, code):
    with pytest.raises(cpr.GdnError) as e:
        cpr.Policy(*args).validate()
    assert e.value.code == code


@pytest.mark.parametrize("dims", [16, 32, 64, 128])
def test_supported_policies(dims):
    cpr.Policy(2, 4, dims, dims, io="f32").validate()
    cpr.Policy(2, 4, dims, dims, io="bf16").validate()


def test_check_cu_seqlens():
    cpr.gdn_check_cu_seqlens([0, 3, 3, 10], 10)
    for bad, n in (([1, 3], 3), ([0, 5, 4], 4), ([0, 5], 6)):
        with pytest.raises(cpr.GdnError):
            cpr.gdn_check_cu_seqlens(bad, n)


def test_chunk_rows_match_oracle_and_bound():
    rng = np.random.default_rng(0)
    for chunk in (1, 7, 16, 64):
        for _ in range(20):
            B = int(rng.integers(1, 12))
            lens = rng.integers(0, 300, B)
            pos0 = rng.integers(0, 500, B)
            cu = np.concatenate([[0], np.cumsum(lens)])
            off = cpr.gdn_chunk_rows(cu, chunk, pos0).numpy()
            expect = np.concatenate([[0], np.cumsum([num_boundary_rows(int(p), int(L), chunk)
                                                     for p, L in zip(pos0, lens)])])
            assert np.array_equal(off, expect)
            assert off[-1] <= cpr.gdn_chunk_rows_bound(int(cu[-1]), B, chunk)


def test_chunk_rows_bound_errors():
    with pytest.raises(cpr.GdnError):
        cpr.gdn_chunk_rows_bound(10, 1, 0)


def test_prefill_argument_errors_before_launch():
    """Errors the host detects return GDN_EINVAL before any kernel is launched (no GPU needed).
    The state handle binds fake device addresses that are never dereferenced."""
    lib = cpr._lib
    pol = cpr.Policy(2, 4, 16, 16, io="f32").c()
    h = ctypes.c_void_p()
    nbytes = lib.gdn_state_bytes(ctypes.byref(pol), 3)
    assert nbytes == 3 * 4 * 16 * 16 * 4
    fake = 0x10000
    assert lib.gdn_state_alloc(ctypes.byref(pol), 3, fake, fake, nbytes, None, None, ctypes.byref(h)) == 0
    try:
        # wrong state size
        h2 = ctypes.c_void_p()
        assert lib.gdn_state_alloc(ctypes.byref(pol), 3, fake, fake, nbytes + 4, None, None, ctypes.byref(h2)) == 1
        assert h2.value is None
        # boundary without boundary_pos
        assert lib.gdn_state_alloc(ctypes.byref(pol), 3, fake, fake, nbytes, fake, None, ctypes.byref(h2)) == 1
        # too few chunk-state rows: bound(100 tokens, 2 seqs, C=64) = 1 + 4 = 5
        rc = lib.gdn_prefill(h, fake, 2, 100, fake, 0, fake, fake, fake, fake, fake, fake, fake, 4, None, None, None)
        assert rc == 1 and b"chunk_state_rows" in lib.gdn_last_error()
        rc = lib.gdn_prefill(h, fake, -1, 100, fake, 0, fake, fake, fake, fake, fake, fake, fake, 99, None, None, None)
        assert rc == 1
        rc = lib.gdn_prefill(h, fake, 2, 100, fake, 2, fake, fake, fake, fake, fake, fake, fake, 99, None, None, None)
        assert rc == 1
        rc = lib.gdn_prefill(h, fake, 2, 100, fake, 0, None, fake, fake, fake, fake, fake, fake, 99, None, None, None)
        assert rc == 1
        rc = lib.gdn_prefill(None, fake, 2, 100, fake, 0, fake, fake, fake, fake, fake, fake, fake, 99, None, None, None)
        assert rc == 1
        # a c stash that is not 16-byte aligned
        rc = lib.gdn_prefill(h, fake, 2, 100, fake, 0, fake, fake, fake, fake, fake, fake, fake, 99, fake + 4, None, None)
        assert rc == 1 and b"c stash" in lib.gdn_last_error()
        # the single-launch prefills share the prefill checks
        for fn in (lib.gdn_prefill_fused, lib.gdn_prefill_overlapped):
            rc = fn(None, fake, 2, 100, fake, 0, fake, fake, fake, fake, fake, fake, fake, 99, None, None)
            assert rc == 1 and b"state handle" in lib.gdn_last_error()
            rc = fn(h, fake, 2, 100, fake, 0, fake, fake, fake, fake, fake, fake, fake, 4, None, None)
            assert rc == 1 and b"chunk_state_rows" in lib.gdn_last_error()
            rc = fn(h, fake, 2, 100, fake, 3, fake, fake, fake, fake, fake, fake, fake, 99, None, None)
            assert rc == 1 and b"from_state" in lib.gdn_last_error()
        rc = lib.gdn_decode_step(h, fake, -1, fake, fake, fake, fake, fake, fake, None, None)
        assert rc == 1
        rc = lib.gdn_decode_step(h, None, 3, fake, fake, fake, fake, fake, fake, None, None)
        assert rc == 1
        rc = lib.gdn_state_resync(h, None, 2, None)
        assert rc == 1
        # empty work launches nothing and succeeds
        assert lib.gdn_decode_step(h, None, 0, None, None, None, None, None, None, None, None) == 0
        assert lib.gdn_state_resync(h, None, 0, None) == 0
        assert lib.gdn_last_error() == b""
        # launch-shape cap: 0 and positive values below 2^31 are accepted
        for n in (0, 1, 7, 0x7FFFFFFF):
            assert lib.gdn_state_set_max_workgroups(h, n) == 0
        for n in (-1, 1 << 31):
            assert lib.gdn_state_set_max_workgroups(h, n) == 1 and b"max_workgroups" in lib.gdn_last_error()
        assert lib.gdn_state_set_max_workgroups(None, 4) == 1 and b"state handle" in lib.gdn_last_error()
        # the prefill with static scratch refuses, before touching the GPU, a batch whose chunk-start
        # rows exceed its buffer: 5,000,000 tokens at chunk 64 need 78,127 rows of 4 KiB (305 MiB)
        rc = lib.gdn_prefill_static(h, fake, 2, 5_000_000, fake, 0, fake, fake, fake, fake, fake, fake, None, None)
        assert rc == 1 and b"static" in lib.gdn_last_error()
        assert lib.gdn_prefill_static(None, fake, 2, 100, fake, 0, fake, fake, fake, fake, fake, fake, None, None) == 1
        assert cpr.GDN_STATIC_SCRATCH_BYTES == 256 << 20
        # R2 resynchronisation: this pool has fp32 io and no boundary record
        assert lib.gdn_state_attach_r2(h, fake, 1 << 30, fake, 1 << 30) == 2
        assert lib.gdn_r2_ring_bytes(ctypes.byref(pol), 3) == -1
        # the overlapped kernel's wait bound: any value is accepted, a NULL handle is not
        for n in (0, 1, 0xFFFFFFFF):
            assert lib.gdn_state_set_wait_limit(h, n) == 0
        assert lib.gdn_state_set_wait_limit(None, 1) == 1 and b"state handle" in lib.gdn_last_error()
    finally:
        assert lib.gdn_state_free(h) == 0
    assert lib.gdn_state_free(None) == 0


def test_backward_workspace_bytes():
    # dL/dS at every chunk boundary: (N/C + B) chunk rows plus one more boundary per sequence,
    # each H_v * dk * dv * 4 bytes; then three per-token arrays (dc, c, w) of N * H_v * dv * 4
    # bytes; each part padded to 256 bytes
    pad = lambda x: -(-x // 256) * 256
    # then the parts of <dL/dS, S> at every boundary: 32 fp64 per value head at d = 128, 1 at d = 16
    p = cpr.Policy(16, 32, 128, 128, chunk=64)
    adj = (10240 // 64 + 4 + 4) * 32 * 128 * 128 * 4
    tok = 10240 * 32 * 128 * 4
    parts = (10240 // 64 + 4 + 4) * 32 * 32 * 8
    xv = 10240 * 32 * 4                                                  # v_t . dv_t per token-head
    assert cpr.gdn_backward_workspace_bytes(p, 10240, 4) == pad(adj) + 3 * pad(tok) + pad(parts) + pad(xv)
    # bf16 boundaries below 64 tokens: the gradient passes run at the forward's chunk
    p = cpr.Policy(1, 2, 16, 16, chunk=8, io="f32", boundary="bf16")
    adj, tok = (100 // 8 + 3 + 3) * 2 * 16 * 16 * 4, 100 * 2 * 16 * 4
    assert cpr.gdn_backward_workspace_bytes(p, 100, 3) == pad(adj) + 3 * pad(tok) + pad((100 // 8 + 3 + 3) * 2 * 8) + \
        pad(100 * 2 * 4)
    # fp32 boundaries at any chunk but 64 are differentiated on a rebuilt 64-token stash: the
    # gradient parts are those of chunk 64, then the 64-token stash ((N/64 + B) states), an int32
    # slot id per sequence and an int64 position per row of the forward's (N/C + B)-row stash
    for C in (8, 20, 200):
        p = cpr.Policy(2, 4, 32, 32, chunk=C, io="f32")
        plane = 4 * 32 * 32 * 4
        adj, tok = (1000 // 64 + 5 + 5) * plane, 1000 * 4 * 32 * 4
        parts = (1000 // 64 + 5 + 5) * 4 * 2 * 8                        # 2 parts per value head at d = 32
        extra = pad((1000 // 64 + 5) * plane) + pad(5 * 4) + pad((1000 // C + 5) * 8)
        assert cpr.gdn_backward_workspace_bytes(p, 1000, 5) == pad(adj) + 3 * pad(tok) + pad(parts) + \
            pad(1000 * 4 * 4) + extra, C
    with pytest.raises(cpr.GdnError):
        cpr.gdn_backward_workspace_bytes(p, -1, 3)


def test_backward_argument_errors_before_launch():
    """gdn_backward's host checks (no GPU needed; the fake addresses are never dereferenced)."""
    lib = cpr._lib
    fake = 0x10000

    def call(pol, rows=99, ws_bytes=1 << 40, num_seqs=2, total=100, ws=fake, d_o=fake):
        return lib.gdn_backward(ctypes.byref(pol.c()), fake, num_seqs, total, fake, fake, fake, fake, fake, fake,
                                rows, None, d_o, None, fake, fake, fake, fake, fake, None, ws, ws_bytes, None, None)

    f32 = cpr.Policy(2, 4, 16, 16, chunk=64, io="f32")
    # the bf16 boundary dtype has a backward (straight-through) and meets the same checks
    assert call(cpr.Policy(2, 4, 16, 16, chunk=64, io="f32", boundary="bf16"), rows=2) == 1
    assert b"chunk_state_rows" in lib.gdn_last_error()
    # chunks above 64 tokens: fp32 boundaries meet the usual checks (rows >= 100/128 + 2 = 2),
    # bf16 boundaries are unsupported there
    assert call(cpr.Policy(2, 4, 16, 16, chunk=128, io="f32"), rows=1) == 1
    assert b"chunk_state_rows" in lib.gdn_last_error()
    assert call(cpr.Policy(2, 4, 16, 16, chunk=128, io="f32"), ws_bytes=16) == 1
    assert call(cpr.Policy(2, 4, 16, 16, chunk=128, io="f32", boundary="bf16")) == 2
    assert call(cpr.Policy(2, 3, 16, 16, chunk=64, io="f32")) == 1            # H_v not a multiple of H_k
    assert call(f32, rows=2) == 1 and b"chunk_state_rows" in lib.gdn_last_error()   # needs 100/64 + 2 = 3
    assert call(f32, ws_bytes=16) == 1 and b"workspace" in lib.gdn_last_error()
    assert call(f32, ws=fake + 4) == 1 and b"aligned" in lib.gdn_last_error()
    assert call(f32, d_o=None) == 1
    assert call(f32, num_seqs=-1) == 1
    # empty work launches nothing and succeeds
    assert lib.gdn_backward(ctypes.byref(f32.c()), None, 0, 0, None, None, None, None, None, None, 0, None, None,
                            None, None, None, None, None, None, None, None, 0, None, None) == 0


def test_chunked_workspace_and_argument_errors():
    """gdn_prefill_chunked's host checks (no GPU needed; fake addresses are never dereferenced)."""
    lib = cpr._lib
    p = cpr.Policy(2, 4, 128, 128, chunk=64, io="bf16")
    # per (chunk row, value head): W, U and C^T (64 x d fp32 each) and 72 doubles of log products
    per = (3 * 64 * 128 + 144) * 4
    assert cpr.gdn_prefill_chunked_workspace_bytes(p, 1000, 3) == cpr.gdn_chunk_rows_bound(1000, 3, 64) * 4 * per
    assert lib.gdn_prefill_chunked_workspace_bytes(ctypes.byref(cpr.Policy(2, 4, 16, 16, io="bf16").c()), 10, 1) == -1
    fake = 0x10000
    msgs = []

    def call(pol, outputs=0, ws_bytes=1 << 40, ws=fake, rows=99):
        h = ctypes.c_void_p()
        nbytes = lib.gdn_state_bytes(ctypes.byref(pol.c()), 3)
        assert lib.gdn_state_alloc(ctypes.byref(pol.c()), 3, fake, fake, nbytes, None, None, ctypes.byref(h)) == 0
        try:
            rc = lib.gdn_prefill_chunked(h, fake, 2, 100, fake, 0, fake, fake, fake, fake, fake, fake, fake, rows,
                                         outputs, ws, ws_bytes, None, None)
            msgs.append(lib.gdn_last_error())
            return rc
        finally:
            lib.gdn_state_free(h)

    assert call(cpr.Policy(2, 4, 64, 64, io="f32")) == 2                     # bf16 io only
    assert call(cpr.Policy(2, 4, 64, 64, io="bf16", boundary="bf16")) == 2   # fp32 boundaries only
    assert call(cpr.Policy(2, 4, 64, 64, chunk=128, io="bf16")) == 2
    assert call(cpr.Policy(2, 4, 64, 64, io="bf16"), outputs=2) == 1
    assert call(cpr.Policy(2, 4, 64, 64, io="bf16"), ws_bytes=64) == 1 and b"workspace" in msgs[-1]
    assert call(cpr.Policy(2, 4, 64, 64, io="bf16"), ws=fake + 8) == 1
    assert call(cpr.Policy(2, 4, 64, 64, io="bf16"), rows=2) == 1


def test_r2_sizes_and_attach_errors():
    """R2 ring and workspace sizes, attach checks, and the refusal of R1 calls on an R2 pool (no
    GPU: host checks only, fake addresses never dereferenced)."""
    lib = cpr._lib
    pad = lambda x: -(-x // 256) * 256
    p = cpr.Policy(16, 32, 128, 128, chunk=64, io="bf16")
    n = 256 * 64
    ring = 2 * pad(n * 16 * 128 * 2) + pad(n * 32 * 128 * 2) + 2 * pad(n * 32 * 4)
    assert lib.gdn_r2_ring_bytes(ctypes.byref(p.c()), 256) == ring
    # the one-chunk batch (cu_seqlens, slot ids, gates, positions), the list of gated slots, their
    # batch entries and the count, then the chunk form's workspace for one row per slot
    ws = pad(257 * 4) + 2 * pad(256 * 4) + pad(256 * 8) + 2 * pad(256 * 4) + pad(4) + 256 * 32 * (3 * 64 * 128 + 2 * 72) * 4
    assert lib.gdn_r2_workspace_bytes(ctypes.byref(p.c()), 256) == ws
    assert lib.gdn_r2_ring_bytes(ctypes.byref(cpr.Policy(16, 32, 128, 128, chunk=100).c()), 4) == -1
    assert lib.gdn_r2_ring_bytes(ctypes.byref(cpr.Policy(16, 32, 16, 16).c()), 4) == -1
    fake = 0x10000
    small = cpr.Policy(2, 4, 32, 32, chunk=16, io="bf16")
    nb = lib.gdn_state_bytes(ctypes.byref(small.c()), 3)
    rb, wb = lib.gdn_r2_ring_bytes(ctypes.byref(small.c()), 3), lib.gdn_r2_workspace_bytes(ctypes.byref(small.c()), 3)
    h = ctypes.c_void_p()
    assert lib.gdn_state_alloc(ctypes.byref(small.c()), 3, fake, fake, nb, None, None, ctypes.byref(h)) == 0
    try:
        assert lib.gdn_state_attach_r2(h, fake, rb, fake, wb) == 1 and b"boundary record" in lib.gdn_last_error()
    finally:
        lib.gdn_state_free(h)
    assert lib.gdn_state_alloc(ctypes.byref(small.c()), 3, fake, fake, nb, fake, fake, ctypes.byref(h)) == 0
    try:
        assert lib.gdn_state_attach_r2(h, fake, rb - 1, fake, wb) == 1
        assert lib.gdn_state_attach_r2(h, fake + 4, rb, fake, wb) == 1
        assert lib.gdn_state_attach_r2(h, fake, rb, None, wb) == 1
        assert lib.gdn_state_attach_r2(h, fake, rb, fake, wb) == 0
        # R1 calls would leave the ring behind: refused before any launch
        rc = lib.gdn_prefill(h, fake, 2, 100, fake, 0, fake, fake, fake, fake, fake, fake, fake, 99, None, None, None)
        assert rc == 1 and b"R2" in lib.gdn_last_error()
        rc = lib.gdn_prefill_fused(h, fake, 2, 100, fake, 0, fake, fake, fake, fake, fake, fake, None, 0, None, None)
        assert rc == 1 and b"R2" in lib.gdn_last_error()
        assert lib.gdn_state_resync(h, fake, 2, None) == 1
        rc = lib.gdn_prefill_chunked(h, fake, 2, 100, fake, 0, fake, fake, fake, fake, fake, fake, fake, 99, 0, fake,
                                     1 << 40, None, None)
        assert rc == 1 and b"R2" in lib.gdn_last_error()
        assert lib.gdn_state_attach_r2(h, None, 0, None, 0) == 0          # detached: R1 checks as usual
        rc = lib.gdn_prefill(h, fake, 2, 100, fake, 0, fake, fake, fake, fake, fake, fake, fake, 4, None, None, None)
        assert rc == 1 and b"chunk_state_rows" in lib.gdn_last_error()
    finally:
        lib.gdn_state_free(h)


def test_chunked_trainer_sizes_and_argument_errors():
    """The chunkwise trainer's stash and backward workspace sizes, and the host checks of
    gdn_trainer_forward_chunked and gdn_backward_chunked (no GPU: fake addresses are never
    dereferenced)."""
    lib = cpr._lib
    pad = lambda x: -(-x // 256) * 256
    N, B = 1000, 3
    for d, parts in ((32, 4), (64, 8), (128, 16)):
        p = cpr.Policy(2, 4, d, d, chunk=64, io="bf16")
        rows = cpr.gdn_chunk_rows_bound(N, B, 64)
        ws = cpr.gdn_prefill_chunked_workspace_bytes(p, N, B)
        # the forward's workspace, then T^T (64 x 64) and W^T (d x 64) per chunk row and value head,
        # then every token's c
        stash = pad(ws) + pad(rows * 4 * (64 * 64 + 64 * d) * 4 + N * 4 * d * 4)
        assert cpr.gdn_trainer_forward_chunked_stash_bytes(p, N, B) == stash
        # G at every boundary, dc and w, the <G, S> parts (4 per 32 columns), v . dv
        adj = (rows + B) * 4 * d * d * 4
        wsb = pad(adj) + 2 * pad(N * 4 * d * 4) + pad((rows + B) * 4 * parts * 8) + pad(N * 4 * 4)
        assert cpr.gdn_backward_chunked_workspace_bytes(p, N, B) == wsb
    bad = cpr.Policy(2, 4, 16, 16, io="bf16")                                  # head dim not built
    assert lib.gdn_trainer_forward_chunked_stash_bytes(ctypes.byref(bad.c()), 10, 1) == -1
    assert lib.gdn_backward_chunked_workspace_bytes(ctypes.byref(bad.c()), 10, 1) == -1
    fake = 0x10000
    p = cpr.Policy(2, 4, 64, 64, chunk=64, io="bf16")
    need = cpr.gdn_trainer_forward_chunked_stash_bytes(p, 100, 2)
    h = ctypes.c_void_p()
    nbytes = lib.gdn_state_bytes(ctypes.byref(p.c()), 3)
    assert lib.gdn_state_alloc(ctypes.byref(p.c()), 3, fake, fake, nbytes, None, None, ctypes.byref(h)) == 0
    try:
        rc = lib.gdn_trainer_forward_chunked(h, fake, 2, 100, fake, 0, fake, fake, fake, fake, fake, fake, fake, 99,
                                             fake, need - 1, None, None)
        assert rc == 1 and b"stash" in lib.gdn_last_error()
    finally:
        lib.gdn_state_free(h)
    wneed = cpr.gdn_backward_chunked_workspace_bytes(p, 100, 2)

    def bwd(pol, stash_bytes=need, ws_bytes=wneed, ws=fake, rows=99):
        return lib.gdn_backward_chunked(ctypes.byref(pol.c()), fake, 2, 100, fake, fake, fake, fake, fake, fake, rows,
                                        fake, stash_bytes, fake, None, fake, fake, fake, fake, fake, None, ws, ws_bytes,
                                        None, None)

    assert bwd(cpr.Policy(2, 4, 64, 64, io="f32")) == 2
    assert bwd(cpr.Policy(2, 4, 64, 64, io="bf16", boundary="bf16")) == 2
    assert bwd(cpr.Policy(2, 4, 64, 64, chunk=100, io="bf16")) == 2
    assert bwd(p, stash_bytes=need - 1) == 1 and b"stash" in lib.gdn_last_error()
    assert bwd(p, ws_bytes=wneed - 1) == 1 and b"workspace" in lib.gdn_last_error()
    assert bwd(p, ws=fake + 8) == 1
    assert bwd(p, rows=2) == 1
