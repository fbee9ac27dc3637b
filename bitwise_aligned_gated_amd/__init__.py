"""Python binding of libcpr_gdn: CPR Gated DeltaNet on MI355X (gfx950).

Argument marshalling only.  Every step of the computation runs in the library's HIP kernels;
PyTorch supplies device memory and the current HIP stream.  Importing this package loads the
built ``libcpr_gdn.so`` and raises ImportError when it is missing -- there is no fallback path.
The function names mirror the C entry points declared in ``include/cpr_gdn.h``.
"""
from __future__ import annotations

import ctypes
import functools
import os
from dataclasses import dataclass

import torch

__all__ = [
    "LIB_PATH", "GdnError", "Policy", "StatePool", "gdn_policy_digest", "gdn_policy_check",
    "gdn_semantic_digest", "gdn_deployment_digest",
    "gdn_sha256", "gdn_chunk_rows", "gdn_chunk_rows_bound", "gdn_check_cu_seqlens", "gdn_prefill",
    "gdn_prefill_fused", "gdn_prefill_overlapped", "gdn_decode_step", "gdn_state_resync", "gdn_device_status",
    "gdn_backward", "gdn_backward_workspace_bytes",
    "gdn_prefill_chunked", "gdn_prefill_chunked_workspace_bytes", "GDN_CHUNKED_NATIVE", "GDN_CHUNKED_R2",
    "gdn_trainer_forward", "gdn_prefill_static", "GDN_STATIC_SCRATCH_BYTES",
    "gdn_trainer_forward_chunked", "gdn_trainer_forward_chunked_stash_bytes", "gdn_backward_chunked",
    "gdn_backward_chunked_workspace_bytes",
    "EXPORTS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcpr_gdn.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"libcpr_gdn.so is not built at {LIB_PATH}; run "
                      "`python bitwise_aligned_gated_amd/build.py` (or __graft_entry__.build())")
_lib = ctypes.CDLL(LIB_PATH)

GDN_OK, GDN_EINVAL, GDN_EUNSUPPORTED, GDN_EHIP, GDN_EPOLICY = 0, 1, 2, 3, 4
GDN_F32, GDN_BF16 = 0, 1
GDN_CHUNKED_NATIVE, GDN_CHUNKED_R2 = 0, 1
GDN_STATIC_SCRATCH_BYTES = 256 << 20
_CODES = {1: "GDN_EINVAL", 2: "GDN_EUNSUPPORTED", 3: "GDN_EHIP", 4: "GDN_EPOLICY"}


class GdnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_CODES.get(code, code)}: {msg}")
        self.code = code


class _CPolicy(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("h_k", "h_v", "dk", "dv", "chunk", "io_dtype", "state_dtype", "schedule")]


_P = ctypes.c_void_p
_i32, _i64, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_u8p = ctypes.POINTER(ctypes.c_uint8)
_SIGS = {
    "gdn_last_error": (ctypes.c_char_p, []),
    "gdn_policy_digest": (ctypes.c_int, [ctypes.POINTER(_CPolicy), _u8p]),
    "gdn_sha256": (ctypes.c_int, [_P, _sz, _u8p]),
    "gdn_semantic_digest": (ctypes.c_int, [ctypes.POINTER(_CPolicy), _u8p]),
    "gdn_deployment_digest": (ctypes.c_int, [ctypes.POINTER(_CPolicy), _u8p]),
    "gdn_policy_check": (ctypes.c_int, [_u8p, _u8p]),
    "gdn_policy_validate": (ctypes.c_int, [ctypes.POINTER(_CPolicy)]),
    "gdn_state_bytes": (_sz, [ctypes.POINTER(_CPolicy), _i32]),
    "gdn_state_alloc": (ctypes.c_int, [ctypes.POINTER(_CPolicy), _i32, _P, _P, _sz, _P, _P,
                                       ctypes.POINTER(_P)]),
    "gdn_state_free": (ctypes.c_int, [_P]),
    "gdn_state_data": (_P, [_P]),
    "gdn_state_positions": (_P, [_P]),
    "gdn_state_set_max_workgroups": (ctypes.c_int, [_P, _i64]),
    "gdn_state_set_wait_limit": (ctypes.c_int, [_P, ctypes.c_uint32]),
    "gdn_device_status": (ctypes.c_int, [_P]),
    "gdn_check_cu_seqlens": (ctypes.c_int, [_P, _i32, _i64]),
    "gdn_chunk_rows_bound": (_i64, [_i64, _i32, _i32]),
    "gdn_chunk_rows": (ctypes.c_int, [_P, _P, _i32, _i32, _P]),
    "gdn_prefill": (ctypes.c_int, [_P, _P, _i32, _i64, _P, _i32, _P, _P, _P, _P, _P, _P, _P, _i64, _P, _P, _P]),
    "gdn_prefill_fused": (ctypes.c_int, [_P, _P, _i32, _i64, _P, _i32, _P, _P, _P, _P, _P, _P, _P, _i64, _P, _P]),
    "gdn_prefill_overlapped": (ctypes.c_int, [_P, _P, _i32, _i64, _P, _i32, _P, _P, _P, _P, _P, _P, _P, _i64, _P, _P]),
    "gdn_decode_step": (ctypes.c_int, [_P, _P, _i32, _P, _P, _P, _P, _P, _P, _P, _P]),
    "gdn_state_resync": (ctypes.c_int, [_P, _P, _i32, _P]),
    "gdn_backward_workspace_bytes": (_i64, [ctypes.POINTER(_CPolicy), _i64, _i32]),
    "gdn_prefill_chunked_workspace_bytes": (_i64, [ctypes.POINTER(_CPolicy), _i64, _i32]),
    "gdn_prefill_chunked": (ctypes.c_int, [_P, _P, _i32, _i64, _P, _i32, _P, _P, _P, _P, _P, _P, _P, _i64, _i32,
                                           _P, _sz, _P, _P]),
    "gdn_backward": (ctypes.c_int, [ctypes.POINTER(_CPolicy), _P, _i32, _i64, _P, _P, _P, _P, _P, _P, _i64, _P,
                                    _P, _P, _P, _P, _P, _P, _P, _P, _P, _sz, _P, _P]),
    "gdn_trainer_forward": (ctypes.c_int, [_P, _P, _i32, _i64, _P, _i32, _P, _P, _P, _P, _P, _P, _P, _i64, _P, _P,
                                           _P]),
    "gdn_prefill_static": (ctypes.c_int, [_P, _P, _i32, _i64, _P, _i32, _P, _P, _P, _P, _P, _P, _P, _P]),
    "gdn_r2_ring_bytes": (_i64, [ctypes.POINTER(_CPolicy), _i32]),
    "gdn_r2_workspace_bytes": (_i64, [ctypes.POINTER(_CPolicy), _i32]),
    "gdn_state_attach_r2": (ctypes.c_int, [_P, _P, _sz, _P, _sz]),
    "gdn_trainer_forward_chunked_stash_bytes": (_i64, [ctypes.POINTER(_CPolicy), _i64, _i32]),
    "gdn_trainer_forward_chunked": (ctypes.c_int, [_P, _P, _i32, _i64, _P, _i32, _P, _P, _P, _P, _P, _P, _P, _i64,
                                                   _P, _sz, _P, _P]),
    "gdn_backward_chunked_workspace_bytes": (_i64, [ctypes.POINTER(_CPolicy), _i64, _i32]),
    "gdn_backward_chunked": (ctypes.c_int, [ctypes.POINTER(_CPolicy), _P, _i32, _i64, _P, _P, _P, _P, _P, _P, _i64,
                                            _P, _sz, _P, _P, _P, _P, _P, _P, _P, _P, _P, _sz, _P, _P]),
}
EXPORTS = tuple(_SIGS)
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


def _check(rc: int):
    if rc != GDN_OK:
        raise GdnError(rc, _lib.gdn_last_error().decode())


@dataclass(frozen=True)
class Policy:
    """Numerical policy (C struct gdn_policy)."""
    h_k: int
    h_v: int
    dk: int
    dv: int
    chunk: int = 64
    io: str = "bf16"            # "f32" or "bf16"
    schedule: int = 1
    boundary: str = "f32"       # boundary dtype: "f32" (exact resync) or "bf16" (rounding resync)

    @property
    def io_dtype(self) -> int:
        return {"f32": GDN_F32, "bf16": GDN_BF16}[self.io]

    @property
    def torch_io(self) -> torch.dtype:
        return {"f32": torch.float32, "bf16": torch.bfloat16}[self.io]

    def c(self) -> _CPolicy:
        return _CPolicy(self.h_k, self.h_v, self.dk, self.dv, self.chunk, self.io_dtype,
                        {"f32": GDN_F32, "bf16": GDN_BF16}[self.boundary], self.schedule)

    def validate(self):
        _check(_lib.gdn_policy_validate(ctypes.byref(self.c())))


def gdn_policy_digest(policy: Policy) -> bytes:
    out = (ctypes.c_uint8 * 32)()
    _check(_lib.gdn_policy_digest(ctypes.byref(policy.c()), out))
    return bytes(out)


def gdn_semantic_digest(policy: Policy) -> bytes:
    out = (ctypes.c_uint8 * 32)()
    _check(_lib.gdn_semantic_digest(ctypes.byref(policy.c()), out))
    return bytes(out)


def gdn_deployment_digest(policy: Policy) -> bytes:
    out = (ctypes.c_uint8 * 32)()
    _check(_lib.gdn_deployment_digest(ctypes.byref(policy.c()), out))
    return bytes(out)


def gdn_policy_check(mine: bytes, theirs: bytes):
    a = (ctypes.c_uint8 * 32).from_buffer_copy(mine)
    b = (ctypes.c_uint8 * 32).from_buffer_copy(theirs)
    _check(_lib.gdn_policy_check(a, b))


def gdn_sha256(data) -> bytes:
    buf = bytes(data)
    out = (ctypes.c_uint8 * 32)()
    _check(_lib.gdn_sha256(buf, len(buf), out))
    return bytes(out)


def _host_i32(x) -> torch.Tensor:
    t = torch.as_tensor(x, dtype=torch.int32, device="cpu").contiguous()
    return t


def gdn_check_cu_seqlens(cu_seqlens, total_tokens: int):
    cu = _host_i32(cu_seqlens)
    _check(_lib.gdn_check_cu_seqlens(cu.data_ptr(), cu.numel() - 1, total_tokens))


def gdn_chunk_rows_bound(total_tokens: int, num_seqs: int, chunk: int) -> int:
    r = _lib.gdn_chunk_rows_bound(total_tokens, num_seqs, chunk)
    if r < 0:
        _check(GDN_EINVAL)
    return int(r)


def gdn_chunk_rows(cu_seqlens, chunk: int, pos0=None) -> torch.Tensor:
    """Row offsets [num_seqs + 1] of each sequence's chunk states (host computation)."""
    cu = _host_i32(cu_seqlens)
    n = cu.numel() - 1
    p = None if pos0 is None else torch.as_tensor(pos0, dtype=torch.int64).contiguous()
    out = torch.zeros(n + 1, dtype=torch.int64)
    _check(_lib.gdn_chunk_rows(cu.data_ptr(), None if p is None else p.data_ptr(), n, chunk,
                               out.data_ptr()))
    return out


def _events(events, n: int):
    """None, or a ctypes array of n hipEvent_t handles (ints / c_void_p)."""
    if events is None:
        return None
    if len(events) != n:
        raise ValueError(f"expected {n} events")
    arr = (ctypes.c_void_p * n)()
    for i, e in enumerate(events):
        arr[i] = e.value if isinstance(e, ctypes.c_void_p) else e
    return arr


def _stream_ptr(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _on_stream(fn):
    """Run a binding with the caller's `stream` (a torch.cuda.Stream) as torch's current stream, so
    that every tensor it allocates (outputs, scratch, device copies of host arguments) belongs to the
    stream the kernels run on and the caching allocator cannot hand that memory to other streams'
    work while the kernels still use it."""
    @functools.wraps(fn)
    def run(*args, stream=None, **kw):
        if stream is None:
            return fn(*args, stream=None, **kw)
        with torch.cuda.stream(stream):
            return fn(*args, stream=stream, **kw)
    return run


def _dev(t: torch.Tensor, name: str, dtype, shape, device, align: int = 16) -> torch.Tensor:
    """Check a device tensor argument; vector-loaded tensors need 16-byte alignment, scalars 4."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() and t.data_ptr() % align:
        raise ValueError(f"{name} must be {align}-byte aligned")
    return t


class StatePool:
    """A pool of recurrent states (slots) in torch device memory, bound to a C handle.

    state [num_slots, H_v, dv, dk] fp32 (S transposed), pos [num_slots] int64, and optionally a
    boundary record of the same shapes that resynchronisation commits chunk-start states to."""

    def __init__(self, policy: Policy, num_slots: int, device="cuda", boundary: bool = False):
        policy.validate()
        self.policy = policy
        self.num_slots = num_slots
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        shape = (num_slots, policy.h_v, policy.dv, policy.dk)
        self.state = torch.zeros(shape, dtype=torch.float32, device=self.device)
        self.pos = torch.zeros(num_slots, dtype=torch.int64, device=self.device)
        self.boundary = torch.zeros(shape, dtype=torch.float32, device=self.device) if boundary else None
        self.boundary_pos = (torch.full((num_slots,), -1, dtype=torch.int64, device=self.device)
                             if boundary else None)
        h = _P()
        nbytes = self.state.numel() * 4
        _check(_lib.gdn_state_alloc(ctypes.byref(policy.c()), num_slots, self.state.data_ptr(),
                                    self.pos.data_ptr(), nbytes,
                                    self.boundary.data_ptr() if boundary else None,
                                    self.boundary_pos.data_ptr() if boundary else None,
                                    ctypes.byref(h)))
        self._h = h

    @property
    def handle(self):
        return self._h

    def set_max_workgroups(self, n: int) -> None:
        """Cap the compute kernels of later calls at n workgroups (C gdn_state_set_max_workgroups);
        0 restores one workgroup per work item.  Results are bitwise the same either way."""
        _check(_lib.gdn_state_set_max_workgroups(self._h, int(n)))

    def attach_r2(self, ring=None, workspace=None) -> None:
        """R2 resynchronisation in decode (C gdn_state_attach_r2): allocate the token ring and the
        workspace (or use the given uint8 device tensors) and bind them; needs a boundary record.
        attach_r2(False) detaches."""
        if ring is False:
            _check(_lib.gdn_state_attach_r2(self._h, None, 0, None, 0))
            self.r2_ring = self.r2_workspace = None
            return
        c = ctypes.byref(self.policy.c())
        rb = int(_lib.gdn_r2_ring_bytes(c, self.num_slots))
        wb = int(_lib.gdn_r2_workspace_bytes(c, self.num_slots))
        if rb < 0 or wb < 0:
            _check(GDN_EUNSUPPORTED)
        ring = torch.zeros(rb, dtype=torch.uint8, device=self.device) if ring is None else ring
        workspace = torch.zeros(wb, dtype=torch.uint8, device=self.device) if workspace is None else workspace
        _dev(ring, "ring", torch.uint8, (ring.numel(),), self.device)
        _dev(workspace, "workspace", torch.uint8, (workspace.numel(),), self.device)
        _check(_lib.gdn_state_attach_r2(self._h, ring.data_ptr(), ring.numel(), workspace.data_ptr(),
                                        workspace.numel()))
        self.r2_ring, self.r2_workspace = ring, workspace

    def set_wait_limit(self, polls: int) -> None:
        """Bound of each wait in the overlapped prefill's later calls (C gdn_state_set_wait_limit);
        0 restores the default.  A tiny bound makes waits give up, reported by gdn_device_status."""
        _check(_lib.gdn_state_set_wait_limit(self._h, int(polls)))

    def close(self):
        if getattr(self, "_h", None):
            _lib.gdn_state_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def gdn_device_status(stream=None) -> None:
    """Synchronise the stream and raise GdnError (GDN_EHIP) if a wait of an overlapped prefill on
    the current device gave up since the last check (C gdn_device_status); the check clears it."""
    _check(_lib.gdn_device_status(_stream_ptr(stream)))


def _ids(ids, n: int, device) -> torch.Tensor:
    if ids is None:
        return torch.arange(n, dtype=torch.int32, device=device)
    t = torch.as_tensor(ids, dtype=torch.int32)
    return t.to(device).contiguous()


def _prefill_args(pool, cu_seqlens, q, k, v, a, b, slot_ids, o):
    P, dev = pool.policy, pool.device
    N = q.shape[0]
    if isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.device.type == "cuda":
        cu_d = _dev(cu_seqlens, "cu_seqlens", torch.int32, cu_seqlens.shape, dev, align=4)
    else:
        cu_h = _host_i32(cu_seqlens)
        gdn_check_cu_seqlens(cu_h, N)
        cu_d = cu_h.to(dev)
    B = cu_d.numel() - 1
    ids = _ids(slot_ids, B, dev)
    _dev(ids, "slot_ids", torch.int32, (B,), dev, align=4)
    io = P.torch_io
    _dev(q, "q", io, (N, P.h_k, P.dk), dev)
    _dev(k, "k", io, (N, P.h_k, P.dk), dev)
    _dev(v, "v", io, (N, P.h_v, P.dv), dev)
    _dev(a, "a", torch.float32, (N, P.h_v), dev, align=4)
    _dev(b, "b", torch.float32, (N, P.h_v), dev, align=4)
    if o is None:
        o = torch.empty((N, P.h_v, P.dv), dtype=io, device=dev)
    _dev(o, "o", io, (N, P.h_v, P.dv), dev)
    return N, B, cu_d, ids, o


@_on_stream
def gdn_prefill_fused(pool: StatePool, cu_seqlens, q, k, v, a, b, slot_ids=None, from_state: bool = False,
                      o=None, chunk_states=None, stream=None, events=None):
    """One-pass prefill (C gdn_prefill_fused); bitwise equal to gdn_prefill.  chunk_states None:
    no stash.  Returns (o, chunk_states)."""
    P, dev = pool.policy, pool.device
    N, B, cu_d, ids, o = _prefill_args(pool, cu_seqlens, q, k, v, a, b, slot_ids, o)
    rows = 0
    if chunk_states is not None:
        _dev(chunk_states, "chunk_states", torch.float32, (chunk_states.shape[0], P.h_v, P.dv, P.dk), dev)
        rows = chunk_states.shape[0]
    _check(_lib.gdn_prefill_fused(pool.handle, cu_d.data_ptr(), B, N, ids.data_ptr(), int(bool(from_state)),
                                  q.data_ptr(), k.data_ptr(), v.data_ptr(), a.data_ptr(), b.data_ptr(),
                                  o.data_ptr(), None if chunk_states is None else chunk_states.data_ptr(), rows,
                                  _stream_ptr(stream), _events(events, 2)))
    return o, chunk_states


@_on_stream
def gdn_prefill_overlapped(pool: StatePool, cu_seqlens, q, k, v, a, b, slot_ids=None, from_state: bool = False,
                           o=None, chunk_states=None, stream=None, events=None):
    """Overlapped prefill (C gdn_prefill_overlapped): pass 1 and the chunk outputs in one launch;
    bitwise equal to gdn_prefill.  More workgroups than CUs, or chunks above 64 tokens, run the
    one-pass kernel instead.  chunk_states None: no stash.  Returns (o, chunk_states)."""
    P, dev = pool.policy, pool.device
    N, B, cu_d, ids, o = _prefill_args(pool, cu_seqlens, q, k, v, a, b, slot_ids, o)
    rows = 0
    if chunk_states is not None:
        _dev(chunk_states, "chunk_states", torch.float32, (chunk_states.shape[0], P.h_v, P.dv, P.dk), dev)
        rows = chunk_states.shape[0]
    _check(_lib.gdn_prefill_overlapped(pool.handle, cu_d.data_ptr(), B, N, ids.data_ptr(), int(bool(from_state)),
                                       q.data_ptr(), k.data_ptr(), v.data_ptr(), a.data_ptr(), b.data_ptr(),
                                       o.data_ptr(), None if chunk_states is None else chunk_states.data_ptr(),
                                       rows, _stream_ptr(stream), _events(events, 2)))
    return o, chunk_states


@_on_stream
def gdn_prefill(pool: StatePool, cu_seqlens, q, k, v, a, b, slot_ids=None, from_state: bool = False,
                o=None, chunk_states=None, c_stash=True, stream=None, events=None):
    """Prefill / trainer forward over a packed batch (C gdn_prefill).

    cu_seqlens: host sequence (checked on the host, then copied) or a device int32 tensor.
    c_stash: True allocates the [N][H_v][dv] fp32 scratch in which pass 1 keeps every token's c for
    pass 2 (168 MB for 10240 tokens at 32 heads of 128: callers that cannot allocate per call, such
    as code under graph capture, pass a tensor they own); a tensor is used as that scratch; None or
    False passes NULL (pass 2 predicts c again).  The bits of every result are the same either way.
    stream: a torch.cuda.Stream (default: the current stream); every tensor the call allocates is
    allocated on it.
    Returns (o, chunk_states); chunk_states is allocated with the bound's row count when None."""
    P, dev = pool.policy, pool.device
    N, B, cu_d, ids, o = _prefill_args(pool, cu_seqlens, q, k, v, a, b, slot_ids, o)
    bound = gdn_chunk_rows_bound(N, B, P.chunk)
    if chunk_states is None:
        chunk_states = torch.empty((max(bound, 1), P.h_v, P.dv, P.dk), dtype=torch.float32, device=dev)
    _dev(chunk_states, "chunk_states", torch.float32, (chunk_states.shape[0], P.h_v, P.dv, P.dk), dev)
    if c_stash is True:
        c_stash = torch.empty((N, P.h_v, P.dv), dtype=torch.float32, device=dev) if N > 0 else None
    if c_stash is not None and c_stash is not False:
        _dev(c_stash, "c_stash", torch.float32, (N, P.h_v, P.dv), dev)
    stash_ptr = c_stash.data_ptr() if isinstance(c_stash, torch.Tensor) else None
    _check(_lib.gdn_prefill(pool.handle, cu_d.data_ptr(), B, N, ids.data_ptr(), int(bool(from_state)),
                            q.data_ptr(), k.data_ptr(), v.data_ptr(), a.data_ptr(), b.data_ptr(),
                            o.data_ptr(), chunk_states.data_ptr(), chunk_states.shape[0], stash_ptr,
                            _stream_ptr(stream), _events(events, 3)))
    return o, chunk_states


def gdn_prefill_static(pool: StatePool, cu_seqlens: torch.Tensor, q, k, v, a, b, slot_ids: torch.Tensor,
                       o: torch.Tensor, from_state: bool = False, stream=None, events=None):
    """gdn_prefill that allocates nothing (C gdn_prefill_static): its scratch is a library-owned
    static device buffer of GDN_STATIC_SCRATCH_BYTES.  Every argument is a caller-owned device
    tensor (cu_seqlens and slot_ids int32 on the pool's device, o preallocated), so that neither the
    library nor this binding allocates; the results are gdn_prefill's bits.  Calls that overlap on
    one device race on the buffer.  Returns o."""
    P, dev = pool.policy, pool.device
    N = q.shape[0]
    _dev(cu_seqlens, "cu_seqlens", torch.int32, cu_seqlens.shape, dev, align=4)
    B = cu_seqlens.numel() - 1
    _dev(slot_ids, "slot_ids", torch.int32, (B,), dev, align=4)
    io = P.torch_io
    _dev(q, "q", io, (N, P.h_k, P.dk), dev)
    _dev(k, "k", io, (N, P.h_k, P.dk), dev)
    _dev(v, "v", io, (N, P.h_v, P.dv), dev)
    _dev(a, "a", torch.float32, (N, P.h_v), dev, align=4)
    _dev(b, "b", torch.float32, (N, P.h_v), dev, align=4)
    _dev(o, "o", io, (N, P.h_v, P.dv), dev)
    _check(_lib.gdn_prefill_static(pool.handle, cu_seqlens.data_ptr(), B, N, slot_ids.data_ptr(),
                                   int(bool(from_state)), q.data_ptr(), k.data_ptr(), v.data_ptr(), a.data_ptr(),
                                   b.data_ptr(), o.data_ptr(), _stream_ptr(stream), _events(events, 3)))
    return o


@_on_stream
def gdn_trainer_forward(pool: StatePool, cu_seqlens, q, k, v, a, b, slot_ids=None, from_state: bool = False,
                        o=None, chunk_states=None, cw=None, stream=None, events=None):
    """Trainer forward (C gdn_trainer_forward): gdn_prefill that also keeps every token's c and w
    for gdn_backward.  Returns (o, chunk_states, cw)."""
    P, dev = pool.policy, pool.device
    N, B, cu_d, ids, o = _prefill_args(pool, cu_seqlens, q, k, v, a, b, slot_ids, o)
    bound = gdn_chunk_rows_bound(N, B, P.chunk)
    if chunk_states is None:
        chunk_states = torch.empty((max(bound, 1), P.h_v, P.dv, P.dk), dtype=torch.float32, device=dev)
    _dev(chunk_states, "chunk_states", torch.float32, (chunk_states.shape[0], P.h_v, P.dv, P.dk), dev)
    if cw is None:
        cw = torch.empty((2, N, P.h_v, P.dv), dtype=torch.float32, device=dev)
    _dev(cw, "cw", torch.float32, (2, N, P.h_v, P.dv), dev)
    _check(_lib.gdn_trainer_forward(pool.handle, cu_d.data_ptr(), B, N, ids.data_ptr(), int(bool(from_state)),
                                    q.data_ptr(), k.data_ptr(), v.data_ptr(), a.data_ptr(), b.data_ptr(),
                                    o.data_ptr(), chunk_states.data_ptr(), chunk_states.shape[0], cw.data_ptr(),
                                    _stream_ptr(stream), _events(events, 3)))
    return o, chunk_states, cw


@_on_stream
def gdn_decode_step(pool: StatePool, q, k, v, a, b, slot_ids=None, o=None, stream=None, events=None):
    """One token for each listed slot (C gdn_decode_step).  Returns o [batch, H_v, dv]."""
    P, dev = pool.policy, pool.device
    n = q.shape[0]
    ids = _ids(slot_ids, n, dev)
    _dev(ids, "slot_ids", torch.int32, (n,), dev, align=4)
    io = P.torch_io
    _dev(q, "q", io, (n, P.h_k, P.dk), dev)
    _dev(k, "k", io, (n, P.h_k, P.dk), dev)
    _dev(v, "v", io, (n, P.h_v, P.dv), dev)
    _dev(a, "a", torch.float32, (n, P.h_v), dev, align=4)
    _dev(b, "b", torch.float32, (n, P.h_v), dev, align=4)
    if o is None:
        o = torch.empty((n, P.h_v, P.dv), dtype=io, device=dev)
    _dev(o, "o", io, (n, P.h_v, P.dv), dev)
    _check(_lib.gdn_decode_step(pool.handle, ids.data_ptr(), n, q.data_ptr(), k.data_ptr(),
                                v.data_ptr(), a.data_ptr(), b.data_ptr(), o.data_ptr(),
                                _stream_ptr(stream), _events(events, 2)))
    return o


@_on_stream
def gdn_state_resync(pool: StatePool, slot_ids, stream=None):
    """Resynchronise listed slots at chunk starts (C gdn_state_resync)."""
    dev = pool.device
    ids = _ids(slot_ids, 0, dev)
    _check(_lib.gdn_state_resync(pool.handle, ids.data_ptr(), ids.numel(), _stream_ptr(stream)))


def gdn_backward_workspace_bytes(policy: Policy, total_tokens: int, num_seqs: int) -> int:
    r = _lib.gdn_backward_workspace_bytes(ctypes.byref(policy.c()), total_tokens, num_seqs)
    if r < 0:
        _check(GDN_EINVAL)
    return int(r)


def _backward_args(P, cu_seqlens, q, k, v, a, b, chunk_states, d_o, d_state, want_d_state0, out):
    """Checks of a backward call's inputs; the gradient outputs (allocated where `out` has none)."""
    dev = q.device
    N = q.shape[0]
    if isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.device.type == "cuda":
        cu_d = _dev(cu_seqlens, "cu_seqlens", torch.int32, cu_seqlens.shape, dev, align=4)
    else:
        cu_h = _host_i32(cu_seqlens)
        gdn_check_cu_seqlens(cu_h, N)
        cu_d = cu_h.to(dev)
    B = cu_d.numel() - 1
    io = P.torch_io
    _dev(q, "q", io, (N, P.h_k, P.dk), dev)
    _dev(k, "k", io, (N, P.h_k, P.dk), dev)
    _dev(v, "v", io, (N, P.h_v, P.dv), dev)
    _dev(a, "a", torch.float32, (N, P.h_v), dev, align=4)
    _dev(b, "b", torch.float32, (N, P.h_v), dev, align=4)
    _dev(d_o, "d_o", io, (N, P.h_v, P.dv), dev)
    _dev(chunk_states, "chunk_states", torch.float32, (chunk_states.shape[0], P.h_v, P.dv, P.dk), dev)
    if d_state is not None:
        _dev(d_state, "d_state", torch.float32, (B, P.h_v, P.dv, P.dk), dev)
    out = dict(out or {})
    shapes = {"dq": (N, P.h_k, P.dk), "dk": (N, P.h_k, P.dk), "dv": (N, P.h_v, P.dv), "da": (N, P.h_v),
              "db": (N, P.h_v)}
    if want_d_state0:
        shapes["d_state0"] = (B, P.h_v, P.dv, P.dk)
    for name, shape in shapes.items():
        if out.get(name) is None:
            out[name] = torch.empty(shape, dtype=torch.float32, device=dev)
        _dev(out[name], name, torch.float32, shape, dev)
    return dev, N, B, cu_d, out


@_on_stream
def gdn_backward(policy: Policy, cu_seqlens, q, k, v, a, b, chunk_states, d_o, d_state=None,
                 want_d_state0: bool = False, workspace=None, out=None, stream=None, events=None, cw=None):
    """Gradients of a trainer forward (C gdn_backward) from its inputs and chunk-state stash.

    Returns a dict of fp32 device tensors dq, dk [N, H_k, d_k], dv [N, H_v, d_v], da, db [N, H_v]
    and, when want_d_state0, d_state0 [num_seqs, H_v, d_v, d_k].  `out` may supply any of them."""
    P = policy
    dev, N, B, cu_d, out = _backward_args(P, cu_seqlens, q, k, v, a, b, chunk_states, d_o, d_state, want_d_state0,
                                          out)
    if cw is not None:
        _dev(cw, "cw", torch.float32, (2, N, P.h_v, P.dv), dev)
    need = gdn_backward_workspace_bytes(P, N, B)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _dev(workspace, "workspace", torch.uint8, (workspace.numel(),), dev)
    d0 = out.get("d_state0")
    _check(_lib.gdn_backward(ctypes.byref(P.c()), cu_d.data_ptr(), B, N, q.data_ptr(), k.data_ptr(),
                             v.data_ptr(), a.data_ptr(), b.data_ptr(), chunk_states.data_ptr(),
                             chunk_states.shape[0], None if cw is None else cw.data_ptr(), d_o.data_ptr(),
                             None if d_state is None else d_state.data_ptr(),
                             out["dq"].data_ptr(), out["dk"].data_ptr(), out["dv"].data_ptr(),
                             out["da"].data_ptr(), out["db"].data_ptr(), None if d0 is None else d0.data_ptr(),
                             workspace.data_ptr(), workspace.numel(), _stream_ptr(stream), _events(events, 4)))
    return out


def gdn_prefill_chunked_workspace_bytes(policy: Policy, total_tokens: int, num_seqs: int) -> int:
    r = _lib.gdn_prefill_chunked_workspace_bytes(ctypes.byref(policy.c()), total_tokens, num_seqs)
    if r < 0:
        _check(GDN_EUNSUPPORTED if policy.dk not in (32, 64, 128) else GDN_EINVAL)
    return int(r)


@_on_stream
def gdn_prefill_chunked(pool: StatePool, cu_seqlens, q, k, v, a, b, slot_ids=None, from_state: bool = False,
                        outputs: int = GDN_CHUNKED_NATIVE, o=None, chunk_states=None, workspace=None, stream=None,
                        events=None):
    """Chunkwise evaluation on matrix cores (C gdn_prefill_chunked): outputs=GDN_CHUNKED_NATIVE
    or GDN_CHUNKED_R2.  Returns (o, chunk_states)."""
    P, dev = pool.policy, pool.device
    N, B, cu_d, ids, o = _prefill_args(pool, cu_seqlens, q, k, v, a, b, slot_ids, o)
    bound = gdn_chunk_rows_bound(N, B, P.chunk)
    if chunk_states is None:
        chunk_states = torch.empty((max(bound, 1), P.h_v, P.dv, P.dk), dtype=torch.float32, device=dev)
    _dev(chunk_states, "chunk_states", torch.float32, (chunk_states.shape[0], P.h_v, P.dv, P.dk), dev)
    need = gdn_prefill_chunked_workspace_bytes(P, N, B)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _dev(workspace, "workspace", torch.uint8, (workspace.numel(),), dev)
    _check(_lib.gdn_prefill_chunked(pool.handle, cu_d.data_ptr(), B, N, ids.data_ptr(), int(bool(from_state)),
                                    q.data_ptr(), k.data_ptr(), v.data_ptr(), a.data_ptr(), b.data_ptr(),
                                    o.data_ptr(), chunk_states.data_ptr(), chunk_states.shape[0], int(outputs),
                                    workspace.data_ptr(), workspace.numel(), _stream_ptr(stream),
                                    _events(events, 4)))
    return o, chunk_states


def gdn_trainer_forward_chunked_stash_bytes(policy: Policy, total_tokens: int, num_seqs: int) -> int:
    r = _lib.gdn_trainer_forward_chunked_stash_bytes(ctypes.byref(policy.c()), total_tokens, num_seqs)
    if r < 0:
        _check(GDN_EUNSUPPORTED if policy.dk not in (32, 64, 128) else GDN_EINVAL)
    return int(r)


@_on_stream
def gdn_trainer_forward_chunked(pool: StatePool, cu_seqlens, q, k, v, a, b, slot_ids=None, from_state: bool = False,
                                o=None, chunk_states=None, stash=None, stream=None, events=None):
    """Chunkwise trainer forward on matrix cores (C gdn_trainer_forward_chunked): the native
    chunked prefill that also keeps the stash gdn_backward_chunked reads.  Returns
    (o, chunk_states, stash)."""
    P, dev = pool.policy, pool.device
    N, B, cu_d, ids, o = _prefill_args(pool, cu_seqlens, q, k, v, a, b, slot_ids, o)
    bound = gdn_chunk_rows_bound(N, B, P.chunk)
    if chunk_states is None:
        chunk_states = torch.empty((max(bound, 1), P.h_v, P.dv, P.dk), dtype=torch.float32, device=dev)
    _dev(chunk_states, "chunk_states", torch.float32, (chunk_states.shape[0], P.h_v, P.dv, P.dk), dev)
    need = gdn_trainer_forward_chunked_stash_bytes(P, N, B)
    if stash is None:
        stash = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _dev(stash, "stash", torch.uint8, (stash.numel(),), dev)
    _check(_lib.gdn_trainer_forward_chunked(pool.handle, cu_d.data_ptr(), B, N, ids.data_ptr(), int(bool(from_state)),
                                            q.data_ptr(), k.data_ptr(), v.data_ptr(), a.data_ptr(), b.data_ptr(),
                                            o.data_ptr(), chunk_states.data_ptr(), chunk_states.shape[0],
                                            stash.data_ptr(), stash.numel(), _stream_ptr(stream),
                                            _events(events, 4)))
    return o, chunk_states, stash


def gdn_backward_chunked_workspace_bytes(policy: Policy, total_tokens: int, num_seqs: int) -> int:
    r = _lib.gdn_backward_chunked_workspace_bytes(ctypes.byref(policy.c()), total_tokens, num_seqs)
    if r < 0:
        _check(GDN_EUNSUPPORTED if policy.dk not in (32, 64, 128) else GDN_EINVAL)
    return int(r)


@_on_stream
def gdn_backward_chunked(policy: Policy, cu_seqlens, q, k, v, a, b, chunk_states, stash, d_o, d_state=None,
                         want_d_state0: bool = False, workspace=None, out=None, stream=None, events=None):
    """Gradients of a chunkwise trainer forward (C gdn_backward_chunked) from its inputs, chunk
    states and stash.  Returns the dict gdn_backward returns."""
    P = policy
    dev, N, B, cu_d, out = _backward_args(P, cu_seqlens, q, k, v, a, b, chunk_states, d_o, d_state, want_d_state0,
                                          out)
    _dev(stash, "stash", torch.uint8, (stash.numel(),), dev)
    need = gdn_backward_chunked_workspace_bytes(P, N, B)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _dev(workspace, "workspace", torch.uint8, (workspace.numel(),), dev)
    d0 = out.get("d_state0")
    _check(_lib.gdn_backward_chunked(ctypes.byref(P.c()), cu_d.data_ptr(), B, N, q.data_ptr(), k.data_ptr(),
                                     v.data_ptr(), a.data_ptr(), b.data_ptr(), chunk_states.data_ptr(),
                                     chunk_states.shape[0], stash.data_ptr(), stash.numel(), d_o.data_ptr(),
                                     None if d_state is None else d_state.data_ptr(),
                                     out["dq"].data_ptr(), out["dk"].data_ptr(), out["dv"].data_ptr(),
                                     out["da"].data_ptr(), out["db"].data_ptr(),
                                     None if d0 is None else d0.data_ptr(),
                                     workspace.data_ptr(), workspace.numel(), _stream_ptr(stream),
                                     _events(events, 4)))
    return out
