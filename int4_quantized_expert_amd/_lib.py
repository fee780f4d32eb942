"""ctypes binding of libmoe_layer.so: argument marshalling only.

Each function takes torch tensors that live on the GPU, passes their device
pointers and byte sizes to the C entry point of the same name, and raises
MoeError on a non-zero return code.  `stream` defaults to torch's current
stream on the tensors' device.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_layer.so")

MOE_F32 = 0
MOE_BF16 = 1

ERRORS = {
    -1: "MOE_EINVAL",
    -2: "MOE_ENODEV",
    -3: "MOE_EHIP",
    -4: "MOE_ENOMEM",
    -5: "MOE_ERANGE",
    -6: "MOE_ENOSPC",
    -7: "MOE_ETIMEOUT",
    -8: "MOE_EIO",
    -9: "MOE_EOVERFLOW",
}


class MoeError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{ERRORS.get(code, code)}: {message}")
        self.code = code


class MoeDesc(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32),
        ("n_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("inter", ctypes.c_int32),
        ("shared_inter", ctypes.c_int32),
        ("bits", ctypes.c_int32),
        ("group_size", ctypes.c_int32),
        ("act_dtype", ctypes.c_int32),
        ("sb_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("blob_stride", ctypes.c_int64),
        ("shared_stride", ctypes.c_int64),
        ("pool_bytes", ctypes.c_int64),
    ]


class GdnDesc(ctypes.Structure):
    """Descriptor of the gated-delta-rule recurrence (gdn_recurrence.h)."""
    _fields_ = [
        ("n_k_heads", ctypes.c_int32),
        ("n_v_heads", ctypes.c_int32),
        ("d_k", ctypes.c_int32),
        ("d_v", ctypes.c_int32),
        ("act_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("eps", ctypes.c_float),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(hipcc --offload-arch=gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        dp = ctypes.POINTER(MoeDesc)
        L.moe_blob_bytes.argtypes = [dp, i32]
        L.moe_blob_bytes.restype = i64
        L.moe_workspace_bytes.argtypes = [dp, i32]
        L.moe_workspace_bytes.restype = sz
        L.moe_workspace_init.argtypes = [vp, sz, vp]
        L.moe_workspace_init.restype = ctypes.c_int
        L.moe_layer_forward.argtypes = [dp, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp]
        L.moe_layer_forward.restype = ctypes.c_int
        L.moe_layer_forward_staged.argtypes = [dp, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp]
        L.moe_layer_forward_staged.restype = ctypes.c_int
        L.moe_layer_forward_scalar.argtypes = [dp, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp]
        L.moe_layer_forward_scalar.restype = ctypes.c_int
        L.moe_router_topk.argtypes = [dp, i32, vp, vp, vp, vp, vp, sz, vp]
        L.moe_router_topk.restype = ctypes.c_int
        L.moe_experts_forward.argtypes = [dp, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_experts_forward.restype = ctypes.c_int
        L.moe_layer_forward_chain.argtypes = [dp, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp]
        L.moe_layer_forward_chain.restype = ctypes.c_int
        L.moe_stack_forward.argtypes = [dp, i32, i32, vp, i64, vp, i64, vp, i64, vp, vp, i64, vp, i64, vp, i64,
                                        vp, vp, vp, sz, vp]
        L.moe_stack_forward.restype = ctypes.c_int
        L.moe_layer_forward_noalloc.argtypes = [dp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.moe_layer_forward_noalloc.restype = ctypes.c_int
        L.moe_residual_add.argtypes = [i32, i32, i32, vp, vp, vp, vp]
        L.moe_residual_add.restype = ctypes.c_int
        L.moe_status_check.argtypes = [vp, vp]
        L.moe_status_check.restype = ctypes.c_int
        L.moe_cache_create.argtypes = [i32, i64, vp, vp, i32, i32]
        L.moe_cache_create.restype = vp
        L.moe_cache_acquire.argtypes = [vp, i32, vp, i32, vp, vp, vp]
        L.moe_cache_acquire.restype = ctypes.c_int
        L.moe_cache_release.argtypes = [vp, i32, vp]
        L.moe_cache_release.restype = ctypes.c_int
        L.moe_cache_stats.argtypes = [vp, ctypes.POINTER(i64), ctypes.POINTER(i64), ctypes.POINTER(i64)]
        L.moe_cache_stats.restype = None
        L.moe_cache_set_policy.argtypes = [vp, i32]
        L.moe_cache_set_policy.restype = ctypes.c_int
        L.moe_cache_inject_fault.argtypes = [vp, i32]
        L.moe_cache_inject_fault.restype = ctypes.c_int
        L.moe_cache_slot_of.argtypes = [vp, i32, i32]
        L.moe_cache_slot_of.restype = ctypes.c_int
        L.moe_cache_destroy.argtypes = [vp]
        L.moe_cache_destroy.restype = None
        L.moe_cache_last_error.argtypes = []
        L.moe_cache_last_error.restype = ctypes.c_char_p
        L.moe_cache_create_from_store.argtypes = [i32, vp, vp, vp, i32]
        L.moe_cache_create_from_store.restype = vp
        L.moe_store_create.argtypes = [ctypes.c_char_p, i32, i32, i64, i64]
        L.moe_store_create.restype = vp
        L.moe_store_open.argtypes = [ctypes.c_char_p, i32]
        L.moe_store_open.restype = vp
        L.moe_store_info.argtypes = [vp, ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(i64),
                                     ctypes.POINTER(i64)]
        L.moe_store_info.restype = ctypes.c_int
        L.moe_store_read.argtypes = [vp, i32, i32, vp]
        L.moe_store_read.restype = ctypes.c_int
        L.moe_store_write.argtypes = [vp, i32, i32, vp]
        L.moe_store_write.restype = ctypes.c_int
        L.moe_store_close.argtypes = [vp]
        L.moe_store_close.restype = None
        L.moe_set_launch_events.argtypes = [ctypes.POINTER(vp), i32, ctypes.POINTER(i32)]
        L.moe_set_launch_events.restype = ctypes.c_int
        L.gdn_recurrence_forward.argtypes = [ctypes.POINTER(GdnDesc), i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]
        L.gdn_recurrence_forward.restype = ctypes.c_int
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def last_error() -> str:
    return lib().moe_last_error().decode()


def _check(rc: int) -> None:
    if rc != 0:
        raise MoeError(rc, last_error())


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _stream(stream, like=None):
    if stream is None:
        import torch
        dev = like.device if like is not None else None
        return torch.cuda.current_stream(dev).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def desc_for(hidden, n_experts, top_k, inter, shared_inter, bits=4, act="bf16", sb="bf16", out="f32",
             pool_bytes=0, blob_stride=None, shared_stride=None) -> MoeDesc:
    """Descriptor with strides defaulting to the blob size rounded up to 4096 bytes."""
    code = {"f32": MOE_F32, "bf16": MOE_BF16}
    d = MoeDesc(hidden, n_experts, top_k, inter, shared_inter, bits, 64, code[act], code[sb], code[out],
                0, 0, pool_bytes)
    d.blob_stride = 1 << 40   # placeholder so the size query validates
    d.shared_stride = 1 << 40
    d.pool_bytes = max(pool_bytes, 1 << 40)
    rb = blob_bytes(d, False)
    sb_ = blob_bytes(d, True)
    d.blob_stride = blob_stride if blob_stride is not None else (rb + 4095) // 4096 * 4096
    d.shared_stride = shared_stride if shared_stride is not None else (sb_ + 4095) // 4096 * 4096
    d.pool_bytes = pool_bytes
    return d


def blob_bytes(d: MoeDesc, shared: bool) -> int:
    n = lib().moe_blob_bytes(ctypes.byref(d), 1 if shared else 0)
    if n < 0:
        raise MoeError(-1, "invalid descriptor")
    return n


def workspace_bytes(d: MoeDesc, T_max: int) -> int:
    n = lib().moe_workspace_bytes(ctypes.byref(d), T_max)
    if n == 0:
        raise MoeError(-1, "invalid descriptor or T_max")
    return n


def workspace_init(ws, stream=None) -> None:
    _check(lib().moe_workspace_init(_ptr(ws), _nbytes(ws), _stream(stream, ws)))


def layer_forward(d: MoeDesc, T: int, x, router_w, slot_table, pool, shared_w, out, ws,
                  topk_ids=None, topk_w=None, stream=None) -> None:
    _check(lib().moe_layer_forward(ctypes.byref(d), T, _ptr(x), _ptr(router_w), _ptr(slot_table), _ptr(pool),
                                   _ptr(shared_w), _ptr(out), _ptr(ws), _nbytes(ws), _ptr(topk_ids),
                                   _ptr(topk_w), _stream(stream, ws)))


def layer_forward_noalloc(d: MoeDesc, T: int, x, router_w, slot_table, pool, shared_w, out, topk_ids=None,
                          topk_w=None, status=None, stream=None) -> None:
    """layer_forward on the library's own fixed scratch (moe_layer_forward_noalloc): no workspace argument,
    no device allocation.  status: optional 4-byte device tensor that receives the device error flags."""
    _check(lib().moe_layer_forward_noalloc(ctypes.byref(d), T, _ptr(x), _ptr(router_w), _ptr(slot_table), _ptr(pool),
                                           _ptr(shared_w), _ptr(out), _ptr(topk_ids), _ptr(topk_w), _ptr(status),
                                           _stream(stream, out)))


def layer_forward_chain(d: MoeDesc, T: int, x, router_w, slot_table, pool, shared_w, out, x_next, ws,
                        topk_ids=None, topk_w=None, stream=None) -> None:
    """layer_forward, then x_next = x + out (moe_layer_forward_chain)."""
    _check(lib().moe_layer_forward_chain(ctypes.byref(d), T, _ptr(x), _ptr(router_w), _ptr(slot_table), _ptr(pool),
                                         _ptr(shared_w), _ptr(out), _ptr(x_next), _ptr(ws), _nbytes(ws),
                                         _ptr(topk_ids), _ptr(topk_w), _stream(stream, ws)))


def layer_forward_staged(d: MoeDesc, T: int, x, router_w, slot_table, pool, shared_w, out, ws,
                         topk_ids=None, topk_w=None, stream=None) -> None:
    """Same as layer_forward but always on the staged (multi-launch) kernels."""
    _check(lib().moe_layer_forward_staged(ctypes.byref(d), T, _ptr(x), _ptr(router_w), _ptr(slot_table),
                                          _ptr(pool), _ptr(shared_w), _ptr(out), _ptr(ws), _nbytes(ws),
                                          _ptr(topk_ids), _ptr(topk_w), _stream(stream, ws)))


def layer_forward_scalar(d: MoeDesc, T: int, x, router_w, slot_table, pool, shared_w, out, ws,
                         topk_ids=None, topk_w=None, stream=None) -> None:
    """The layer on the scalar kernels (one thread per output value): the fast kernels' order of sums."""
    _check(lib().moe_layer_forward_scalar(ctypes.byref(d), T, _ptr(x), _ptr(router_w), _ptr(slot_table), _ptr(pool),
                                          _ptr(shared_w), _ptr(out), _ptr(ws), _nbytes(ws), _ptr(topk_ids),
                                          _ptr(topk_w), _stream(stream, ws)))


def gdn_desc(n_k_heads, n_v_heads, d_k, d_v, act="bf16", out="f32", scale=None, eps=1e-6) -> GdnDesc:
    """Descriptor for the gated delta rule; scale defaults to 1/sqrt(d_k)."""
    dt = {"f32": MOE_F32, "bf16": MOE_BF16}
    return GdnDesc(n_k_heads, n_v_heads, d_k, d_v, dt[act], dt[out],
                   float(d_k ** -0.5 if scale is None else scale), float(eps))


def gdn_forward(d: GdnDesc, B: int, T: int, q, k, v, alpha, beta, state, out, stream=None) -> None:
    """Advance B sequences by T tokens of the gated delta rule; state is updated in place."""
    _check(lib().gdn_recurrence_forward(ctypes.byref(d), B, T, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                        _ptr(state), _ptr(out), _stream(stream, state)))


def router_topk(d: MoeDesc, T: int, x, router_w, topk_ids, topk_w, ws, stream=None) -> None:
    _check(lib().moe_router_topk(ctypes.byref(d), T, _ptr(x), _ptr(router_w), _ptr(topk_ids), _ptr(topk_w),
                                 _ptr(ws), _nbytes(ws), _stream(stream, ws)))


def experts_forward(d: MoeDesc, T: int, x, topk_ids, topk_w, slot_table, pool, shared_w, out, ws,
                    stream=None) -> None:
    _check(lib().moe_experts_forward(ctypes.byref(d), T, _ptr(x), _ptr(topk_ids), _ptr(topk_w), _ptr(slot_table),
                                     _ptr(pool), _ptr(shared_w), _ptr(out), _ptr(ws), _nbytes(ws),
                                     _stream(stream, ws)))


def stack_forward(d: MoeDesc, n_layers: int, T: int, x, x_stride: int, router_w, router_stride: int, slot_table,
                  slot_stride: int, pool, shared_w, shared_stride: int, out, out_stride: int, ws,
                  x_chain=None, chain_stride: int = 0, topk_ids=None, topk_w=None, stream=None) -> None:
    """n_layers layers in order (moe_stack_forward); strides in bytes; layer l's data at base + l * stride.
    With x_chain, layer l > 0 reads x_chain + (l - 1) * chain_stride and layer l writes its input + output
    at x_chain + l * chain_stride."""
    _check(lib().moe_stack_forward(ctypes.byref(d), n_layers, T, _ptr(x), x_stride, _ptr(router_w), router_stride,
                                   _ptr(slot_table), slot_stride, _ptr(pool), _ptr(shared_w), shared_stride,
                                   _ptr(out), out_stride, _ptr(x_chain), chain_stride, _ptr(topk_ids),
                                   _ptr(topk_w), _ptr(ws), _nbytes(ws), _stream(stream, ws)))


def residual_add(T: int, H: int, act: str, x, y, x_next, stream=None) -> None:
    """x_next = x + y (fp32 sum; rounded to bf16 when act == "bf16"); device tensors or addresses."""
    _check(lib().moe_residual_add(T, H, MOE_BF16 if act == "bf16" else MOE_F32, _ptr(x), _ptr(y), _ptr(x_next),
                                  _stream(stream, x if hasattr(x, "device") else None)))


def status_check(ws, stream=None) -> None:
    """Blocking: raises MoeError(MOE_ERANGE) if a kernel skipped a pair since the last check."""
    _check(lib().moe_status_check(_ptr(ws), _stream(stream, ws)))


class LaunchTimer:
    """Per-kernel execution times of one library call, from moe_set_launch_events.

    Holds `capacity` timing events (torch.cuda.Event objects, so their lifetime
    is torch's); kernel j of the call gets events 2j and 2j+1, stamped by its
    own dispatch.  arm() must directly precede the library call to be timed;
    after a synchronize, kernel_us() gives one duration per kernel.
    """

    def __init__(self, capacity: int = 8):
        import torch
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(capacity)]
        for e in self.events:      # torch creates the HIP event lazily, at the first record
            e.record()
        self._handles = (ctypes.c_void_p * capacity)(*[e.cuda_event for e in self.events])
        self._n = ctypes.c_int32(0)

    def arm(self) -> None:
        _check(lib().moe_set_launch_events(self._handles, len(self.events), ctypes.byref(self._n)))

    @property
    def n_recorded(self) -> int:
        return self._n.value

    def kernel_us(self) -> list[float]:
        n = self._n.value
        return [self.events[j].elapsed_time(self.events[j + 1]) * 1e3 for j in range(0, n - 1, 2)]


def clear_launch_events() -> None:
    _check(lib().moe_set_launch_events(None, 0, None))


def _event_handle(ev) -> int | None:
    if ev is None or isinstance(ev, int):
        return ev
    if ev.cuda_event == 0:      # torch creates the HIP event lazily, at the first record
        ev.record()
    return ev.cuda_event


def _stream_handle(st) -> int | None:
    if st is None or isinstance(st, int):
        return st
    return st.cuda_stream


STORE_DIRECT = 1
CACHE_KEEP_COUNTS = 1


class ExpertStore:
    """One container file of fixed-stride expert blobs (moe_store_*).

    ExpertStore.create(path, ...) makes a writable store; ExpertStore(path)
    opens one read-only (direct=True asks for O_DIRECT reads).  Blobs are
    numpy uint8 arrays (or raw host addresses) of `stride` bytes.
    """

    def __init__(self, path: str, direct: bool = False, _handle=None):
        if _handle is None:
            _handle = lib().moe_store_open(os.fsencode(path), STORE_DIRECT if direct else 0)
            if not _handle:
                raise MoeError(-8, lib().moe_cache_last_error().decode())
        self._h = _handle
        nl, ne, st, bb = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int64()
        self._check(lib().moe_store_info(self._h, ctypes.byref(nl), ctypes.byref(ne), ctypes.byref(st),
                                         ctypes.byref(bb)))
        self.n_layers, self.n_experts, self.stride, self.blob_bytes = nl.value, ne.value, st.value, bb.value

    @classmethod
    def create(cls, path: str, n_layers: int, n_experts: int, stride: int, blob_bytes: int) -> "ExpertStore":
        h = lib().moe_store_create(os.fsencode(path), n_layers, n_experts, stride, blob_bytes)
        if not h:
            raise MoeError(-8, lib().moe_cache_last_error().decode())
        return cls(path, _handle=h)

    def _check(self, rc: int) -> None:
        if rc != 0:
            raise MoeError(rc, lib().moe_cache_last_error().decode())

    def _host_ptr(self, buf) -> int:
        if isinstance(buf, int):
            return buf
        assert buf.nbytes >= self.stride and buf.flags["C_CONTIGUOUS"]
        return buf.ctypes.data

    def read(self, layer: int, expert: int, dst) -> None:
        self._check(lib().moe_store_read(self._h, layer, expert, self._host_ptr(dst)))

    def write(self, layer: int, expert: int, src) -> None:
        self._check(lib().moe_store_write(self._h, layer, expert, self._host_ptr(src)))

    def close(self) -> None:
        if self._h:
            lib().moe_store_close(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class ExpertCache:
    """HBM slot pool caching expert blobs of a pinned host store (moe_cache_*).

    pool / host may be torch tensors or raw addresses; both None gives the
    policy-only planning mode (no device work).  ids and slot tables are numpy
    arrays on the host.  ExpertCache.from_store reads misses from an
    ExpertStore through pinned staging buffers instead.
    """

    def __init__(self, n_slots: int, stride: int, pool, host, n_layers: int, n_experts: int, _handle=None):
        self.n_experts = n_experts
        self._h = _handle or lib().moe_cache_create(n_slots, stride, _ptr(pool), _ptr(host), n_layers, n_experts)
        if not self._h:
            raise MoeError(-1, "moe_cache_create rejected its arguments")

    @classmethod
    def from_store(cls, n_slots: int, pool, store: "ExpertStore", staging, n_staging: int) -> "ExpertCache":
        h = lib().moe_cache_create_from_store(n_slots, _ptr(pool), store._h, _ptr(staging), n_staging)
        if not h:
            raise MoeError(-1, lib().moe_cache_last_error().decode())
        c = cls(n_slots, store.stride, None, None, store.n_layers, store.n_experts, _handle=h)
        c._store = store          # the store must outlive the cache
        return c

    def _check(self, rc: int) -> None:
        if rc != 0:
            raise MoeError(rc, lib().moe_cache_last_error().decode())

    def acquire(self, layer: int, ids_host, slot_table_host, copy_stream=None, ready=None) -> None:
        import numpy as np
        ids = np.ascontiguousarray(ids_host, dtype=np.int32).reshape(-1)
        assert slot_table_host.dtype == np.int64 and slot_table_host.size >= self.n_experts
        assert slot_table_host.flags["C_CONTIGUOUS"]
        self._check(lib().moe_cache_acquire(self._h, layer, ids.ctypes.data, ids.size, slot_table_host.ctypes.data,
                                            _stream_handle(copy_stream), _event_handle(ready)))

    def release(self, layer: int, compute_done=None) -> None:
        self._check(lib().moe_cache_release(self._h, layer, _event_handle(compute_done)))

    def stats(self) -> tuple[int, int, int]:
        h, m, e = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        lib().moe_cache_stats(self._h, ctypes.byref(h), ctypes.byref(m), ctypes.byref(e))
        return h.value, m.value, e.value

    def set_policy(self, keep_counts: bool) -> None:
        self._check(lib().moe_cache_set_policy(self._h, CACHE_KEEP_COUNTS if keep_counts else 0))

    def inject_fault(self, nth_copy: int) -> None:
        """The nth copy issued from now on fails (MOE_EHIP from acquire); -1 disarms."""
        self._check(lib().moe_cache_inject_fault(self._h, nth_copy))

    def slot_of(self, layer: int, expert: int) -> int:
        return lib().moe_cache_slot_of(self._h, layer, expert)

    def close(self) -> None:
        if self._h:
            lib().moe_cache_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
