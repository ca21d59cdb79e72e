"""ctypes binding of libmoe (include/moe.h): argument marshalling only.

Every entry point takes torch tensors (or raw device addresses) and passes
their device pointers and sizes to the C ABI; all arithmetic runs in the HIP
kernels of libmoe.so.  The library must have been built in-tree
(``python -m grouped_expert_ffn_router_amd.build``); importing a missing or
stale library raises instead of falling back to anything else.
"""

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")
# built from the same sources with -DMOE_DEBUG (invariant flags, see use_debug)
LIB_DEBUG_PATH = os.path.join(PKG, "libmoe_debug.so")

MOE_OK, MOE_EINVAL, MOE_EALIGN, MOE_EDTYPE, MOE_ECAP, MOE_EHIP = 0, -1, -2, -3, -4, -5
MOE_ACT_BF16, MOE_ACT_F32 = 0, 1
MOE_MAX_RANKS, MOE_MAX_LOCAL = 1024, 64

ENTRY_POINTS = ["moe_capacity", "moe_workspace_size", "moe_route", "moe_pack_pools", "moe_pack_pools_noalloc",
                "moe_pack_ragged",
                "moe_recv_rank", "moe_recv_waves",
                "moe_expert_gemm", "moe_shared_experts", "moe_combine", "moe_drop_stats", "moe_last_error", "moe_timing_enable",
                "moe_timing_read"]


class MoeError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libmoe error {code}: {msg}")
        self.code = code


class Dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "tokens", "d_model", "latent", "n_experts", "top_k", "n_ranks", "waves",
        "expert_hidden", "shared_experts", "shared_hidden", "my_rank", "act_dtype",
        "send_num", "send_den", "recv_num", "recv_den", "live_waves", "wave_rows")]


class DropReport(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "send_assignments", "send_kept", "send_dropped", "recv_arrivals", "recv_kept",
        "recv_dropped", "recv_bad_ids")] + [
        ("n_ranks", ctypes.c_int32), ("local_experts", ctypes.c_int32),
        ("send_demand", ctypes.c_int32 * MOE_MAX_RANKS), ("send_count", ctypes.c_int32 * MOE_MAX_RANKS),
        ("expert_arrivals", ctypes.c_int32 * MOE_MAX_LOCAL), ("expert_kept", ctypes.c_int32 * MOE_MAX_LOCAL)]

    def as_dict(self):
        R, X = self.n_ranks, self.local_experts
        return dict(send_assignments=self.send_assignments, send_kept=self.send_kept,
                    send_dropped=self.send_dropped, recv_arrivals=self.recv_arrivals,
                    recv_kept=self.recv_kept, recv_dropped=self.recv_dropped,
                    recv_bad_ids=self.recv_bad_ids,
                    send_demand=list(self.send_demand[:R]), send_count=list(self.send_count[:R]),
                    expert_arrivals=list(self.expert_arrivals[:X]), expert_kept=list(self.expert_kept[:X]))


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int32), ("total_ms", ctypes.c_double)]


_lib = None
_loaded = {}
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64


def lib():
    """The library the calls below go to: libmoe.so unless use_debug() selected
    its debug build (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


class use_debug:
    """Context manager: calls made inside go to libmoe_debug.so, whose kernels
    record invariant violations (a slot_of entry outside the return pools, a
    rank inconsistent with its count) in the workspace; moe_drop_stats then
    returns MOE_ECAP.  Results are otherwise those of libmoe.so."""

    def __enter__(self):
        global _lib
        self._prev = lib()
        _lib = _load(LIB_DEBUG_PATH)
        return _lib

    def __exit__(self, *exc):
        global _lib
        _lib = self._prev
        return False


def _load(path):
    if path in _loaded:
        return _loaded[path]
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m grouped_expert_ffn_router_amd.build` (no fallback exists)")
    L = ctypes.CDLL(path)
    DP = ctypes.POINTER(Dims)
    L.moe_capacity.argtypes = [DP, ctypes.POINTER(_I64), ctypes.POINTER(_I64), ctypes.POINTER(_I64)]
    L.moe_workspace_size.argtypes = [DP, ctypes.POINTER(ctypes.c_size_t)]
    L.moe_route.argtypes = [DP, _P, _P, _P, _P, _I32, _P, _P, _P, _P, _P, _P]
    L.moe_pack_pools.argtypes = [DP, _P, _P, _P, _I64, _P, _P, _P, _P]
    L.moe_pack_pools_noalloc.argtypes = [DP, _P, _P, _P, _I64, _P, _P, _P]
    L.moe_pack_ragged.argtypes = [DP, _P, _P, _P, _P, _P, _P, _P, _P]
    L.moe_recv_rank.argtypes = [DP, _P, _I64, _P, _P]
    L.moe_recv_waves.argtypes = [DP, _P, _I64, _I32, _P, _P, _P, _P, _P]
    L.moe_expert_gemm.argtypes = [DP, _I32, _P, _P, _I64, _P, _P, _P, _P, _P, _I64, _P, _P]
    L.moe_shared_experts.argtypes = [DP, _P, _P, _P, _P]
    L.moe_combine.argtypes = [DP, _P, _I64, _P, _P, _P, _P, _P, _P, _P]
    L.moe_drop_stats.argtypes = [DP, _P, ctypes.POINTER(DropReport), _P]
    L.moe_last_error.argtypes = []
    L.moe_last_error.restype = ctypes.c_char_p
    L.moe_timing_enable.argtypes = [_I32]
    L.moe_timing_read.argtypes = [ctypes.POINTER(KernelTime), _I32, ctypes.POINTER(_I32)]
    for n in ENTRY_POINTS:
        if n != "moe_last_error":
            getattr(L, n).restype = ctypes.c_int
    _loaded[path] = L
    return L


def _check(rc):
    if rc != MOE_OK:
        raise MoeError(rc, lib().moe_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_dims(shape, my_rank=0, tokens=None, live_waves=0, wave_rows=0):
    """moe_dims from a workload.configs.Shape-like object."""
    return Dims(live_waves=live_waves, wave_rows=wave_rows, tokens=shape.tokens if tokens is None else tokens,
                d_model=shape.d_model,
                latent=shape.latent, n_experts=shape.n_experts, top_k=shape.top_k,
                n_ranks=shape.n_ranks, waves=shape.waves, expert_hidden=shape.expert_hidden,
                shared_experts=shape.shared_experts, shared_hidden=shape.shared_hidden,
                my_rank=my_rank, act_dtype=MOE_ACT_BF16 if shape.act == "bf16" else MOE_ACT_F32,
                send_num=shape.send_num, send_den=shape.send_den, recv_num=shape.recv_num,
                recv_den=shape.recv_den)


def capacity(dims):
    s, r, p = _I64(), _I64(), _I64()
    _check(lib().moe_capacity(ctypes.byref(dims), ctypes.byref(s), ctypes.byref(r), ctypes.byref(p)))
    return s.value, r.value, p.value


def workspace_size(dims):
    b = ctypes.c_size_t()
    _check(lib().moe_workspace_size(ctypes.byref(dims), ctypes.byref(b)))
    return b.value


def route(dims, x, w_router, w_down, bias, bias_row_tokens, logits, z, topk_idx, topk_w, ws, stream=None):
    _check(lib().moe_route(ctypes.byref(dims), _ptr(x), _ptr(w_router), _ptr(w_down), _ptr(bias),
                           int(bias_row_tokens), _ptr(logits), _ptr(z), _ptr(topk_idx), _ptr(topk_w),
                           _ptr(ws), _stream(stream)))


def pack_pools(dims, z, topk_idx, send_pools, dst_stride_bytes, slot_of, send_count, ws, stream=None):
    _check(lib().moe_pack_pools(ctypes.byref(dims), _ptr(z), _ptr(topk_idx), _ptr(send_pools),
                                int(dst_stride_bytes), _ptr(slot_of), _ptr(send_count), _ptr(ws),
                                _stream(stream)))


def pack_pools_noalloc(dims, z, topk_idx, send_pools, dst_stride_bytes, slot_of, send_count, stream=None):
    _check(lib().moe_pack_pools_noalloc(ctypes.byref(dims), _ptr(z), _ptr(topk_idx), _ptr(send_pools),
                                        int(dst_stride_bytes), _ptr(slot_of), _ptr(send_count), _stream(stream)))


def pack_ragged(dims, z, topk_idx, send_rows, send_off, slot_of, send_count, ws, stream=None):
    _check(lib().moe_pack_ragged(ctypes.byref(dims), _ptr(z), _ptr(topk_idx), _ptr(send_rows), _ptr(send_off),
                                 _ptr(slot_of), _ptr(send_count), _ptr(ws), _stream(stream)))


def recv_rank(dims, recv_pools, src_stride_bytes, ws, stream=None):
    _check(lib().moe_recv_rank(ctypes.byref(dims), _ptr(recv_pools), int(src_stride_bytes), _ptr(ws), _stream(stream)))


def recv_waves(dims, recv_pools, src_stride_bytes, wave, wave_buf, row_src, wave_count, ws, stream=None):
    _check(lib().moe_recv_waves(ctypes.byref(dims), _ptr(recv_pools), int(src_stride_bytes), int(wave),
                                _ptr(wave_buf), _ptr(row_src), _ptr(wave_count), _ptr(ws), _stream(stream)))


def expert_gemm(dims, wave, wave_buf, recv_pools, src_stride_bytes, row_src, wave_count, w13, w2,
                ret_pools, ret_src_stride_bytes, ws, stream=None):
    _check(lib().moe_expert_gemm(ctypes.byref(dims), int(wave), _ptr(wave_buf), _ptr(recv_pools),
                                 int(src_stride_bytes), _ptr(row_src), _ptr(wave_count), _ptr(w13),
                                 _ptr(w2), _ptr(ret_pools), int(ret_src_stride_bytes), _ptr(ws),
                                 _stream(stream)))


def shared_experts(dims, x, ws13, ws, stream=None):
    _check(lib().moe_shared_experts(ctypes.byref(dims), _ptr(x), _ptr(ws13), _ptr(ws), _stream(stream)))


def combine(dims, ret_pools, ret_dst_stride_bytes, slot_of, topk_w, w_up, ws2, out, ws, stream=None):
    _check(lib().moe_combine(ctypes.byref(dims), _ptr(ret_pools), int(ret_dst_stride_bytes),
                             _ptr(slot_of), _ptr(topk_w), _ptr(w_up), _ptr(ws2), _ptr(out), _ptr(ws),
                             _stream(stream)))


def drop_stats(dims, ws, stream=None, raise_on_bad_ids=True):
    rep = DropReport()
    rc = lib().moe_drop_stats(ctypes.byref(dims), _ptr(ws), ctypes.byref(rep), _stream(stream))
    if rc == MOE_ECAP and not raise_on_bad_ids:
        return rep
    _check(rc)
    return rep


def last_error():
    return lib().moe_last_error().decode()


def timing_enable(on=True):
    """Record every library kernel launch with HIP events on its own stream."""
    _check(lib().moe_timing_enable(1 if on else 0))


def timing_read(max_entries=64):
    """{label: (launches, total_ms)} since the last read (waits for the events)."""
    buf = (KernelTime * max_entries)()
    n = _I32()
    _check(lib().moe_timing_read(buf, max_entries, ctypes.byref(n)))
    return {buf[i].name.decode(): (buf[i].launches, buf[i].total_ms) for i in range(min(n.value, max_entries))}
