"""Python binding of libattn_scores.so (include/attn_scores.h) for MI355X / gfx950.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  torch supplies device memory and the current
stream; nothing here computes on the CPU, and there is no fallback path --
if the library has not been built, every call raises.

Low-level names mirror the C ABI (``gemm_create``, ``gemm_run``, ``gemm_run_no_alloc``,
``gemm_destroy``, ``gemm_plan_info``, ``gemm_plan_tile_of``, ``sscore_run``,
``tilecast_run``, ``as_status_str``, ``as_last_error``) and take raw device
pointers.  ``gemm``, ``sscore`` and ``tilecast`` are tensor conveniences that
read shapes, strides and dtypes from torch tensors.
"""
from __future__ import annotations

import collections
import ctypes
import os
import threading
from typing import Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn_scores.so")

AS_OK, AS_ERR_INVALID, AS_ERR_UNSUPPORTED, AS_ERR_HIP, AS_ERR_NOMEM = 0, 1, 2, 3, 4
AS_BF16, AS_F32 = 0, 1
AS_FLAG_NO_GROUPING = 0x1
AS_FLAG_TILE_128 = 0x2
AS_FLAG_TILE_256 = 0x4
AS_FLAG_TILE_64 = 0x400
AS_FLAG_ONE_TILE_PER_WORKGROUP = 0x8
AS_FLAG_NO_SPLIT_K = 0x10
AS_FLAG_NT_A = 0x20
AS_FLAG_NO_NT_A = 0x40
AS_FLAG_ROTATE_K = 0x80
AS_FLAG_NO_ROTATE_K = 0x100
AS_FLAG_NO_XCD_SPLIT = 0x200
AS_ATTN_CAUSAL = 0x1
AS_ATTN_QUERIES_256 = 0x2
AS_ATTN_QUERIES_128 = 0x4
AS_ATTN_SCHED_STATIC = 0x8
AS_ATTN_SCHED_QUEUE = 0x10

EXPORTED = ("gemm_create", "gemm_run", "gemm_run_no_alloc", "gemm_destroy", "gemm_plan_info", "gemm_plan_tile_of", "gemm_plan_split_k",
            "sscore_run", "attn_fwd_run", "attn_fwd_run_gqa", "attn_fwd_plan_info", "tilecast_run", "as_status_str",
            "as_last_error")


class Strides(ctypes.Structure):
    """as_strides: element strides (row, col, batch)."""
    _fields_ = [("row", ctypes.c_int64), ("col", ctypes.c_int64), ("batch", ctypes.c_int64)]


class AsError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (_status_name(status), message))
        self.status = status


def _status_name(status: int) -> str:
    return {0: "AS_OK", 1: "AS_ERR_INVALID", 2: "AS_ERR_UNSUPPORTED", 3: "AS_ERR_HIP",
            4: "AS_ERR_NOMEM"}.get(status, "AS_UNKNOWN_STATUS")


_lib = None
_lib_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """The loaded C-ABI library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libattn_scores.so is not built (run __graft_entry__.build() or "
                               "python attention_scores_amd/_build.py)")
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, u32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_void_p
        L.gemm_create.argtypes = [ctypes.POINTER(vp), i64, i64, i64, i64, Strides, Strides, Strides,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int, u32]
        L.gemm_create.restype = ctypes.c_int
        L.gemm_run.argtypes = [vp, vp, vp, vp, vp]
        L.gemm_run.restype = ctypes.c_int
        L.gemm_run_no_alloc.argtypes = [vp, vp, vp, vp, vp]
        L.gemm_run_no_alloc.restype = ctypes.c_int
        L.gemm_destroy.argtypes = [vp]
        L.gemm_destroy.restype = ctypes.c_int
        L.gemm_plan_info.argtypes = [vp, ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(i32),
                                     ctypes.POINTER(i64), ctypes.POINTER(i64)]
        L.gemm_plan_info.restype = ctypes.c_int
        L.gemm_plan_tile_of.argtypes = [vp, i64, ctypes.POINTER(i64), ctypes.POINTER(i64), ctypes.POINTER(i64)]
        L.gemm_plan_tile_of.restype = ctypes.c_int
        L.gemm_plan_split_k.argtypes = [vp, ctypes.POINTER(i32), ctypes.POINTER(i64)]
        L.gemm_plan_split_k.restype = ctypes.c_int
        L.sscore_run.argtypes = [vp, vp, vp, i64, i64, i64, i64, Strides, Strides, Strides,
                                 ctypes.c_int, ctypes.c_int, vp]
        L.sscore_run.restype = ctypes.c_int
        L.attn_fwd_run.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, Strides, Strides, Strides, Strides,
                                   ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_uint32, vp]
        L.attn_fwd_run.restype = ctypes.c_int
        L.attn_fwd_run_gqa.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, Strides, Strides, Strides,
                                       Strides, ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_uint32, vp]
        L.attn_fwd_run_gqa.restype = ctypes.c_int
        L.attn_fwd_plan_info.argtypes = [i64, i64, u32, ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(i64)]
        L.attn_fwd_plan_info.restype = ctypes.c_int
        L.tilecast_run.argtypes = [vp, i64, i64, i32, i32, i32, i32, i32, i64, i64, i64, vp, vp]
        L.tilecast_run.restype = ctypes.c_int
        L.as_status_str.argtypes = [ctypes.c_int]
        L.as_status_str.restype = ctypes.c_char_p
        L.as_last_error.argtypes = []
        L.as_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != AS_OK:
        raise AsError(status, as_last_error())


def as_status_str(status: int) -> str:
    return lib().as_status_str(status).decode()


def as_last_error() -> str:
    return lib().as_last_error().decode()


# ------------------------------------------------------------- raw C ABI --

def gemm_create(M: int, N: int, K: int, batch: int, a: Tuple[int, int, int], b: Tuple[int, int, int],
                c: Tuple[int, int, int], a_t: int = AS_BF16, b_t: int = AS_BF16, c_t: int = AS_F32,
                flags: int = 0) -> int:
    h = ctypes.c_void_p()
    _check(lib().gemm_create(ctypes.byref(h), M, N, K, batch, Strides(*a), Strides(*b), Strides(*c),
                             a_t, b_t, c_t, flags))
    return h.value


def gemm_run(plan: int, A: int, B: int, C: int, stream: int = 0) -> None:
    _check(lib().gemm_run(plan, A, B, C, stream))


def gemm_run_no_alloc(plan: int, A: int, B: int, C: int, stream: int = 0) -> None:
    """gemm_run that allocates nothing: a split plan uses the library's static
    per-GPU scratch array (calls overlapping on one GPU race; see the header)."""
    _check(lib().gemm_run_no_alloc(plan, A, B, C, stream))


def gemm_destroy(plan: int) -> None:
    _check(lib().gemm_destroy(plan))


def gemm_plan_info(plan: int):
    """(tile_m, tile_n, tile_k, tiles, workgroups) the plan chose."""
    tm, tn, tk = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    nt, wg = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().gemm_plan_info(plan, ctypes.byref(tm), ctypes.byref(tn), ctypes.byref(tk), ctypes.byref(nt),
                                ctypes.byref(wg)))
    return tm.value, tn.value, tk.value, nt.value, wg.value


def gemm_plan_split_k(plan: int):
    """(K chunks, workspace bytes) of a plan; (1, 0) when it does not split K."""
    sp, wb = ctypes.c_int32(), ctypes.c_int64()
    _check(lib().gemm_plan_split_k(plan, ctypes.byref(sp), ctypes.byref(wb)))
    return sp.value, wb.value


def gemm_plan_tile_of(plan: int, slot: int):
    """(batch, tile row, tile column) computed in execution slot `slot` (runs on XCD slot % 8)."""
    b, r, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(lib().gemm_plan_tile_of(plan, slot, ctypes.byref(b), ctypes.byref(r), ctypes.byref(c)))
    return b.value, r.value, c.value


def attn_fwd_run(Q: int, K: int, V: int, O: int, batch: int, Lq: int, Lk: int, d: int, dv: int,
                 q: Tuple[int, int, int], k: Tuple[int, int, int], v: Tuple[int, int, int],
                 o: Tuple[int, int, int], scale: float, qkv_t: int = AS_BF16, o_t: int = AS_BF16,
                 flags: int = 0, stream: int = 0) -> None:
    """O = softmax(scale Q K^T) V on device pointers (see attn_fwd_run in attn_scores.h)."""
    _check(lib().attn_fwd_run(Q, K, V, O, batch, Lq, Lk, d, dv, Strides(*q), Strides(*k), Strides(*v),
                              Strides(*o), float(scale), qkv_t, o_t, flags, stream))


def attn_fwd_run_gqa(Q: int, K: int, V: int, O: int, batch: int, kv_group: int, Lq: int, Lk: int, d: int, dv: int,
                     q: Tuple[int, int, int], k: Tuple[int, int, int], v: Tuple[int, int, int],
                     o: Tuple[int, int, int], scale: float, qkv_t: int = AS_BF16, o_t: int = AS_BF16,
                     flags: int = 0, stream: int = 0) -> None:
    """attn_fwd_run with query slice b reading K/V slice b // kv_group (see attn_scores.h)."""
    _check(lib().attn_fwd_run_gqa(Q, K, V, O, batch, kv_group, Lq, Lk, d, dv, Strides(*q), Strides(*k),
                                  Strides(*v), Strides(*o), float(scale), qkv_t, o_t, flags, stream))


def attn_fwd_plan_info(batch: int, Lq: int, flags: int = 0):
    """(queries per workgroup, keys per stage, workgroups) attn_fwd_run chooses."""
    qw, ks, wg = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
    _check(lib().attn_fwd_plan_info(batch, Lq, flags, ctypes.byref(qw), ctypes.byref(ks), ctypes.byref(wg)))
    return qw.value, ks.value, wg.value


def sscore_run(Q: int, K: int, S: int, batch: int, Lq: int, Lk: int, dim: int, q: Tuple[int, int, int],
               k: Tuple[int, int, int], s: Tuple[int, int, int], qk_t: int = AS_BF16, s_t: int = AS_F32,
               stream: int = 0) -> None:
    _check(lib().sscore_run(Q, K, S, batch, Lq, Lk, dim, Strides(*q), Strides(*k), Strides(*s), qk_t, s_t, stream))


def tilecast_run(buf: int, rows: int, cols: int, tile_m: int, tile_n: int, consumers: int, group: int,
                 grouped: bool, iters: int, warmup: int, stride: int, out_checksum: int, stream: int = 0) -> None:
    _check(lib().tilecast_run(buf, rows, cols, tile_m, tile_n, consumers, group, int(bool(grouped)), iters,
                              warmup, stride, out_checksum, stream))


# ---------------------------------------------------- torch conveniences --

def _torch():
    import torch
    return torch


def _dtype_code(dt) -> int:
    torch = _torch()
    if dt == torch.bfloat16:
        return AS_BF16
    if dt == torch.float32:
        return AS_F32
    raise AsError(AS_ERR_UNSUPPORTED, "dtype %s" % dt)


def _stream_handle(t) -> int:
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def _strides3(t):
    """(row, col, batch) element strides of a 2-D or 3-D tensor."""
    if t.dim() == 2:
        return (t.stride(0), t.stride(1), 0)
    if t.dim() == 3:
        return (t.stride(1), t.stride(2), t.stride(0))
    raise AsError(AS_ERR_INVALID, "expected a 2-D or 3-D tensor")


def _require_cuda(*ts):
    for t in ts:
        if not t.is_cuda:
            raise AsError(AS_ERR_INVALID, "tensors must be on the GPU")


_PLAN_CACHE_SIZE = 64
_plan_cache = collections.OrderedDict()
_plan_cache_lock = threading.Lock()
# Split plans evicted from the cache.  A HIP graph that recorded a run of a
# split plan replays into that plan's workspace, and nothing tells the cache
# whether one did, so an evicted split plan is kept (never destroyed) until
# the process ends.  Plans without a split hold no device memory and are
# destroyed on eviction.
_retired_split_plans = []


def plan_for(M, N, K, batch, sa, sb, sc, a_t, b_t, c_t, flags=0, stream=0) -> int:
    """Cached gemm_create for a shape/stride/dtype/flags/stream key: the last
    64 plans are kept; the least recently used is destroyed, or, if it splits
    K, set aside for the life of the process (with its workspace).  The stream
    is part of the key because a split plan's runs share its workspace: calls
    on different streams get their own plans."""
    key = (M, N, K, batch, tuple(sa), tuple(sb), tuple(sc), a_t, b_t, c_t, flags, stream)
    with _plan_cache_lock:
        p = _plan_cache.get(key)
        if p is not None:
            _plan_cache.move_to_end(key)
            return p
        p = gemm_create(M, N, K, batch, sa, sb, sc, a_t, b_t, c_t, flags)
        _plan_cache[key] = p
        while len(_plan_cache) > _PLAN_CACHE_SIZE:
            _, old = _plan_cache.popitem(last=False)
            if gemm_plan_split_k(old)[0] > 1:
                _retired_split_plans.append(old)
            else:
                gemm_destroy(old)
        return p


def gemm(A, B, out=None, out_dtype=None, flags: int = 0):
    """C = A @ B for bf16 A [M,K] / [b,M,K] and B [K,N] / [b,K,N] (any unit-stride orientation)."""
    torch = _torch()
    _require_cuda(A, B)
    batched = A.dim() == 3 or B.dim() == 3
    M, K = A.shape[-2], A.shape[-1]
    K2, N = B.shape[-2], B.shape[-1]
    if K != K2:
        raise AsError(AS_ERR_INVALID, "inner dimensions differ (%d vs %d)" % (K, K2))
    batch = max(A.shape[0] if A.dim() == 3 else 1, B.shape[0] if B.dim() == 3 else 1)
    for t in (A, B):
        if t.dim() == 3 and t.shape[0] not in (1, batch):
            raise AsError(AS_ERR_INVALID, "batch sizes differ")
    sa, sb = list(_strides3(A)), list(_strides3(B))
    if A.dim() == 3 and A.shape[0] == 1:
        sa[2] = 0
    if B.dim() == 3 and B.shape[0] == 1:
        sb[2] = 0
    if out is None:
        od = out_dtype if out_dtype is not None else torch.float32
        out = torch.empty((batch, M, N) if batched else (M, N), dtype=od, device=A.device)
    _require_cuda(out)
    sc = _strides3(out)
    stream = _stream_handle(A)
    plan = plan_for(M, N, K, batch, sa, sb, sc, _dtype_code(A.dtype), _dtype_code(B.dtype),
                    _dtype_code(out.dtype), flags, stream)
    gemm_run(plan, A.data_ptr(), B.data_ptr(), out.data_ptr(), stream)
    return out


def sscore(Q, K, out=None, out_dtype=None):
    """S = Q @ K^T per slice: Q [b,Lq,d], K [b,Lk,d] bf16 -> S [b,Lq,Lk] (no scale, no softmax)."""
    torch = _torch()
    _require_cuda(Q, K)
    if Q.dim() != 3 or K.dim() != 3:
        raise AsError(AS_ERR_INVALID, "Q and K must be [batch, L, d]")
    b, Lq, d = Q.shape
    if K.shape[0] != b or K.shape[2] != d:
        raise AsError(AS_ERR_INVALID, "Q and K shapes do not match")
    Lk = K.shape[1]
    if out is None:
        od = out_dtype if out_dtype is not None else torch.float32
        out = torch.empty((b, Lq, Lk), dtype=od, device=Q.device)
    _require_cuda(out)
    sscore_run(Q.data_ptr(), K.data_ptr(), out.data_ptr(), b, Lq, Lk, d, _strides3(Q), _strides3(K),
               _strides3(out), _dtype_code(Q.dtype), _dtype_code(out.dtype), _stream_handle(Q))
    return out


def attention(Q, K, V, scale=None, out=None, out_dtype=None, causal=False):
    """O = softmax(scale Q K^T) V per slice: Q [b,Lq,d], K [bk,Lk,d], V [bk,Lk,dv]
    bf16 -> O [b,Lq,dv] (default scale 1/sqrt(d), bf16 output).  bk may divide b
    (grouped key/value heads: query slice i reads K/V slice i // (b // bk)).
    causal: query i sees keys j <= i + Lk - Lq only."""
    torch = _torch()
    _require_cuda(Q, K, V)
    if Q.dim() != 3 or K.dim() != 3 or V.dim() != 3:
        raise AsError(AS_ERR_INVALID, "Q, K and V must be [batch, L, d]")
    b, Lq, d = Q.shape
    bk, Lk, dv = V.shape
    if K.shape[0] != bk or K.shape[2] != d or K.shape[1] != Lk or bk <= 0 or b % bk:
        raise AsError(AS_ERR_INVALID, "Q, K and V shapes do not match")
    if scale is None:
        scale = d ** -0.5
    if out is None:
        od = out_dtype if out_dtype is not None else torch.bfloat16
        out = torch.empty((b, Lq, dv), dtype=od, device=Q.device)
    _require_cuda(out)
    attn_fwd_run_gqa(Q.data_ptr(), K.data_ptr(), V.data_ptr(), out.data_ptr(), b, b // bk, Lq, Lk, d, dv,
                     _strides3(Q), _strides3(K), _strides3(V), _strides3(out), scale, _dtype_code(Q.dtype),
                     _dtype_code(out.dtype), AS_ATTN_CAUSAL if causal else 0, _stream_handle(Q))
    return out


def tilecast(buf, tile_m: int = 128, tile_n: int = 64, consumers: int = 256, group: int = 2,
             grouped: bool = True, iters: int = 5000, warmup: int = 0, stride: int = 0, out=None):
    """Run the tile fan-out microbenchmark over a 2-D bf16 CUDA tensor; returns the checksum tensor."""
    torch = _torch()
    _require_cuda(buf)
    if buf.dim() != 2 or buf.stride(1) != 1 or buf.stride(0) != buf.shape[1]:
        raise AsError(AS_ERR_INVALID, "buf must be a contiguous 2-D tensor")
    if out is None:
        out = torch.zeros(2 * consumers, dtype=torch.int32, device=buf.device)
    tilecast_run(buf.data_ptr(), buf.shape[0], buf.shape[1], tile_m, tile_n, consumers, group, grouped,
                 iters, warmup, stride, out.data_ptr(), _stream_handle(buf))
    return out
