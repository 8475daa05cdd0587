"""Plain CPU oracle for the dense bf16 contractions (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the GPU library
(``attention_scores_amd``) and never imports it; the GPU library never
imports this.

The arithmetic lives in ``oracle.c`` (plain C, fp64, ascending-k sums, built
with gcc -O2 and no fast-math); this module marshals numpy arrays into it and
holds the tolerance check.

What is computed (pages cited by title and section):
  * GEMM C = A.B, grid rows sharing A, grid columns sharing B -- lesson 07
    "Clusters, distributed shared memory & cluster launch control", section
    "TMA multicast -- one load, many CTAs".
  * Attention scores S_i = Q_i K^T, no scale and no softmax -- "Hopper TMA
    Multicast" deep-dive, Attention/GEMM reuse use-case, equation
    S_0 = Q_0 K^T, S_1 = Q_1 K^T.
  * Attention forward O = softmax(scale * Q K^T) V (textbook scaled dot
    product, no mask), the FlashAttention-class operator the score product
    belongs to -- same deep-dive, Attention/GEMM reuse use-case and the
    "Attention K/V" row of its comparison table.
  * Tile fan-out microbenchmark accounting (consumers x iterations x tile
    bytes) and per-consumer data checksum -- same deep-dive, sections
    "Microbenchmark source" and "run results".

Tolerance (stated for the GPU results against this oracle):
  |C_gpu - C_ref| <= 1e-3 * T + 1e-5 per element, T = sum_k |a_ik * b_kj|.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

RTOL = 1e-3
ATOL = 1e-5


def build() -> str:
    """Compile liboracle.so with gcc (plain C, -O2, no fast-math)."""
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-D_GNU_SOURCE", "-fPIC", "-shared", "-pthread",
           "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    i64, i32, u16p, dp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = ctypes.c_double
    lib.oracle_f64_to_bf16_rne.argtypes = [ctypes.c_double]
    lib.oracle_f64_to_bf16_rne.restype = ctypes.c_uint16
    lib.oracle_f64_to_bf16_rne_array.argtypes = [dp, u16p, i64]
    lib.oracle_f64_to_bf16_rne_array.restype = None
    lib.oracle_gemm.argtypes = [u16p, u16p, dp, dp, i64, i64, i64, i64] + [i64] * 6 + [i32]
    lib.oracle_gemm.restype = i32
    lib.oracle_gemm_points.argtypes = [u16p, u16p, ctypes.c_void_p, i64, dp, dp, i64] + [i64] * 6 + [i32]
    lib.oracle_gemm_points.restype = i32
    lib.oracle_sscore.argtypes = [u16p, u16p, dp, dp, i64, i64, i64, i64] + [i64] * 6 + [i32]
    lib.oracle_sscore.restype = i32
    lib.oracle_sscore_points.argtypes = [u16p, u16p, ctypes.c_void_p, i64, dp, dp, i64] + [i64] * 6 + [i32]
    lib.oracle_sscore_points.restype = i32
    lib.oracle_attention.argtypes = [u16p, u16p, u16p, ctypes.c_void_p, i64, dp, dp] + [i64] * 5 + [i64] * 9 + \
        [ctypes.c_double, i32, i64, i32]
    lib.oracle_attention.restype = i32
    lib.oracle_tilecast_bytes.argtypes = [i64, i64, i64]
    lib.oracle_tilecast_bytes.restype = ctypes.c_double
    lib.oracle_tilecast_group.argtypes = [i64, i64, i64, i32]
    lib.oracle_tilecast_group.restype = i64
    lib.oracle_tilecast_checksum.argtypes = [u16p, i64, i64, i64, i64, i64, i64, i64, i32, i64, i64,
                                             ctypes.POINTER(ctypes.c_uint32)]
    lib.oracle_tilecast_checksum.restype = ctypes.c_uint32
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _as_bits(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns as a uint16 array (no copy when already uint16)."""
    if x.dtype == np.uint16:
        return x
    if x.dtype == np.int16:
        return x.view(np.uint16)
    raise TypeError("oracle inputs are bf16 bit patterns (uint16), got %s" % x.dtype)


def _span_ok(buf: np.ndarray, dims, strides) -> None:
    """Every addressed element of a strided view must lie inside buf."""
    hi = sum((d - 1) * s for d, s in zip(dims, strides) if d > 0)
    lo = min(0, *[(d - 1) * s for d, s in zip(dims, strides)])
    if lo < 0 or hi >= buf.size:
        raise ValueError("strided view exceeds the buffer (%d elements)" % buf.size)


def bf16_to_f64(bits) -> float:
    return _load().oracle_bf16_to_f64(int(bits) & 0xFFFF)


def f64_to_bf16_rne(x: float) -> int:
    return int(_load().oracle_f64_to_bf16_rne(float(x)))


def f64_to_bf16_rne_array(x: np.ndarray) -> np.ndarray:
    """Element-wise round-to-nearest-even of doubles to bf16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_f64_to_bf16_rne_array(_ptr(x), _ptr(out), x.size)
    return out


def bf16_bits_to_f64_array(bits: np.ndarray) -> np.ndarray:
    """Vector decode of bf16 bit patterns (same rule as the C decoder)."""
    b = _as_bits(np.ascontiguousarray(bits))
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gemm(A: np.ndarray, B: np.ndarray, batch: int, M: int, N: int, K: int,
         sa: Tuple[int, int, int], sb: Tuple[int, int, int], want_T: bool = True,
         nthreads: int = 0):
    """C[b,i,j] = sum_k A[b,i,k] B[b,k,j] in fp64; returns (C, T) as [batch, M, N].

    ``sa``/``sb`` are (row, col, batch) element strides into the flat bf16
    bit arrays ``A``/``B``.
    """
    A = np.ascontiguousarray(_as_bits(A)).reshape(-1)
    B = np.ascontiguousarray(_as_bits(B)).reshape(-1)
    _span_ok(A, (batch, M, K), (sa[2], sa[0], sa[1]))
    _span_ok(B, (batch, K, N), (sb[2], sb[0], sb[1]))
    C = np.empty((batch, M, N), dtype=np.float64)
    T = np.empty((batch, M, N), dtype=np.float64) if want_T else None
    rc = _load().oracle_gemm(_ptr(A), _ptr(B), _ptr(C), _ptr(T) if want_T else None,
                             batch, M, N, K, sa[0], sa[1], sa[2], sb[0], sb[1], sb[2], nthreads)
    if rc != 0:
        raise RuntimeError("oracle_gemm failed")
    return C, T


def gemm_points(A: np.ndarray, B: np.ndarray, pts: np.ndarray, K: int,
                sa: Tuple[int, int, int], sb: Tuple[int, int, int],
                dims: Optional[Tuple[int, int, int]] = None, nthreads: int = 0):
    """C and T at the (b, i, j) rows of ``pts`` (shape [n, 3]); same arithmetic as gemm()."""
    A = np.ascontiguousarray(_as_bits(A)).reshape(-1)
    B = np.ascontiguousarray(_as_bits(B)).reshape(-1)
    pts = np.ascontiguousarray(pts, dtype=np.int64).reshape(-1, 3)
    if dims is not None:
        batch, M, N = dims
        _span_ok(A, (batch, M, K), (sa[2], sa[0], sa[1]))
        _span_ok(B, (batch, K, N), (sb[2], sb[0], sb[1]))
        if pts.size and ((pts < 0).any() or (pts[:, 0] >= batch).any() or (pts[:, 1] >= M).any()
                         or (pts[:, 2] >= N).any()):
            raise ValueError("sample point outside the output")
    n = pts.shape[0]
    C = np.empty(n, dtype=np.float64)
    T = np.empty(n, dtype=np.float64)
    rc = _load().oracle_gemm_points(_ptr(A), _ptr(B), _ptr(pts), n, _ptr(C), _ptr(T), K,
                                    sa[0], sa[1], sa[2], sb[0], sb[1], sb[2], nthreads)
    if rc != 0:
        raise RuntimeError("oracle_gemm_points failed")
    return C, T


def sscore(Q: np.ndarray, Kt: np.ndarray, batch: int, Lq: int, Lk: int, d: int,
           sq: Tuple[int, int, int], sk: Tuple[int, int, int], nthreads: int = 0):
    """S[b,i,j] = sum_d Q[b,i,d] K[b,j,d] (no scale, no softmax); returns (S, T)."""
    Q = np.ascontiguousarray(_as_bits(Q)).reshape(-1)
    Kt = np.ascontiguousarray(_as_bits(Kt)).reshape(-1)
    _span_ok(Q, (batch, Lq, d), (sq[2], sq[0], sq[1]))
    _span_ok(Kt, (batch, Lk, d), (sk[2], sk[0], sk[1]))
    S = np.empty((batch, Lq, Lk), dtype=np.float64)
    T = np.empty((batch, Lq, Lk), dtype=np.float64)
    rc = _load().oracle_sscore(_ptr(Q), _ptr(Kt), _ptr(S), _ptr(T), batch, Lq, Lk, d,
                               sq[0], sq[1], sq[2], sk[0], sk[1], sk[2], nthreads)
    if rc != 0:
        raise RuntimeError("oracle_sscore failed")
    return S, T


def sscore_points(Q: np.ndarray, Kt: np.ndarray, pts: np.ndarray, d: int,
                  sq: Tuple[int, int, int], sk: Tuple[int, int, int], nthreads: int = 0):
    Q = np.ascontiguousarray(_as_bits(Q)).reshape(-1)
    Kt = np.ascontiguousarray(_as_bits(Kt)).reshape(-1)
    pts = np.ascontiguousarray(pts, dtype=np.int64).reshape(-1, 3)
    n = pts.shape[0]
    S = np.empty(n, dtype=np.float64)
    T = np.empty(n, dtype=np.float64)
    rc = _load().oracle_sscore_points(_ptr(Q), _ptr(Kt), _ptr(pts), n, _ptr(S), _ptr(T), d,
                                      sq[0], sq[1], sq[2], sk[0], sk[1], sk[2], nthreads)
    if rc != 0:
        raise RuntimeError("oracle_sscore_points failed")
    return S, T


def attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, batch: int, Lq: int, Lk: int, d: int, dv: int,
              sq: Tuple[int, int, int], sk: Tuple[int, int, int], sv: Tuple[int, int, int], scale: float,
              rows: Optional[np.ndarray] = None, nthreads: int = 0, causal: bool = False, kv_group: int = 1):
    """O = softmax(scale * Q K^T) V per (b, i) row in fp64; returns (O, TO).

    causal: query i sees keys j <= i + (Lk - Lq) only (needs Lk >= Lq).
    kv_group: query slice b reads K and V slice b // kv_group (K and V hold
    batch // kv_group slices).

    Q [b,i,d], K [b,j,d], V [b,j,c] addressed by (row, col, batch) element
    strides.  ``rows``: optional [n, 2] array of (b, i) pairs; then O and TO
    are [n, dv], else [batch, Lq, dv].  TO = sum_j p_j |V_jc| / sum_j p_j.
    """
    Q = np.ascontiguousarray(_as_bits(Q)).reshape(-1)
    K = np.ascontiguousarray(_as_bits(K)).reshape(-1)
    V = np.ascontiguousarray(_as_bits(V)).reshape(-1)
    _span_ok(Q, (batch, Lq, d), (sq[2], sq[0], sq[1]))
    if kv_group <= 0 or batch % kv_group:
        raise ValueError("kv_group must divide batch")
    _span_ok(K, (batch // kv_group, Lk, d), (sk[2], sk[0], sk[1]))
    _span_ok(V, (batch // kv_group, Lk, dv), (sv[2], sv[0], sv[1]))
    if rows is not None:
        r = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 2)
        if r.size and (r[:, 0].min() < 0 or r[:, 0].max() >= batch or r[:, 1].min() < 0 or r[:, 1].max() >= Lq):
            raise ValueError("row pair out of range")
        n = r.shape[0]
        shape = (n, dv)
    else:
        r = None
        n = 0
        shape = (batch, Lq, dv)
    O = np.empty(shape, dtype=np.float64)
    TO = np.empty(shape, dtype=np.float64)
    rc = _load().oracle_attention(_ptr(Q), _ptr(K), _ptr(V), _ptr(r) if r is not None else None, n,
                                  _ptr(O), _ptr(TO), batch, Lq, Lk, d, dv, sq[0], sq[1], sq[2],
                                  sk[0], sk[1], sk[2], sv[0], sv[1], sv[2], float(scale), int(bool(causal)),
                                  int(kv_group), nthreads)
    if rc != 0:
        raise RuntimeError("oracle_attention failed")
    return O, TO


# Attention tolerance.  A fused kernel rounds the probabilities p_j to bf16
# (unit roundoff 2^-8) before the p.V product; that alone moves O by at most
# 2^-8 * TO.  Score, exponential and fp32 accumulation errors are orders of
# magnitude smaller at these sizes.  The bound allows twice the rounding term.
ATTN_RTOL = 2.0 ** -7
ATTN_ATOL = 1e-6


def check_attention(out: np.ndarray, O_ref: np.ndarray, TO: np.ndarray, out_bf16: bool = False):
    """(n_fail, max_util) for |O_gpu - O_ref| <= 2^-7 * TO + 1e-6 (+ 2^-8 |O_ref|
    for a bf16 output, its own rounding)."""
    extra = 2.0 ** -8 * np.abs(O_ref) if out_bf16 else 0.0
    out = np.asarray(out, dtype=np.float64)
    bound = ATTN_RTOL * TO + ATTN_ATOL + extra
    diff = np.abs(out - O_ref)
    bad = ~np.isfinite(out) | ~(diff <= bound)
    util = np.where(np.isfinite(diff), diff / bound, np.inf)
    return int(bad.sum()), float(util.max()) if util.size else 0.0


def tilecast_bytes(consumers: int, iters: int, tile_bytes: int) -> float:
    return _load().oracle_tilecast_bytes(consumers, iters, tile_bytes)


def tilecast_group(w: int, consumers: int, group: int, grouped: bool) -> int:
    return int(_load().oracle_tilecast_group(w, consumers, group, int(bool(grouped))))


def tilecast_checksum(buf: np.ndarray, rows: int, cols: int, tile_m: int, tile_n: int, w: int,
                      consumers: int, group: int, grouped: bool, iters: int, stride: int):
    """(sum over all loaded tiles, sum over the last tile), both modulo 2^32."""
    b = np.ascontiguousarray(_as_bits(buf)).reshape(-1)
    if b.size < rows * cols:
        raise ValueError("buffer smaller than rows*cols")
    last = ctypes.c_uint32(0)
    tot = _load().oracle_tilecast_checksum(_ptr(b), rows, cols, tile_m, tile_n, w, consumers, group,
                                           int(bool(grouped)), iters, stride, ctypes.byref(last))
    return int(tot), int(last.value)


def tolerance(T: np.ndarray) -> np.ndarray:
    """Per-element bound 1e-3*T + 1e-5."""
    return RTOL * T + ATOL


def check(out: np.ndarray, C_ref: np.ndarray, T: np.ndarray, extra: Optional[np.ndarray] = None):
    """Compare a decoded GPU result with the oracle.

    Returns (n_fail, max_util) where util = |out - ref| / bound; NaN or Inf
    in ``out`` fails.  ``extra`` adds a per-element allowance (used only
    where a bf16 output's own rounding is documented to exceed the stated
    bound on same-sign data).
    """
    out = np.asarray(out, dtype=np.float64)
    bound = tolerance(T)
    if extra is not None:
        bound = bound + extra
    diff = np.abs(out - C_ref)
    bad = ~np.isfinite(out) | ~(diff <= bound)
    util = np.where(np.isfinite(diff), diff / bound, np.inf)
    return int(bad.sum()), float(util.max()) if util.size else 0.0
