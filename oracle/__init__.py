"""CPU oracle for the Ulysses 4D relayout: ctypes wrapper over liboracle.so.

TEST INFRASTRUCTURE ONLY.  The product path (the HIP library and its
Python binding) never imports this package; only the tests, the smoke check
and the benchmark's CPU-baseline leg do.  The C source, oracle.c, states
which passage of the pages each function follows.

Arrays are numpy arrays on the host, contiguous, d innermost.  bfloat16
data travels as uint16 bit patterns.  Every function is pinned by the
tests in tests/test_oracle_pins.py against values that do not come from the
oracle itself.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB points the wrapper at another build of oracle.c; the mutation
# test uses it to check that the pins catch planted mistakes.
_LIB_PATH = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        if "ORACLE_LIB" in os.environ:
            raise ImportError(f"ORACLE_LIB={_LIB_PATH} does not exist")
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_shape.argtypes = [ctypes.c_int, ctypes.c_int, _i64, _i64, _p, _p,
                                 ctypes.c_int, ctypes.c_int, _p]
    lib.oracle_shape.restype = ctypes.c_int
    lib.oracle_window_bytes.argtypes = [ctypes.c_int, ctypes.c_int, _i64, _i64, _p, _p]
    lib.oracle_window_bytes.restype = _i64
    lib.oracle_a2a_4d.argtypes = [ctypes.c_int, ctypes.c_int, _i64, _i64, _i64, _p, _p,
                                  _p, _p]
    lib.oracle_a2a_4d.restype = ctypes.c_int
    lib.oracle_a2a_4d_threads.argtypes = [ctypes.c_int, ctypes.c_int, _i64, _i64, _i64, _p, _p,
                                          _p, _p, ctypes.c_int]
    lib.oracle_a2a_4d_threads.restype = ctypes.c_int
    lib.oracle_a2a_4d_sample.argtypes = [ctypes.c_int, ctypes.c_int, _i64, _i64, _i64,
                                         _p, _p, _p, _i64, _p, _p]
    lib.oracle_a2a_4d_sample.restype = ctypes.c_int
    lib.oracle_f32_to_bf16.argtypes = [_p, _p, _i64]
    lib.oracle_f32_to_bf16.restype = None
    lib.oracle_bf16_to_f32.argtypes = [_p, _p, _i64]
    lib.oracle_bf16_to_f32.restype = None
    lib.oracle_rope_table.argtypes = [ctypes.c_double, _i64, _i64, _p, _p]
    lib.oracle_rope_table.restype = ctypes.c_int
    lib.oracle_qknorm_rope_mode0.argtypes = [ctypes.c_int, _i64, _i64, _p, _p, _p, _p,
                                             _p, ctypes.c_float, _p, _p]
    lib.oracle_qknorm_rope_mode0.restype = ctypes.c_int
    lib.oracle_qknorm_rope_mode0_threads.argtypes = [ctypes.c_int, _i64, _i64, _p, _p, _p, _p,
                                                     _p, ctypes.c_float, _p, _p, ctypes.c_int]
    lib.oracle_qknorm_rope_mode0_threads.restype = ctypes.c_int
    lib.oracle_qknorm_rope_mode0_sample.argtypes = [ctypes.c_int, _i64, _i64, _p, _p,
                                                    _p, _p, ctypes.c_float, _p, _p,
                                                    _i64, _p, _p]
    lib.oracle_qknorm_rope_mode0_sample.restype = ctypes.c_int
    lib.oracle_row_sum_of_squares.argtypes = [_i64, _p, _p]
    lib.oracle_row_sum_of_squares.restype = ctypes.c_int
    _lib = lib
    return lib


def _splits(seq_splits, head_splits):
    s = np.ascontiguousarray(np.asarray(seq_splits, dtype=np.int64))
    h = np.ascontiguousarray(np.asarray(head_splits, dtype=np.int64))
    if s.shape != h.shape or s.ndim != 1:
        raise ValueError("seq_splits and head_splits must be 1-D of equal length")
    return s, h


def _ptrs(arrays):
    for a in arrays:
        if not a.flags.c_contiguous:
            raise ValueError("oracle arrays must be C-contiguous")
    return (ctypes.c_void_p * len(arrays))(*[a.ctypes.data for a in arrays])


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments")


def shape(mode, b, d, seq_splits, head_splits, rank, is_dst):
    """Shard shape of `rank` for the input (is_dst False) or output of `mode`."""
    s, h = _splits(seq_splits, head_splits)
    out = np.zeros(4, dtype=np.int64)
    _check(_load().oracle_shape(mode, len(s), b, d, s.ctypes.data, h.ctypes.data,
                                rank, int(bool(is_dst)), out.ctypes.data), "shape")
    return tuple(int(v) for v in out)


def window_bytes(mode, d, esz, seq_splits, head_splits):
    """Per-rank, per-batch-plane window bytes of the plane-at-a-time exchange."""
    s, h = _splits(seq_splits, head_splits)
    v = _load().oracle_window_bytes(mode, len(s), d, esz, s.ctypes.data, h.ctypes.data)
    if v < 0:
        raise ValueError("oracle window_bytes: invalid arguments")
    return int(v)


def a2a_4d(mode, b, d, seq_splits, head_splits, srcs, threads=1):
    """Full relayout of the W source shards; returns the W destination shards.
    threads > 1 hands whole destination rows to that many threads (the same
    loops; identical results)."""
    s, h = _splits(seq_splits, head_splits)
    world = len(s)
    if len(srcs) != world:
        raise ValueError("need one source shard per rank")
    dtype = srcs[0].dtype
    for r, a in enumerate(srcs):
        want = shape(mode, b, d, s, h, r, False)
        if tuple(a.shape) != want or a.dtype != dtype:
            raise ValueError(f"source {r}: shape {a.shape} {a.dtype}, want {want} {dtype}")
    dsts = [np.empty(shape(mode, b, d, s, h, r, True), dtype=dtype) for r in range(world)]
    if threads > 1:
        _check(_load().oracle_a2a_4d_threads(mode, world, b, d, dtype.itemsize, s.ctypes.data,
                                             h.ctypes.data, _ptrs(srcs), _ptrs(dsts),
                                             int(threads)), "a2a_4d")
    else:
        _check(_load().oracle_a2a_4d(mode, world, b, d, dtype.itemsize, s.ctypes.data,
                                     h.ctypes.data, _ptrs(srcs), _ptrs(dsts)), "a2a_4d")
    return dsts


def a2a_4d_sample(mode, b, d, seq_splits, head_splits, srcs, coords):
    """Destination elements at coords (n x 5: rank, bi, s, h, e)."""
    s, h = _splits(seq_splits, head_splits)
    coords = np.ascontiguousarray(np.asarray(coords, dtype=np.int64).reshape(-1, 5))
    dtype = srcs[0].dtype
    out = np.empty(coords.shape[0], dtype=dtype)
    _check(_load().oracle_a2a_4d_sample(mode, len(s), b, d, dtype.itemsize,
                                        s.ctypes.data, h.ctypes.data, _ptrs(srcs),
                                        coords.shape[0], coords.ctypes.data,
                                        out.ctypes.data), "a2a_4d_sample")
    return out


def f32_to_bf16(x):
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_f32_to_bf16(x.ctypes.data, out.ctypes.data, x.size)
    return out


def bf16_to_f32(x):
    x = np.ascontiguousarray(np.asarray(x, dtype=np.uint16))
    out = np.empty(x.shape, dtype=np.float32)
    _load().oracle_bf16_to_f32(x.ctypes.data, out.ctypes.data, x.size)
    return out


def rope_table(theta, s_global, d):
    """(cos, sin), each float32 [s_global, d/2]."""
    c = np.empty((s_global, d // 2), dtype=np.float32)
    sn = np.empty((s_global, d // 2), dtype=np.float32)
    _check(_load().oracle_rope_table(float(theta), s_global, d, c.ctypes.data,
                                     sn.ctypes.data), "rope_table")
    return c, sn


def qknorm_rope_mode0(b, d, seq_splits, head_splits, srcs, gamma, eps, cos_tab, sin_tab,
                      threads=1):
    """Fused mode 0 of one bf16 tensor (uint16 arrays); returns W shards.
    threads > 1 hands whole destination rows to that many threads."""
    s, h = _splits(seq_splits, head_splits)
    world = len(s)
    for r, a in enumerate(srcs):
        if a.dtype != np.uint16 or tuple(a.shape) != shape(0, b, d, s, h, r, False):
            raise ValueError(f"source {r}: bad shape or dtype")
    gamma = np.ascontiguousarray(np.asarray(gamma, dtype=np.float32))
    cos_tab = np.ascontiguousarray(cos_tab, dtype=np.float32)
    sin_tab = np.ascontiguousarray(sin_tab, dtype=np.float32)
    if gamma.shape != (d,) or cos_tab.shape != (int(s.sum()), d // 2) \
            or sin_tab.shape != cos_tab.shape:
        raise ValueError("gamma must be [d], tables [s_global, d/2]")
    dsts = [np.empty(shape(0, b, d, s, h, r, True), dtype=np.uint16) for r in range(world)]
    args = (world, b, d, s.ctypes.data, h.ctypes.data, _ptrs(srcs), _ptrs(dsts),
            gamma.ctypes.data, float(eps), cos_tab.ctypes.data, sin_tab.ctypes.data)
    if threads > 1:
        _check(_load().oracle_qknorm_rope_mode0_threads(*args, int(threads)),
               "qknorm_rope_mode0")
    else:
        _check(_load().oracle_qknorm_rope_mode0(*args), "qknorm_rope_mode0")
    return dsts


def qknorm_rope_mode0_sample(b, d, seq_splits, head_splits, srcs, gamma, eps,
                             cos_tab, sin_tab, rows):
    """Fused outputs of the destination rows in rows (n x 4: rank, bi, S, h)."""
    s, h = _splits(seq_splits, head_splits)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 4))
    gamma = np.ascontiguousarray(np.asarray(gamma, dtype=np.float32))
    cos_tab = np.ascontiguousarray(cos_tab, dtype=np.float32)
    sin_tab = np.ascontiguousarray(sin_tab, dtype=np.float32)
    out = np.empty((rows.shape[0], d), dtype=np.uint16)
    _check(_load().oracle_qknorm_rope_mode0_sample(
        len(s), b, d, s.ctypes.data, h.ctypes.data, _ptrs(srcs), gamma.ctypes.data,
        float(eps), cos_tab.ctypes.data, sin_tab.ctypes.data, rows.shape[0],
        rows.ctypes.data, out.ctypes.data), "qknorm_rope_mode0_sample")
    return out


def row_sum_of_squares(d, row_bits):
    """The fused row operation's fp32 sum of squares of one bf16 row (uint16
    bit patterns, d elements), in its fixed order."""
    row = np.ascontiguousarray(np.asarray(row_bits, dtype=np.uint16))
    if row.shape != (d,):
        raise ValueError("row must hold d bf16 values")
    out = np.zeros(1, dtype=np.float32)
    _check(_load().oracle_row_sum_of_squares(int(d), row.ctypes.data, out.ctypes.data),
           "row_sum_of_squares")
    return out[0]
