"""ctypes binding of libulysses.so (include/ulysses.h), same names as the C ABI.

Argument marshalling only: every step of the relayout runs in the library's
HIP kernels.  Device buffers may be given as torch tensors (their
data_ptr() is passed) or as integer device addresses; streams as a
torch.cuda.Stream, an integer hipStream_t, or None for torch's current
stream (the null stream without torch).  A negative status raises
UlyssesError with the library's message.  The library must be built
(python -m sequence_attention_relayout_amd.build); there is no fallback.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libulysses.so")

ULYSSES_MAX_WORLD = 8
ULYSSES_MAX_TENSORS = 4
DTYPE_CODES = {"bf16": 0, "fp16": 1, "fp32": 2, "fp8_e4m3": 3, "fp8_e5m2": 4,
               "int8": 5, "uint8": 6}
STATUS_NAMES = {0: "ULYSSES_OK", -1: "ULYSSES_EINVAL", -2: "ULYSSES_EALIGN",
                -3: "ULYSSES_EDTYPE", -4: "ULYSSES_EWINDOW", -5: "ULYSSES_EOVERLAP",
                -6: "ULYSSES_EHIP"}

_i64 = ctypes.c_int64
_p = ctypes.c_void_p
_lib = None


class UlyssesError(RuntimeError):
    def __init__(self, code, message):
        self.code = code
        super().__init__(f"{STATUS_NAMES.get(code, code)}: {message}")


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run "
                          "`python -m sequence_attention_relayout_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.ulysses_plan_create.argtypes = [ctypes.POINTER(_p), ctypes.c_int, _i64, _i64, _p, _p,
                                        ctypes.c_int, _i64]
    lib.ulysses_plan_create.restype = ctypes.c_int
    lib.ulysses_plan_destroy.argtypes = [_p]
    lib.ulysses_plan_destroy.restype = None
    lib.ulysses_plan_shape.argtypes = [_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _p]
    lib.ulysses_plan_shape.restype = ctypes.c_int
    lib.ulysses_plan_window_bytes.argtypes = [_p, ctypes.c_int]
    lib.ulysses_plan_window_bytes.restype = _i64
    lib.ulysses_plan_bytes.argtypes = [_p, ctypes.c_int]
    lib.ulysses_plan_bytes.restype = _i64
    lib.ulysses_a2a_4d.argtypes = [_p, ctypes.c_int, _p, _p, _p]
    lib.ulysses_a2a_4d.restype = ctypes.c_int
    lib.ulysses_a2a_4d_multi.argtypes = [_p, ctypes.c_int, ctypes.c_int, _p, _p, _p]
    lib.ulysses_a2a_4d_multi.restype = ctypes.c_int
    lib.ulysses_a2a_4d_chunked.argtypes = [_p, ctypes.c_int, _p, _p, _p, _p]
    lib.ulysses_a2a_4d_chunked.restype = ctypes.c_int
    lib.ulysses_a2a_4d_chunked_static.argtypes = [_p, ctypes.c_int, _p, _p, _p]
    lib.ulysses_a2a_4d_chunked_static.restype = ctypes.c_int
    lib.ulysses_a2a_4d_qknorm_rope.argtypes = [_p, _p, _p, _p, _p, _p, _p, ctypes.c_float,
                                               _p, _p, _p]
    lib.ulysses_a2a_4d_qknorm_rope.restype = ctypes.c_int
    lib.ulysses_rope_table.argtypes = [ctypes.c_double, _i64, _i64, _p, _p]
    lib.ulysses_rope_table.restype = ctypes.c_int
    lib.ulysses_last_error.argtypes = []
    lib.ulysses_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def library():
    """The loaded ctypes.CDLL (loads it on first use)."""
    return _load()


def ulysses_last_error():
    return _load().ulysses_last_error().decode("utf-8", "replace")


def _check(rc):
    if rc < 0:
        raise UlyssesError(int(rc), ulysses_last_error())
    return rc


def _dtype_code(dtype):
    if isinstance(dtype, int):
        return dtype
    if isinstance(dtype, str):
        return DTYPE_CODES[dtype]
    name = str(dtype).replace("torch.", "")
    return {"bfloat16": 0, "float16": 1, "float32": 2, "float8_e4m3fn": 3,
            "float8_e5m2": 4, "int8": 5, "uint8": 6}[name]


ELEM_BYTES = {0: 2, 1: 2, 2: 4, 3: 1, 4: 1, 5: 1, 6: 1}


def _nm(what, index):
    return what if index is None else f"{what}[{index}]"


def _addr(x, need=None, what="buffer", index=None):
    """Device address of x.  A tensor must be contiguous and, when the call
    reads or writes `need` > 0 bytes through it, hold at least that many
    bytes on a HIP device: the library takes bare pointers and cannot check
    either.  Integer addresses are passed through unchecked."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        if hasattr(x, "is_contiguous") and not x.is_contiguous():
            raise ValueError(f"{_nm(what, index)}: device buffers must be contiguous")
        if need and hasattr(x, "nbytes"):
            if x.nbytes < need:
                raise ValueError(f"{_nm(what, index)}: holds {x.nbytes} bytes, the call uses {need}")
            if not getattr(x, "is_cuda", True):
                raise ValueError(f"{_nm(what, index)}: is on {x.device}, not on a HIP device")
        return x.data_ptr()
    raise TypeError(f"{_nm(what, index)}: expected a tensor or an integer address, got {type(x)}")


def _ptr_array(items, world, what, needs=None):
    items = list(items)
    if len(items) != world:
        raise ValueError(f"{what}: need {world} pointers, got {len(items)}")
    needs = needs if needs is not None else [None] * world
    return (_p * world)(*[_addr(v, n, what, i) for i, (v, n) in enumerate(zip(items, needs))])


def _stream(stream):
    if stream is None:
        try:
            import torch
            if torch.cuda.is_available():
                return torch.cuda.current_stream().cuda_stream
        except ImportError:
            pass
        return 0
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


class Plan:
    """Owns one ulysses_plan handle (freed with the object)."""

    def __init__(self, handle, world, b, d, seq_splits, head_splits, dtype, window_cap_bytes):
        self._handle = handle
        self.world, self.b, self.d = world, b, d
        self.seq_splits, self.head_splits = list(seq_splits), list(head_splits)
        self.dtype = dtype
        self.window_cap_bytes = window_cap_bytes
        self._bytes = {}

    @property
    def handle(self):
        if self._handle is None:
            raise ValueError("plan was destroyed")
        return self._handle

    def shard_bytes(self, mode, is_dst):
        """Bytes of each rank's shard: the input (is_dst False) or output of
        `mode`, as a list over ranks (cached)."""
        key = (int(mode), bool(is_dst))
        if key not in self._bytes:
            esz = ELEM_BYTES[self.dtype]
            self._bytes[key] = [int(np.prod(ulysses_plan_shape(self, mode, r, is_dst))) * esz
                                for r in range(self.world)]
        return self._bytes[key]

    def destroy(self):
        if self._handle is not None and _lib is not None:
            _lib.ulysses_plan_destroy(self._handle)
        self._handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def ulysses_plan_create(world, b, d, seq_splits, head_splits, dtype, window_cap_bytes=0):
    lib = _load()
    seq = np.ascontiguousarray(np.asarray(seq_splits, dtype=np.int64))
    head = np.ascontiguousarray(np.asarray(head_splits, dtype=np.int64))
    if seq.shape != (world,) or head.shape != (world,):
        raise ValueError("seq_splits and head_splits need `world` entries")
    h = _p()
    _check(lib.ulysses_plan_create(ctypes.byref(h), int(world), int(b), int(d), seq.ctypes.data,
                                   head.ctypes.data, _dtype_code(dtype), int(window_cap_bytes)))
    return Plan(h.value, world, b, d, seq.tolist(), head.tolist(), _dtype_code(dtype),
                window_cap_bytes)


def ulysses_plan_destroy(plan):
    plan.destroy()


def ulysses_plan_shape(plan, mode, rank, is_dst):
    out = np.zeros(4, dtype=np.int64)
    _check(_load().ulysses_plan_shape(plan.handle, int(mode), int(rank), int(bool(is_dst)),
                                      out.ctypes.data))
    return tuple(int(v) for v in out)


def ulysses_plan_window_bytes(plan, mode):
    return int(_check(_load().ulysses_plan_window_bytes(plan.handle, int(mode))))


def ulysses_plan_bytes(plan, mode):
    return int(_check(_load().ulysses_plan_bytes(plan.handle, int(mode))))


def ulysses_a2a_4d(plan, mode, src, dst, stream=None):
    w = plan.world
    _check(_load().ulysses_a2a_4d(
        plan.handle, int(mode), _ptr_array(src, w, "src", plan.shard_bytes(mode, False)),
        _ptr_array(dst, w, "dst", plan.shard_bytes(mode, True)), _stream(stream)))


def ulysses_a2a_4d_multi(plan, mode, srcs, dsts, stream=None):
    """srcs, dsts: one list of W shards per tensor (at most 4 tensors)."""
    w = plan.world
    srcs, dsts = list(srcs), list(dsts)
    if len(srcs) != len(dsts) or not srcs:
        raise ValueError("need the same number (>= 1) of source and destination tensors")
    flat_s = [x for t in srcs for x in _check_len(t, w, "src")]
    flat_d = [x for t in dsts for x in _check_len(t, w, "dst")]
    _check(_load().ulysses_a2a_4d_multi(
        plan.handle, int(mode), len(srcs),
        _ptr_array(flat_s, len(flat_s), "src", plan.shard_bytes(mode, False) * len(srcs)),
        _ptr_array(flat_d, len(flat_d), "dst", plan.shard_bytes(mode, True) * len(dsts)),
        _stream(stream)))


def _check_len(items, world, what):
    items = list(items)
    if len(items) != world:
        raise ValueError(f"{what}: need {world} shards per tensor, got {len(items)}")
    return items


def ulysses_a2a_4d_chunked(plan, mode, src, dst, window=None, stream=None):
    """window: W device buffers, window r holding one batch plane of
    destination r (ulysses_plan_window_bytes is enough for every rank), or
    None: each plane is relayed straight into its place in dst (no copy-out)."""
    w = plan.world
    planes = [n // plan.b for n in plan.shard_bytes(mode, True)]
    win = None if window is None else _ptr_array(window, w, "window", planes)
    _check(_load().ulysses_a2a_4d_chunked(
        plan.handle, int(mode), _ptr_array(src, w, "src", plan.shard_bytes(mode, False)),
        _ptr_array(dst, w, "dst", plan.shard_bytes(mode, True)), win, _stream(stream)))


def ulysses_a2a_4d_chunked_static(plan, mode, src, dst, stream=None):
    """The plane-at-a-time call with the library's static windows (no
    allocation anywhere in the call)."""
    w = plan.world
    _check(_load().ulysses_a2a_4d_chunked_static(
        plan.handle, int(mode), _ptr_array(src, w, "src", plan.shard_bytes(mode, False)),
        _ptr_array(dst, w, "dst", plan.shard_bytes(mode, True)), _stream(stream)))


def ulysses_a2a_4d_qknorm_rope(plan, q_src, q_dst, k_src, k_dst, gamma_q, gamma_k, eps,
                               rope_cos, rope_sin, stream=None):
    w = plan.world
    sb, db = plan.shard_bytes(0, False), plan.shard_bytes(0, True)
    gb = 4 * plan.d
    tb = 4 * sum(plan.seq_splits) * (plan.d // 2)
    _check(_load().ulysses_a2a_4d_qknorm_rope(
        plan.handle, _ptr_array(q_src, w, "q_src", sb), _ptr_array(q_dst, w, "q_dst", db),
        _ptr_array(k_src, w, "k_src", sb), _ptr_array(k_dst, w, "k_dst", db),
        _addr(gamma_q, gb, "gamma_q"), _addr(gamma_k, gb, "gamma_k"), float(eps),
        _addr(rope_cos, tb, "rope_cos"), _addr(rope_sin, tb, "rope_sin"), _stream(stream)))


def ulysses_rope_table(theta, s_global, d):
    """Host tables (cos, sin), float32 [s_global, d/2], computed by the library."""
    c = np.empty((int(s_global), int(d) // 2), dtype=np.float32)
    s = np.empty_like(c)
    _check(_load().ulysses_rope_table(float(theta), int(s_global), int(d), c.ctypes.data,
                                      s.ctypes.data))
    return c, s
