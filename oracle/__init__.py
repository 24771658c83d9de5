"""CPU oracle for TQ1_0 x Q8_1 mat-vec -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product (``bit_quantized_mat_amd``)
never imports it, and nothing here imports the product.

This module only marshals numpy arrays into the plain C implementation in
``tq1_oracle.c`` (which carries the citations) and parses byte fields.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

TQ1_BLOCK_BYTES = 54
Q81_BLOCK_BYTES = 36

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def lib():
    """Load the oracle library, compiling it first only if it is not built."""
    global _lib
    if _lib is None:
        # TQ1_ORACLE_LIB lets the mutation test load a deliberately broken copy
        path = os.environ.get("TQ1_ORACLE_LIB", _build.LIB)
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        L.oracle_f16_to_f32.restype = ctypes.c_float
        L.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.oracle_f32_to_f16.restype = ctypes.c_uint16
        L.oracle_f32_to_f16.argtypes = [ctypes.c_float]
        L.oracle_f32_to_f16_array.argtypes = [_p, _p, _i64]
        L.oracle_f16_to_f32_array.argtypes = [_p, _p, _i64]
        L.oracle_tq1_element_slot.argtypes = [ctypes.c_int, _p, _p]
        L.oracle_tq1_slot_element.argtypes = [ctypes.c_int, ctypes.c_int]
        L.oracle_tq1_slot_element.restype = ctypes.c_int
        L.oracle_base3_digit.argtypes = [ctypes.c_int, ctypes.c_int]
        L.oracle_base3_digit.restype = ctypes.c_int
        for name in ("oracle_tq1_pack", "oracle_tq1_unpack"):
            getattr(L, name).argtypes = [_p, _p, _p, _i64, _i64]
            getattr(L, name).restype = ctypes.c_int
        L.oracle_q8_1_quantize.argtypes = [_p, _p, _i64, _i64]
        L.oracle_q8_1_quantize.restype = ctypes.c_int
        for name in ("oracle_block_isums_elem", "oracle_block_isums_bytes"):
            getattr(L, name).argtypes = [_p, _p, _p, _i64, _i64, _i64]
            getattr(L, name).restype = ctypes.c_int
        L.oracle_mmvq.argtypes = [_p, _p, _p, _p, _p, _i64, _i64, _i64]
        L.oracle_mmvq.restype = ctypes.c_int
        L.oracle_mmvq_add.argtypes = [_p, _p, _p, _p, _p, _p, _i64, _i64, _i64]
        L.oracle_mmvq_add.restype = ctypes.c_int
        L.oracle_mmvq_glu.argtypes = [_p] * 9 + [_i64, _i64, _i64]
        L.oracle_mmvq_glu.restype = ctypes.c_int
        L.oracle_mmvq_id.argtypes = [_p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64]
        L.oracle_mmvq_id.restype = ctypes.c_int
        L.oracle_mmvq_id_slots.argtypes = [_p, _p, _p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64]
        L.oracle_mmvq_id_slots.restype = ctypes.c_int
        L.oracle_tq2_element_slot.argtypes = [ctypes.c_int, _p, _p]
        for name in ("oracle_tq2_pack", "oracle_tq2_unpack"):
            getattr(L, name).argtypes = [_p, _p, _p, _i64, _i64]
            getattr(L, name).restype = ctypes.c_int
        for name in ("oracle_tq2_block_isums_elem", "oracle_tq2_block_isums_bytes"):
            getattr(L, name).argtypes = [_p, _p, _p, _i64, _i64, _i64]
            getattr(L, name).restype = ctypes.c_int
        L.oracle_tq2_mmvq.argtypes = [_p, _p, _p, _p, _p, _i64, _i64, _i64]
        L.oracle_tq2_mmvq.restype = ctypes.c_int
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_tq1_dequantize_rows.argtypes = [_p, _p, _p, _i64, _i64, _i64, ctypes.c_int]
        L.oracle_tq1_dequantize_rows.restype = ctypes.c_int
        L.oracle_set_threads.argtypes = [ctypes.c_int]
        L.oracle_max_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None else None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class OracleError(ValueError):
    pass


def _check(rc, what):
    if rc != 0:
        raise OracleError("%s rejected its input (rc=%d)" % (what, rc))


# ---- fp16 -------------------------------------------------------------------

def f32_to_f16_bits(x):
    x = _c(x, np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().oracle_f32_to_f16_array(_ptr(x), _ptr(out), x.size)
    return out


def f16_bits_to_f32(h):
    h = _c(h, np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    lib().oracle_f16_to_f32_array(_ptr(h), _ptr(out), h.size)
    return out


# ---- TQ1_0 format -------------------------------------------------------------

def element_slot(e):
    b = ctypes.c_int()
    c = ctypes.c_int()
    lib().oracle_tq1_element_slot(int(e), ctypes.byref(b), ctypes.byref(c))
    return b.value, c.value


def slot_element(byte_index, digit):
    return lib().oracle_tq1_slot_element(int(byte_index), int(digit))


def base3_digit(v, c):
    return lib().oracle_base3_digit(int(v), int(c))


def tq1_pack(trits, d16):
    """trits int8 [N, K] in {-1,0,1}; d16 uint16 [N, K/256] (fp16 bits) -> uint8 [N, K/256*54]."""
    trits = _c(trits, np.int8)
    d16 = _c(d16, np.uint16)
    N, K = trits.shape
    out = np.empty((N, (K // 256) * TQ1_BLOCK_BYTES), dtype=np.uint8)
    _check(lib().oracle_tq1_pack(_ptr(trits), _ptr(d16), _ptr(out), N, K), "tq1_pack")
    return out


def tq1_unpack(w, N, K):
    w = _c(w, np.uint8)
    trits = np.empty((N, K), dtype=np.int8)
    d16 = np.empty((N, K // 256), dtype=np.uint16)
    _check(lib().oracle_tq1_unpack(_ptr(w), _ptr(trits), _ptr(d16), N, K), "tq1_unpack")
    return trits, d16


# ---- Q8_1 -----------------------------------------------------------------------

def q8_1_quantize(x):
    """x float32 [T, K] -> uint8 [T, K/32*36]."""
    x = _c(x, np.float32)
    T, K = x.shape
    out = np.empty((T, (K // 32) * Q81_BLOCK_BYTES), dtype=np.uint8)
    _check(lib().oracle_q8_1_quantize(_ptr(x), _ptr(out), T, K), "q8_1_quantize")
    return out


def q8_1_fields(a, T, K):
    """Split Q8_1 bytes into (q int8 [T,K], d16 uint16 [T,K/32], s16 uint16 [T,K/32])."""
    blk = _c(a, np.uint8).reshape(T, K // 32, Q81_BLOCK_BYTES)
    q = blk[:, :, :32].view(np.int8).reshape(T, K)
    d16 = np.ascontiguousarray(blk[:, :, 32:34]).view(np.uint16).reshape(T, K // 32)
    s16 = np.ascontiguousarray(blk[:, :, 34:36]).view(np.uint16).reshape(T, K // 32)
    return q, d16, s16


# ---- products --------------------------------------------------------------------

def block_isums(w, a, N, K, T, method="elem"):
    """Per-32-element integer sums, int32 [T, N, K/32]."""
    w = _c(w, np.uint8)
    a = _c(a, np.uint8)
    out = np.empty((T, N, K // 32), dtype=np.int32)
    fn = {"elem": lib().oracle_block_isums_elem,
          "bytes": lib().oracle_block_isums_bytes}[method]
    _check(fn(_ptr(w), _ptr(a), _ptr(out), N, K, T), "block_isums")
    return out


def mmvq(w, a, N, K, T):
    """Returns (y float32 [T,N], y64 float64 [T,N], abs64 float64 [T,N])."""
    w = _c(w, np.uint8)
    a = _c(a, np.uint8)
    y = np.empty((T, N), dtype=np.float32)
    y64 = np.empty((T, N), dtype=np.float64)
    ab = np.empty((T, N), dtype=np.float64)
    _check(lib().oracle_mmvq(_ptr(w), _ptr(a), _ptr(y), _ptr(y64), _ptr(ab), N, K, T), "mmvq")
    return y, y64, ab


def mmvq_add(w, a, r, N, K, T):
    """The mat-vec plus a residual r float32 [T, N]: returns (y, y64, abs64),
    each [T, N], with abs64 = sum |terms| + |r|."""
    w = _c(w, np.uint8)
    a = _c(a, np.uint8)
    r = _c(r, np.float32)
    assert r.shape == (T, N)
    y = np.empty((T, N), dtype=np.float32)
    y64 = np.empty((T, N), dtype=np.float64)
    ab = np.empty((T, N), dtype=np.float64)
    _check(lib().oracle_mmvq_add(_ptr(w), _ptr(a), _ptr(r), _ptr(y), _ptr(y64), _ptr(ab), N, K,
                                 T), "mmvq_add")
    return y, y64, ab


def mmvq_glu(w_gate, w_up, a, N, K, T):
    """The gate-up pair with its gated-linear-unit epilogue, y = silu(g) * u:
    returns (y float32, y64, g64, u64, absg, absu), each [T, N], where g and
    u are the two exact mat-vecs and absg, absu their sum |terms|."""
    wg = _c(w_gate, np.uint8)
    wu = _c(w_up, np.uint8)
    a = _c(a, np.uint8)
    out = [np.empty((T, N), dtype=np.float32)] + [np.empty((T, N), dtype=np.float64)
                                                   for _ in range(5)]
    _check(lib().oracle_mmvq_glu(_ptr(wg), _ptr(wu), _ptr(a), *[_ptr(o) for o in out], N, K, T),
           "mmvq_glu")
    return tuple(out)


def mmvq_id(w, a, ids, E, N, K, T, n_used, per_slot=False):
    """Returns (y, y64, abs64), each [T, n_used, N]. a holds one Q8_1 column
    per token ([T, K/32] blocks), or per (token, slot) pair with per_slot
    ([T, n_used, K/32] blocks)."""
    w = _c(w, np.uint8)
    a = _c(a, np.uint8)
    ids = _c(ids, np.int32)
    shape = (T, n_used, N)
    y = np.empty(shape, dtype=np.float32)
    y64 = np.empty(shape, dtype=np.float64)
    ab = np.empty(shape, dtype=np.float64)
    f = lib().oracle_mmvq_id_slots if per_slot else lib().oracle_mmvq_id
    _check(f(_ptr(w), _ptr(a), _ptr(ids), _ptr(y), _ptr(y64), _ptr(ab), E, N, K, T, n_used),
           "mmvq_id")
    return y, y64, ab


# ---- TQ2_0 (2-bit digit fields; the reading is stated in tq1_oracle.c) -----------

TQ2_BLOCK_BYTES = 66


def tq2_element_slot(e):
    b = ctypes.c_int()
    f = ctypes.c_int()
    lib().oracle_tq2_element_slot(int(e), ctypes.byref(b), ctypes.byref(f))
    return b.value, f.value


def tq2_pack(trits, d16):
    """trits int8 [N, K] in {-1,0,1}; d16 uint16 [N, K/256] -> uint8 [N, K/256*66]."""
    trits = _c(trits, np.int8)
    d16 = _c(d16, np.uint16)
    N, K = trits.shape
    out = np.empty((N, (K // 256) * TQ2_BLOCK_BYTES), dtype=np.uint8)
    _check(lib().oracle_tq2_pack(_ptr(trits), _ptr(d16), _ptr(out), N, K), "tq2_pack")
    return out


def tq2_unpack(w, N, K):
    w = _c(w, np.uint8)
    trits = np.empty((N, K), dtype=np.int8)
    d16 = np.empty((N, K // 256), dtype=np.uint16)
    _check(lib().oracle_tq2_unpack(_ptr(w), _ptr(trits), _ptr(d16), N, K), "tq2_unpack")
    return trits, d16


def tq2_block_isums(w, a, N, K, T, method="elem"):
    """Per-32-element integer sums of TQ2_0 rows, int32 [T, N, K/32]."""
    w = _c(w, np.uint8)
    a = _c(a, np.uint8)
    out = np.empty((T, N, K // 32), dtype=np.int32)
    fn = {"elem": lib().oracle_tq2_block_isums_elem,
          "bytes": lib().oracle_tq2_block_isums_bytes}[method]
    _check(fn(_ptr(w), _ptr(a), _ptr(out), N, K, T), "tq2_block_isums")
    return out


def tq2_mmvq(w, a, N, K, T):
    """TQ2_0 mat-vec: (y float32 [T,N], y64 float64 [T,N], abs64 float64 [T,N])."""
    w = _c(w, np.uint8)
    a = _c(a, np.uint8)
    y = np.empty((T, N), dtype=np.float32)
    y64 = np.empty((T, N), dtype=np.float64)
    ab = np.empty((T, N), dtype=np.float64)
    _check(lib().oracle_tq2_mmvq(_ptr(w), _ptr(a), _ptr(y), _ptr(y64), _ptr(ab), N, K, T),
           "tq2_mmvq")
    return y, y64, ab


DTYPES = {"f32": (0, np.float32), "f16": (1, np.uint16), "bf16": (2, np.uint16)}


def f32_to_bf16_bits(x):
    """bfloat16 bit patterns (uint16) of fp32 values, round to nearest even."""
    x = np.asarray(x, dtype=np.float32)
    f = lib().oracle_f32_to_bf16
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint16).reshape(x.shape)


def tq1_dequantize(w, N, K, dtype="f32", rows=None):
    """Dequantized rows [n_rows, K] of a packed [N, K] matrix: fp32 values,
    or fp16 / bf16 bit patterns (uint16); rows=None takes rows 0..N-1."""
    code, npdt = DTYPES[dtype]
    w = _c(w, np.uint8)
    rws = None if rows is None else _c(rows, np.int32)
    n_rows = N if rows is None else int(rws.size)
    out = np.empty((n_rows, K), dtype=npdt)
    rc = lib().oracle_tq1_dequantize_rows(_ptr(w), None if rws is None else _ptr(rws), _ptr(out),
                                          N, K, n_rows, code)
    _check(rc, "tq1_dequantize")
    return out


def set_threads(n):
    lib().oracle_set_threads(int(n))


def max_threads():
    return lib().oracle_max_threads()
