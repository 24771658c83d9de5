"""MI355X (gfx950) TQ1_0 (and TQ2_0) x Q8_1 quantized mat-vec.

A thin binding over the C ABI in ``include/bqm.h`` (library ``libbqm.so``,
built in-tree by ``bit_quantized_mat_amd.build``). Every function here only
checks and marshals arguments: tensors are torch device tensors used as plain
device memory, and every step of the computation runs in the HIP kernels.
There is no CPU fallback: if the library is missing, calls raise.
"""
import ctypes
import os

__all__ = [
    "BqmError", "library", "library_path", "tq1_pack", "q8_1_quantize", "mmvq_tq1_0", "mm_tq1_0",
    "MM_MAX_COLS",
    "mmvq_tq1_0_f32", "MMVQ_F32_MAX_COLS", "tq1_dequantize", "mmvq_tq1_0_add",
    "mmvq_tq1_0_f32_add", "mmvq_tq1_0_glu", "mmvq_tq1_0_f32_glu", "GLU_MAX_COLS",
    "GLU_F32_MAX_COLS",
    "mmvq_id_tq1_0", "mmvq_id_tq1_0_slots", "mmvq_id_tq1_0_workspace_bytes",
    "mmvq_id_tq1_0_noalloc", "NOALLOC_SCRATCH_BYTES",
    "mmvq_tq1_0_block_isums", "tq2_pack", "mmvq_tq2_0", "mmvq_tq2_0_block_isums",
    "TQ1_BLOCK_BYTES", "TQ2_BLOCK_BYTES", "Q81_BLOCK_BYTES", "MMVQ_MAX_COLS",
]

TQ1_BLOCK_BYTES = 54
TQ2_BLOCK_BYTES = 66
Q81_BLOCK_BYTES = 36
MMVQ_MAX_COLS = 32
MMVQ_F32_MAX_COLS = 8
MM_MAX_COLS = 65536
GLU_MAX_COLS = 32
GLU_F32_MAX_COLS = 2
NOALLOC_SCRATCH_BYTES = 768 * 1024

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

_i32, _i64, _p, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t


class BqmError(RuntimeError):
    """A library entry point returned a non-zero status."""

    def __init__(self, fn, status):
        text = library().bqm_status_string(status).decode()
        super().__init__("%s failed with status %d (%s)" % (fn, status, text))
        self.status = status


def library_path():
    return os.path.join(_HERE, "libbqm.so")


def library():
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError("libbqm.so is not built; run bit_quantized_mat_amd.build.build() "
                               "(or __graft_entry__.build()) first")
        L = ctypes.CDLL(path)
        L.tq1_pack.argtypes = [_p, _p, _p, _i64, _i64, _p]
        L.q8_1_quantize.argtypes = [_p, _p, _i64, _i64, _p]
        L.mmvq_tq1_0.argtypes = [_p, _p, _p, _i64, _i64, _i32, _p]
        L.mmvq_tq1_0_f32.argtypes = [_p, _p, _p, _i64, _i64, _i32, _p]
        L.mmvq_tq1_0_add.argtypes = [_p, _p, _p, _p, _i64, _i64, _i32, _p]
        L.mmvq_tq1_0_f32_add.argtypes = [_p, _p, _p, _p, _i64, _i64, _i32, _p]
        L.mmvq_tq1_0_glu.argtypes = [_p, _p, _p, _p, _i64, _i64, _i32, _p]
        L.mmvq_tq1_0_f32_glu.argtypes = [_p, _p, _p, _p, _i64, _i64, _i32, _p]
        L.mm_tq1_0.argtypes = [_p, _p, _p, _i64, _i64, _i64, _p]
        L.tq1_dequantize.argtypes = [_p, _p, _p, _i64, _i64, _i64, _i32, _p]
        L.mmvq_tq1_0_block_isums.argtypes = [_p, _p, _p, _i64, _i64, _i32, _p]
        L.mmvq_id_tq1_0.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _i32, _p, _sz, _p]
        L.mmvq_id_tq1_0_slots.argtypes = L.mmvq_id_tq1_0.argtypes
        L.mmvq_id_tq1_0_noalloc.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _i32, _p]
        L.tq2_pack.argtypes = [_p, _p, _p, _i64, _i64, _p]
        L.mmvq_tq2_0.argtypes = [_p, _p, _p, _i64, _i64, _i32, _p]
        L.mmvq_tq2_0_block_isums.argtypes = [_p, _p, _p, _i64, _i64, _i32, _p]
        L.mmvq_id_tq1_0_workspace_bytes.argtypes = [_i64, _i64, _i32]
        L.mmvq_id_tq1_0_workspace_bytes.restype = _sz
        L.bqm_status_string.argtypes = [ctypes.c_int]
        L.bqm_status_string.restype = ctypes.c_char_p
        L.bqm_version.restype = ctypes.c_int
        for name in ("tq1_pack", "q8_1_quantize", "mmvq_tq1_0", "mm_tq1_0", "mmvq_tq1_0_f32",
                     "mmvq_tq1_0_add", "mmvq_tq1_0_f32_add", "mmvq_tq1_0_glu",
                     "mmvq_tq1_0_f32_glu", "mmvq_tq1_0_block_isums", "mmvq_id_tq1_0", "mmvq_id_tq1_0_slots",
                     "mmvq_id_tq1_0_noalloc", "tq1_dequantize", "tq2_pack", "mmvq_tq2_0",
                     "mmvq_tq2_0_block_isums"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _torch():
    import torch
    return torch


def _stream(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _dev_tensor(t, name, dtypes, min_bytes, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a GPU tensor" % name)
    if t.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.numel() * t.element_size() < min_bytes:
        raise ValueError("%s holds %d bytes, needs %d" % (name, t.numel() * t.element_size(), min_bytes))
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    return ctypes.c_void_p(t.data_ptr())


def _call(fn, *args):
    rc = getattr(library(), fn)(*args)
    if rc != 0:
        raise BqmError(fn, rc)


def tq1_pack(trits, d16, out=None, stream=None):
    """trits int8 [N, K] (values -1/0/1), d16 fp16 or int16/uint16 bits [N, K/256]
    -> TQ1_0 bytes uint8 [N, K/256*54]."""
    torch = _torch()
    N, K = trits.shape
    nb = K // 256
    if out is None:
        out = torch.empty((N, nb * TQ1_BLOCK_BYTES), dtype=torch.uint8, device=trits.device)
    dtypes16 = (torch.float16, torch.int16, torch.uint16)
    _call("tq1_pack",
          _dev_tensor(trits, "trits", (torch.int8,), N * K),
          _dev_tensor(d16, "d16", dtypes16, N * nb * 2, trits.device),
          _dev_tensor(out, "out", (torch.uint8,), N * nb * TQ1_BLOCK_BYTES, trits.device),
          N, K, _stream(stream, trits.device))
    return out


def q8_1_quantize(x, out=None, stream=None):
    """x fp32 [T, K] -> Q8_1 bytes uint8 [T, K/32*36]."""
    torch = _torch()
    T, K = x.shape
    if out is None:
        out = torch.empty((T, (K // 32) * Q81_BLOCK_BYTES), dtype=torch.uint8, device=x.device)
    _call("q8_1_quantize",
          _dev_tensor(x, "x", (torch.float32,), T * K * 4),
          _dev_tensor(out, "out", (torch.uint8,), T * (K // 32) * Q81_BLOCK_BYTES, x.device),
          T, K, _stream(stream, x.device))
    return out


def _mmvq_args(w, a, N, K, T, block_bytes=TQ1_BLOCK_BYTES):
    torch = _torch()
    return (_dev_tensor(w, "w", (torch.uint8,), N * (K // 256) * block_bytes),
            _dev_tensor(a, "a", (torch.uint8,), T * (K // 32) * Q81_BLOCK_BYTES, w.device))


def mmvq_tq1_0(w, a, N, K, T, out=None, stream=None):
    """y fp32 [T, N] = TQ1_0 weights [N, K] times T Q8_1 activation columns."""
    torch = _torch()
    if out is None:
        out = torch.empty((T, N), dtype=torch.float32, device=w.device)
    pw, pa = _mmvq_args(w, a, N, K, T)
    _call("mmvq_tq1_0", pw, pa, _dev_tensor(out, "out", (torch.float32,), T * N * 4, w.device),
          N, K, T, _stream(stream, w.device))
    return out


def mm_tq1_0(w, a, N, K, T, out=None, stream=None):
    """y fp32 [T, N] = TQ1_0 weights [N, K] times T Q8_1 activation columns,
    any T up to MM_MAX_COLS: within the header's stated bound of the exact
    sums; up to 32 columns the call is mmvq_tq1_0, beyond it not necessarily
    bitwise mmvq_tq1_0's."""
    torch = _torch()
    if out is None:
        out = torch.empty((T, N), dtype=torch.float32, device=w.device)
    pw, pa = _mmvq_args(w, a, N, K, T)
    _call("mm_tq1_0", pw, pa, _dev_tensor(out, "out", (torch.float32,), T * N * 4, w.device),
          N, K, T, _stream(stream, w.device))
    return out


def mmvq_tq1_0_f32(w, x, N, K, T, out=None, stream=None):
    """y fp32 [T, N] = TQ1_0 weights [N, K] times T fp32 activation columns
    x [T, K], quantized to Q8_1 inside the call (bitwise q8_1_quantize then
    mmvq_tq1_0); T <= 8."""
    torch = _torch()
    if out is None:
        out = torch.empty((T, N), dtype=torch.float32, device=w.device)
    _call("mmvq_tq1_0_f32",
          _dev_tensor(w, "w", (torch.uint8,), N * (K // 256) * TQ1_BLOCK_BYTES),
          _dev_tensor(x, "x", (torch.float32,), T * K * 4, w.device),
          _dev_tensor(out, "out", (torch.float32,), T * N * 4, w.device),
          N, K, T, _stream(stream, w.device))
    return out


def mmvq_tq1_0_add(w, a, r, N, K, T, out=None, stream=None):
    """y fp32 [T, N] = mmvq_tq1_0(w, a) + r (r fp32 [T, N]; out may be r
    itself for an in-place accumulate)."""
    torch = _torch()
    if out is None:
        out = torch.empty((T, N), dtype=torch.float32, device=w.device)
    pw, pa = _mmvq_args(w, a, N, K, T)
    _call("mmvq_tq1_0_add", pw, pa, _dev_tensor(r, "r", (torch.float32,), T * N * 4, w.device),
          _dev_tensor(out, "out", (torch.float32,), T * N * 4, w.device),
          N, K, T, _stream(stream, w.device))
    return out


def mmvq_tq1_0_f32_add(w, x, r, N, K, T, out=None, stream=None):
    """y fp32 [T, N] = mmvq_tq1_0_f32(w, x) + r (quantize, multiply and add
    in one launch; out may be r itself)."""
    torch = _torch()
    if out is None:
        out = torch.empty((T, N), dtype=torch.float32, device=w.device)
    _call("mmvq_tq1_0_f32_add",
          _dev_tensor(w, "w", (torch.uint8,), N * (K // 256) * TQ1_BLOCK_BYTES),
          _dev_tensor(x, "x", (torch.float32,), T * K * 4, w.device),
          _dev_tensor(r, "r", (torch.float32,), T * N * 4, w.device),
          _dev_tensor(out, "out", (torch.float32,), T * N * 4, w.device),
          N, K, T, _stream(stream, w.device))
    return out


def mmvq_tq1_0_glu(w_gate, w_up, a, N, K, T, out=None, stream=None):
    """y fp32 [T, N] = silu(mmvq_tq1_0(w_gate, a)) * mmvq_tq1_0(w_up, a),
    1 <= T <= GLU_MAX_COLS (one launch up to two columns, two beyond)."""
    torch = _torch()
    if out is None:
        out = torch.empty((T, N), dtype=torch.float32, device=w_gate.device)
    pw, pa = _mmvq_args(w_gate, a, N, K, T)
    _call("mmvq_tq1_0_glu", pw,
          _dev_tensor(w_up, "w_up", (torch.uint8,), N * (K // 256) * TQ1_BLOCK_BYTES,
                      w_gate.device), pa,
          _dev_tensor(out, "out", (torch.float32,), T * N * 4, w_gate.device),
          N, K, T, _stream(stream, w_gate.device))
    return out


def mmvq_tq1_0_f32_glu(w_gate, w_up, x, N, K, T, out=None, stream=None):
    """The same on fp32 activations x [T, K], quantized inside the call
    (1 <= T <= GLU_F32_MAX_COLS)."""
    torch = _torch()
    if out is None:
        out = torch.empty((T, N), dtype=torch.float32, device=w_gate.device)
    _call("mmvq_tq1_0_f32_glu",
          _dev_tensor(w_gate, "w_gate", (torch.uint8,), N * (K // 256) * TQ1_BLOCK_BYTES),
          _dev_tensor(w_up, "w_up", (torch.uint8,), N * (K // 256) * TQ1_BLOCK_BYTES,
                      w_gate.device),
          _dev_tensor(x, "x", (torch.float32,), T * K * 4, w_gate.device),
          _dev_tensor(out, "out", (torch.float32,), T * N * 4, w_gate.device),
          N, K, T, _stream(stream, w_gate.device))
    return out


def tq1_dequantize(w, N, K, rows=None, dtype=None, out=None, stream=None):
    """Dequantized rows [n_rows, K] of the packed [N, K] matrix w: row
    rows[i] (int32 GPU tensor) or, with rows=None, all N rows; dtype
    torch.float32, torch.float16 (default) or torch.bfloat16."""
    torch = _torch()
    dtype = torch.float16 if dtype is None else dtype
    codes = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
    if dtype not in codes:
        raise TypeError("dtype must be float32, float16 or bfloat16")
    n_rows = N if rows is None else rows.numel()
    if out is None:
        out = torch.empty((n_rows, K), dtype=dtype, device=w.device)
    pr = ctypes.c_void_p(None) if rows is None else _dev_tensor(rows, "rows", (torch.int32,),
                                                                 n_rows * 4, w.device)
    _call("tq1_dequantize",
          _dev_tensor(w, "w", (torch.uint8,), N * (K // 256) * TQ1_BLOCK_BYTES),
          pr, _dev_tensor(out, "out", (dtype,), n_rows * K * out.element_size(), w.device),
          N, K, n_rows, codes[dtype], _stream(stream, w.device))
    return out


def mmvq_tq1_0_block_isums(w, a, N, K, T, out=None, stream=None):
    """Exact per-32 integer sums int32 [T, N, K/32] from the production inner loop."""
    torch = _torch()
    if out is None:
        out = torch.empty((T, N, K // 32), dtype=torch.int32, device=w.device)
    pw, pa = _mmvq_args(w, a, N, K, T)
    _call("mmvq_tq1_0_block_isums", pw, pa,
          _dev_tensor(out, "out", (torch.int32,), T * N * (K // 32) * 4, w.device),
          N, K, T, _stream(stream, w.device))
    return out


def tq2_pack(trits, d16, out=None, stream=None):
    """trits int8 [N, K] (values -1/0/1), d16 fp16 or int16/uint16 bits [N, K/256]
    -> TQ2_0 bytes uint8 [N, K/256*66]."""
    torch = _torch()
    N, K = trits.shape
    nb = K // 256
    if out is None:
        out = torch.empty((N, nb * TQ2_BLOCK_BYTES), dtype=torch.uint8, device=trits.device)
    dtypes16 = (torch.float16, torch.int16, torch.uint16)
    _call("tq2_pack",
          _dev_tensor(trits, "trits", (torch.int8,), N * K),
          _dev_tensor(d16, "d16", dtypes16, N * nb * 2, trits.device),
          _dev_tensor(out, "out", (torch.uint8,), N * nb * TQ2_BLOCK_BYTES, trits.device),
          N, K, _stream(stream, trits.device))
    return out


def mmvq_tq2_0(w, a, N, K, T, out=None, stream=None):
    """y fp32 [T, N] = TQ2_0 weights [N, K] times T Q8_1 activation columns."""
    torch = _torch()
    if out is None:
        out = torch.empty((T, N), dtype=torch.float32, device=w.device)
    pw, pa = _mmvq_args(w, a, N, K, T, TQ2_BLOCK_BYTES)
    _call("mmvq_tq2_0", pw, pa, _dev_tensor(out, "out", (torch.float32,), T * N * 4, w.device),
          N, K, T, _stream(stream, w.device))
    return out


def mmvq_tq2_0_block_isums(w, a, N, K, T, out=None, stream=None):
    """Exact per-32 integer sums int32 [T, N, K/32] of TQ2_0 rows."""
    torch = _torch()
    if out is None:
        out = torch.empty((T, N, K // 32), dtype=torch.int32, device=w.device)
    pw, pa = _mmvq_args(w, a, N, K, T, TQ2_BLOCK_BYTES)
    _call("mmvq_tq2_0_block_isums", pw, pa,
          _dev_tensor(out, "out", (torch.int32,), T * N * (K // 32) * 4, w.device),
          N, K, T, _stream(stream, w.device))
    return out


def mmvq_id_tq1_0_workspace_bytes(E, T, n_used):
    return int(library().mmvq_id_tq1_0_workspace_bytes(E, T, n_used))


def _mmvq_id(name, a_cols, w, a, ids, E, N, K, T, n_used, out, workspace, stream):
    torch = _torch()
    if out is None:
        out = torch.empty((T, n_used, N), dtype=torch.float32, device=w.device)
    need = mmvq_id_tq1_0_workspace_bytes(E, T, n_used)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=w.device)
    pw = _dev_tensor(w, "w", (torch.uint8,), E * N * (K // 256) * TQ1_BLOCK_BYTES)
    pa = _dev_tensor(a, "a", (torch.uint8,), a_cols * (K // 32) * Q81_BLOCK_BYTES, w.device)
    pi = _dev_tensor(ids, "ids", (torch.int32,), T * n_used * 4, w.device)
    py = _dev_tensor(out, "out", (torch.float32,), T * n_used * N * 4, w.device)
    if workspace is None:
        pws, nws = ctypes.c_void_p(None), 0
    else:
        pws = _dev_tensor(workspace, "workspace", (torch.uint8,), need, w.device)
        nws = workspace.numel()
    _call(name, pw, pa, pi, py, E, N, K, T, n_used, pws, nws, _stream(stream, w.device))
    return out


def mmvq_id_tq1_0(w, a, ids, E, N, K, T, n_used, out=None, workspace=None, stream=None):
    """y fp32 [T, n_used, N]: expert ids[t][s]'s matrix times token t's activation."""
    return _mmvq_id("mmvq_id_tq1_0", T, w, a, ids, E, N, K, T, n_used, out, workspace, stream)


def mmvq_id_tq1_0_slots(w, a, ids, E, N, K, T, n_used, out=None, workspace=None, stream=None):
    """y fp32 [T, n_used, N]: expert ids[t][s]'s matrix times pair (t, s)'s own
    activation (a: [T * n_used, K/32] Q8_1 blocks)."""
    return _mmvq_id("mmvq_id_tq1_0_slots", T * n_used, w, a, ids, E, N, K, T, n_used, out,
                    workspace, stream)


def mmvq_id_tq1_0_noalloc(w, a, ids, E, N, K, T, n_used, out=None, stream=None):
    """mmvq_id_tq1_0 with the library's own device scratch instead of a
    workspace: the call allocates nothing (``out`` is allocated here only if
    it is not given)."""
    torch = _torch()
    if out is None:
        out = torch.empty((T, n_used, N), dtype=torch.float32, device=w.device)
    _call("mmvq_id_tq1_0_noalloc",
          _dev_tensor(w, "w", (torch.uint8,), E * N * (K // 256) * TQ1_BLOCK_BYTES),
          _dev_tensor(a, "a", (torch.uint8,), T * (K // 32) * Q81_BLOCK_BYTES, w.device),
          _dev_tensor(ids, "ids", (torch.int32,), T * n_used * 4, w.device),
          _dev_tensor(out, "out", (torch.float32,), T * n_used * N * 4, w.device),
          E, N, K, T, n_used, _stream(stream, w.device))
    return out
