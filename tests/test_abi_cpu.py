"""CPU checks of the C ABI: the library loads, exports every entry point that
include/bqm.h declares, and rejects bad arguments on the host before any
device work (no compute call is made without a GPU)."""
import ctypes

import os
import re

import pytest

import bit_quantized_mat_amd as bqm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "bqm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"#define BQM_API.*", "", text)
    return sorted(set(re.findall(r"BQM_API\s+[\w\s\*]*?\b(\w+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = _declared_functions()
    for n in ("tq1_pack", "q8_1_quantize", "mmvq_tq1_0", "mm_tq1_0", "mmvq_tq1_0_f32",
              "mmvq_id_tq1_0",
              "mmvq_id_tq1_0_slots", "tq1_dequantize",
              "mmvq_id_tq1_0_workspace_bytes", "mmvq_tq1_0_block_isums",
              "tq2_pack", "mmvq_tq2_0", "mmvq_tq2_0_block_isums",
              "bqm_status_string", "bqm_version"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = bqm.library()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert lib.bqm_version() >= 100


def test_status_strings():
    lib = bqm.library()
    for code in range(0, -7, -1):
        assert lib.bqm_status_string(code) not in (b"", b"unknown status")
    assert lib.bqm_status_string(-99) == b"unknown status"


P = ctypes.c_void_p
GOOD = P(0x10000)       # aligned, never dereferenced: validation fails first
ODD = P(0x10002)


@pytest.mark.parametrize("args,expect", [
    # null pointers
    ((None, GOOD, GOOD, 4, 256, None), -1),
    ((GOOD, None, GOOD, 4, 256, None), -1),
    ((GOOD, GOOD, None, 4, 256, None), -1),
    # shapes
    ((GOOD, GOOD, GOOD, 0, 256, None), -2),
    ((GOOD, GOOD, GOOD, 4, 255, None), -2),
    ((GOOD, GOOD, GOOD, 4, 384, None), -2),
    ((GOOD, GOOD, GOOD, 4, 0, None), -2),
    ((GOOD, GOOD, GOOD, 1 << 40, 1 << 20, None), -2),
])
def test_tq1_pack_rejects(args, expect):
    assert bqm.library().tq1_pack(*args) == expect
    # TQ2_0 packing validates the same way
    assert bqm.library().tq2_pack(*args) == expect


def test_tq2_size_limit_counts_66_byte_blocks():
    # 70M blocks: 3.78 GB as TQ1_0 (accepted; then no device here), 4.62 GB as TQ2_0
    args = (GOOD, GOOD, GOOD, 1, 256 * 70_000_000, None)
    assert bqm.library().tq1_pack(*args) == -6
    assert bqm.library().tq2_pack(*args) == -2


@pytest.mark.parametrize("args,expect", [
    ((None, GOOD, 1, 32, None), -1),
    ((GOOD, None, 1, 32, None), -1),
    ((GOOD, GOOD, 0, 32, None), -2),
    ((GOOD, GOOD, 1, 48, None), -2),
    ((GOOD, GOOD, 1, 0, None), -2),
    ((ODD, GOOD, 1, 32, None), -3),
    ((GOOD, ODD, 1, 32, None), -3),
])
def test_q8_1_quantize_rejects(args, expect):
    assert bqm.library().q8_1_quantize(*args) == expect


@pytest.mark.parametrize("fn", ["mmvq_tq1_0", "mmvq_tq1_0_block_isums", "mmvq_tq2_0",
                                "mmvq_tq2_0_block_isums"])
@pytest.mark.parametrize("args,expect", [
    ((None, GOOD, GOOD, 8, 256, 1, None), -1),
    ((GOOD, None, GOOD, 8, 256, 1, None), -1),
    ((GOOD, GOOD, None, 8, 256, 1, None), -1),
    ((GOOD, GOOD, GOOD, 0, 256, 1, None), -2),
    ((GOOD, GOOD, GOOD, 8, 288, 1, None), -2),
    ((GOOD, GOOD, GOOD, 8, 256, 0, None), -2),
    ((GOOD, GOOD, GOOD, 8, 256, 33, None), -2),
    ((GOOD, GOOD, GOOD, 8, 256, -1, None), -2),
    ((ODD, GOOD, GOOD, 8, 256, 1, None), -3),
    ((GOOD, ODD, GOOD, 8, 256, 1, None), -3),
    ((GOOD, GOOD, ODD, 8, 256, 1, None), -3),
])
def test_mmvq_rejects(fn, args, expect):
    assert getattr(bqm.library(), fn)(*args) == expect


@pytest.mark.parametrize("args,expect", [
    ((None, GOOD, GOOD, 8, 256, 1, None), -1),
    ((GOOD, None, GOOD, 8, 256, 1, None), -1),
    ((GOOD, GOOD, None, 8, 256, 1, None), -1),
    ((GOOD, GOOD, GOOD, 0, 256, 1, None), -2),
    ((GOOD, GOOD, GOOD, 8, 288, 1, None), -2),
    ((GOOD, GOOD, GOOD, 8, 256, 0, None), -2),
    ((GOOD, GOOD, GOOD, 8, 256, 9, None), -2),            # beyond BQM_MMVQ_F32_MAX_COLS
    ((GOOD, GOOD, GOOD, 1, 1 << 28, 8, None), -2),        # x above 4 GiB
    ((ODD, GOOD, GOOD, 8, 256, 1, None), -3),
    ((GOOD, ODD, GOOD, 8, 256, 1, None), -3),
    ((GOOD, GOOD, ODD, 8, 256, 1, None), -3),
])
def test_mmvq_f32_rejects(args, expect):
    assert bqm.library().mmvq_tq1_0_f32(*args) == expect


@pytest.mark.parametrize("args,expect", [
    ((None, None, GOOD, 8, 256, 8, 1, None), -1),
    ((GOOD, None, None, 8, 256, 8, 1, None), -1),
    ((GOOD, None, GOOD, 0, 256, 8, 1, None), -2),
    ((GOOD, None, GOOD, 8, 300, 8, 1, None), -2),
    ((GOOD, None, GOOD, 8, 256, 0, 1, None), -2),
    ((GOOD, None, GOOD, 8, 256, 9, 1, None), -2),         # more rows than N without ids
    ((GOOD, GOOD, GOOD, 8, 256, 9, 3, None), -2),         # unknown dtype
    ((GOOD, GOOD, GOOD, 8, 256, 1 << 27, 0, None), -2),   # too many blocks
    ((ODD, None, GOOD, 8, 256, 8, 1, None), -3),
    ((GOOD, ODD, GOOD, 8, 256, 8, 1, None), -3),
    ((GOOD, None, P(0x100008), 8, 256, 8, 0, None), -3),  # fp32 output needs 16 bytes
    ((GOOD, None, P(0x100004), 8, 256, 8, 1, None), -3),  # every output needs 16 bytes
    ((GOOD, None, P(0x100008), 8, 256, 8, 2, None), -3),
])
def test_tq1_dequantize_rejects(args, expect):
    assert bqm.library().tq1_dequantize(*args) == expect


def test_mm_rejects():
    # invalid arguments return before touching the device
    lib = bqm.library()
    mm = lib.mm_tq1_0
    assert mm(None, GOOD, GOOD, 16, 256, 100, None) == -1
    assert mm(GOOD, GOOD, GOOD, 16, 256, 0, None) == -2
    assert mm(GOOD, GOOD, GOOD, 16, 256, 65537, None) == -2        # past BQM_MM_MAX_COLS
    assert mm(GOOD, GOOD, GOOD, 16, 100, 100, None) == -2          # K % 256
    assert mm(GOOD, GOOD, GOOD, 0, 256, 100, None) == -2
    assert mm(GOOD, GOOD, GOOD, 16, 1 << 24, 65536, None) == -2    # activations past 4 GiB
    assert mm(GOOD, ODD, GOOD, 16, 256, 100, None) == -3


def test_mmvq_id_slots_rejects():
    # the per-slot product validates like the shared one, and its activation
    # buffer holds T * n_used columns: 1000 tokens x 8 slots of K = 2^20 is
    # 9.4 GB, past the 4 GiB buffer limit (the shared shape would be 1.2 GB)
    lib = bqm.library()
    ws = P(0x100000)
    base = [GOOD, GOOD, GOOD, GOOD, 8, 16, 256, 4, 2, ws, 1 << 20, None]

    def call(**kw):
        args = list(base)
        names = ["w", "a", "ids", "y", "E", "N", "K", "T", "n_used", "ws", "wsb", "s"]
        for k, v in kw.items():
            args[names.index(k)] = v
        return lib.mmvq_id_tq1_0_slots(*args)

    assert call(a=None) == -1 and call(ids=None) == -1
    assert call(E=0) == -2 and call(n_used=9) == -2 and call(K=100) == -2
    assert call(T=40000, n_used=2) == -2
    assert call(K=1 << 20, T=1000, n_used=8, E=8) == -2
    assert call(a=ODD) == -3 and call(ws=P(0x100010)) == -3
    assert call(T=40, n_used=2, ws=None, wsb=0) == -4        # more than 64 pairs need a workspace


def test_mmvq_id_rejects():
    # every call below carries at least one invalid argument, so it returns
    # before touching the device (the pointers are never dereferenced)
    lib = bqm.library()
    ws = P(0x100000)
    need = lib.mmvq_id_tq1_0_workspace_bytes(8, 4, 2)
    base = [GOOD, GOOD, GOOD, GOOD, 8, 16, 256, 4, 2, ws, max(need, 256), None]

    def call(**kw):
        args = list(base)
        names = ["w", "a", "ids", "y", "E", "N", "K", "T", "n_used", "ws", "wsb", "s"]
        for k, v in kw.items():
            args[names.index(k)] = v
        return lib.mmvq_id_tq1_0(*args)

    assert call(w=None) == -1 and call(ids=None) == -1 and call(y=None) == -1
    assert call(E=0) == -2 and call(n_used=0) == -2 and call(n_used=9) == -2
    assert call(T=0) == -2 and call(K=100) == -2 and call(N=0) == -2
    assert call(T=40000, n_used=2) == -2          # more than 65535 (token, slot) pairs
    assert call(ids=ODD) == -3 and call(a=ODD) == -3
    assert call(ws=P(0x100010)) == -3             # workspace given but not 256-byte aligned
    if need > 0:
        assert call(ws=None) == -4 and call(wsb=need - 1) == -4
    assert need == 0                              # up to 64 pairs: routed inside the wave
    assert lib.mmvq_id_tq1_0_workspace_bytes(0, 4, 2) == 0
    assert lib.mmvq_id_tq1_0_workspace_bytes(8, 4, 9) == 0
    # more pairs: the routing pre-pass needs 2 + 6 * items + pairs int32 words
    # (two item lists of at most (P + 3 * min(E, P) + 3) / 4 entries of three
    # words -- items of up to four pairs -- one run slot per pair), rounded up
    # to 256 bytes
    for E, T, n_used in [(128, 64, 8), (128, 9, 8), (4, 65, 1), (4096, 1000, 4)]:
        pairs = T * n_used
        items = (pairs + 3 * min(E, pairs) + 3) // 4
        words = 2 + 6 * items + pairs
        assert lib.mmvq_id_tq1_0_workspace_bytes(E, T, n_used) == (4 * words + 255) // 256 * 256
    assert lib.mmvq_id_tq1_0_workspace_bytes(128, 8, 8) == 0      # exactly 64 pairs
    assert lib.mmvq_id_tq1_0_workspace_bytes(4097, 100, 1) == 0   # past the pre-pass's experts
    need = lib.mmvq_id_tq1_0_workspace_bytes(8, 40, 2)
    assert need > 0
    args = [GOOD, GOOD, GOOD, GOOD, 8, 16, 256, 40, 2, None, 0, None]
    assert lib.mmvq_id_tq1_0(*args) == -4                         # workspace missing
    args[9], args[10] = ws, need - 1
    assert lib.mmvq_id_tq1_0(*args) == -4                         # workspace too small


def test_binding_raises_without_gpu_tensors():
    import torch
    with pytest.raises(TypeError):
        bqm.mmvq_tq1_0(torch.zeros(54, dtype=torch.uint8), torch.zeros(36, dtype=torch.uint8), 1, 256, 1)


def test_mmvq_id_noalloc_rejects():
    # the allocation-free expert-routed call validates like mmvq_id_tq1_0
    # (every call below fails before touching the device), and every shape it
    # accepts has a workspace no larger than its device scratch
    lib = bqm.library()
    base = [GOOD, GOOD, GOOD, GOOD, 8, 16, 256, 4, 2, None]

    def call(**kw):
        args = list(base)
        names = ["w", "a", "ids", "y", "E", "N", "K", "T", "n_used", "s"]
        for k, v in kw.items():
            args[names.index(k)] = v
        return lib.mmvq_id_tq1_0_noalloc(*args)

    assert call(w=None) == -1 and call(a=None) == -1 and call(ids=None) == -1
    assert call(y=None) == -1
    assert call(E=0) == -2 and call(n_used=0) == -2 and call(n_used=9) == -2
    assert call(T=0) == -2 and call(K=100) == -2 and call(N=0) == -2
    assert call(T=40000, n_used=2) == -2
    assert call(K=1 << 24, T=300, n_used=1) == -2          # activations past 4 GiB
    assert call(w=ODD) == -3 and call(ids=ODD) == -3 and call(y=ODD) == -3
    worst = max(lib.mmvq_id_tq1_0_workspace_bytes(E, 65535 // n, n)
                for E in (1, 64, 4095, 4096) for n in (1, 2, 8, 64) if n <= E)
    assert worst == 729344
    assert worst <= bqm.NOALLOC_SCRATCH_BYTES == 768 * 1024


def test_mmvq_add_rejects():
    # the residual-add products validate like the plain ones, plus the
    # residual: required, 4-byte aligned, the output itself or disjoint from it
    lib = bqm.library()
    Y = P(0x200000)
    for fn, T in (("mmvq_tq1_0_add", 32), ("mmvq_tq1_0_f32_add", 8)):
        f = getattr(lib, fn)
        assert f(GOOD, GOOD, None, Y, 8, 256, 1, None) == -1
        assert f(None, GOOD, GOOD, Y, 8, 256, 1, None) == -1
        assert f(GOOD, GOOD, GOOD, None, 8, 256, 1, None) == -1
        assert f(GOOD, GOOD, GOOD, Y, 8, 256, T + 1, None) == -2
        assert f(GOOD, GOOD, GOOD, Y, 8, 300, 1, None) == -2
        # overlapping but not identical residual and output: -2
        assert f(GOOD, GOOD, P(0x200000 + 16), Y, 8, 256, 2, None) == -2
        assert f(GOOD, GOOD, P(0x200000 - 16), Y, 8, 256, 2, None) == -2
        assert f(GOOD, GOOD, P(0x200002), Y, 8, 256, 1, None) == -2   # overlaps, misaligned
        assert f(GOOD, GOOD, P(0x300002), Y, 8, 256, 1, None) == -3   # disjoint, misaligned
        assert f(GOOD, GOOD, GOOD, P(0x200002), 8, 256, 1, None) == -3


def test_mmvq_glu_rejects():
    # the gated pair: both matrices, the columns and the output required;
    # up to 32 columns (fp32 columns: 2); every pointer 4-byte aligned
    lib = bqm.library()
    Y = P(0x200000)
    assert bqm.GLU_MAX_COLS == 32
    assert bqm.GLU_F32_MAX_COLS == 2
    for fn, tmax in (("mmvq_tq1_0_glu", 32), ("mmvq_tq1_0_f32_glu", 2)):
        f = getattr(lib, fn)
        f.restype = ctypes.c_int
        assert f(GOOD, GOOD, GOOD, Y, 8, 256, tmax + 1, None) == -2
        assert f(None, GOOD, GOOD, Y, 8, 256, 1, None) == -1
        assert f(GOOD, None, GOOD, Y, 8, 256, 1, None) == -1
        assert f(GOOD, GOOD, None, Y, 8, 256, 1, None) == -1
        assert f(GOOD, GOOD, GOOD, None, 8, 256, 1, None) == -1
        assert f(GOOD, GOOD, GOOD, Y, 8, 256, 0, None) == -2
        assert f(GOOD, GOOD, GOOD, Y, 0, 256, 1, None) == -2
        assert f(GOOD, GOOD, GOOD, Y, 8, 300, 1, None) == -2
        assert f(ODD, GOOD, GOOD, Y, 8, 256, 1, None) == -3
        assert f(GOOD, ODD, GOOD, Y, 8, 256, 1, None) == -3
        assert f(GOOD, GOOD, ODD, Y, 8, 256, 1, None) == -3
        assert f(GOOD, GOOD, GOOD, P(0x200002), 8, 256, 1, None) == -3
