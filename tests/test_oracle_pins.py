"""Pins for the CPU oracle, against things other than the oracle itself.

Each test checks one oracle function against a library routine, a closed
form, a hand-worked fixture, an invariant or brute force on tiny inputs, so
that a dropped term, a wrong sign or index, or a transposed operand anywhere
in the oracle fails at least one of them. CPU only.
"""
import os

import numpy as np
import pytest

import oracle
from bit_quantized_mat_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------
# fp16 conversion: pinned to numpy's IEEE binary16 conversion (a library).
# ---------------------------------------------------------------------------

def test_f16_to_f32_all_bit_patterns():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_bits_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f32_to_f16_matches_numpy_rne():
    rng = np.random.default_rng(7)
    # every binary16 value, the midpoints between neighbours (ties), and
    # random floats over the whole binary16 range and beyond
    h = np.arange(0, 0x7C00, dtype=np.uint16)
    v = h.view(np.float16).astype(np.float64)
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float32)         # exact in fp32
    nudges = np.concatenate([np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    rand = (rng.standard_normal(200000) * np.exp2(rng.uniform(-30, 18, 200000))).astype(np.float32)
    edge = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 70000.0, 2.0**-24, 2.0**-25,
                     3 * 2.0**-26, 2.0**-26, 2.0**-14, 2.0**-14 - 2.0**-25, 1e-30, 1e30,
                     np.inf, -np.inf], dtype=np.float32)
    x = np.concatenate([v.astype(np.float32), mids, nudges, rand, -rand, edge, -edge])
    got = oracle.f32_to_f16_bits(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)
    nanbits = oracle.f32_to_f16_bits(np.array([np.nan], dtype=np.float32))
    assert np.isnan(nanbits.view(np.float16)[0])


# ---------------------------------------------------------------------------
# Base-3 digits and the element map.
# ---------------------------------------------------------------------------

def test_base3_digits_exhaustive_against_python_base_conversion():
    for v in range(243):
        digits = [oracle.base3_digit(v, c) for c in range(5)]
        # numpy.base_repr writes the most significant digit first
        assert "".join(str(d) for d in reversed(digits)) == np.base_repr(v, 3).zfill(5)
        assert int("".join(str(d) for d in reversed(digits)), 3) == v


def test_element_map_first_160_is_page_stated_chunk_map():
    # chunk c (elements 32c..32c+31) reads digit c of qs[0..31]
    for e in range(160):
        assert oracle.element_slot(e) == (e % 32, e // 32)


def test_element_map_is_a_bijection_onto_used_slots():
    slots = [oracle.element_slot(e) for e in range(256)]
    assert len(set(slots)) == 256
    for e, (b, c) in enumerate(slots):
        assert 0 <= b < 52
        assert 0 <= c < (5 if b < 48 else 4)
        assert oracle.slot_element(b, c) == e
    used = sum(5 if b < 48 else 4 for b in range(52))
    assert used == 256
    # inside every 32-element chunk, consecutive elements sit on consecutive
    # bytes of one digit, or start a new run at the first byte of a field
    for chunk in range(8):
        s = [oracle.element_slot(e) for e in range(32 * chunk, 32 * chunk + 32)]
        for (b0, c0), (b1, c1) in zip(s, s[1:]):
            assert (b1 == b0 + 1 and c1 == c0) or b1 in (0, 32, 48)


def _parse_golden_blocks():
    cases = []
    with open(os.path.join(GOLDEN, "tq1_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, pat, exp = [s.strip() for s in line.split("|")]
            trits = np.zeros(256, dtype=np.int8)
            for tok in pat.split():
                if tok.startswith("all="):
                    trits[:] = int(tok[4:])
                else:
                    e, t = tok[1:].split("=")
                    trits[int(e)] = int(t)
            expect = np.zeros(52, dtype=np.int64)
            for tok in exp.split():
                k, val = tok.split("=")
                if k == "qs*":
                    expect[:48] = int(val)
                elif k == "qh*":
                    expect[48:] = int(val)
                elif k.startswith("qs["):
                    expect[int(k[3:-1])] = int(val)
                elif k.startswith("qh["):
                    expect[48 + int(k[3:-1])] = int(val)
            cases.append((name, trits, expect))
    return cases


@pytest.mark.parametrize("name,trits,expect", _parse_golden_blocks(), ids=lambda v: v if isinstance(v, str) else "")
def test_pack_hand_worked_blocks(name, trits, expect):
    d = np.array([[0x3C00]], dtype=np.uint16)
    w = oracle.tq1_pack(trits.reshape(1, 256), d)
    assert w.shape == (1, 54)
    assert np.array_equal(w[0, :52].astype(np.int64), expect), name
    assert w[0, 52] == 0x00 and w[0, 53] == 0x3C  # little-endian fp16 1.0
    back, dback = oracle.tq1_unpack(w, 1, 256)
    assert np.array_equal(back[0], trits)
    assert dback[0, 0] == 0x3C00


def test_pack_all_byte_values_roundtrip_exhaustive():
    # every qs digit tuple (3^5) in every qs position class and every qh tuple (3^4)
    digits5 = np.array([[int(ch) for ch in reversed(np.base_repr(v, 3).zfill(5))] for v in range(243)])
    digits4 = np.array([[int(ch) for ch in reversed(np.base_repr(v, 3).zfill(4))] for v in range(81)])
    rows = []
    for v in range(243):
        t = np.zeros(256, dtype=np.int8)
        b_lo, b_hi, b_h = v % 32, 32 + v % 16, v % 4
        for c in range(5):
            t[32 * c + b_lo] = digits5[v, c] - 1
            t[160 + 16 * c + (b_hi - 32)] = digits5[v, c] - 1
        for c in range(4):
            t[240 + 4 * c + b_h] = digits4[v % 81, c] - 1
        rows.append(t)
    trits = np.stack(rows)
    d = np.full((243, 1), 0x3C00, dtype=np.uint16)
    w = oracle.tq1_pack(trits, d)
    for v in range(243):
        assert w[v, v % 32] == v
        assert w[v, 32 + v % 16] == v
        assert w[v, 48 + v % 4] == v % 81
    back, _ = oracle.tq1_unpack(w, 243, 256)
    assert np.array_equal(back, trits)
    # unpack -> pack identity on arbitrary valid bytes
    rng = np.random.default_rng(3)
    wb = np.zeros((64, 54), dtype=np.uint8)
    wb[:, :48] = rng.integers(0, 243, (64, 48))
    wb[:, 48:52] = rng.integers(0, 81, (64, 4))
    wb[:, 52:54] = rng.integers(0, 256, (64, 2))
    tr, dd = oracle.tq1_unpack(wb, 64, 256)
    assert np.array_equal(oracle.tq1_pack(tr, dd), wb)


def test_invalid_inputs_rejected():
    t = np.zeros((1, 256), dtype=np.int8)
    t[0, 5] = 2
    with pytest.raises(oracle.OracleError):
        oracle.tq1_pack(t, np.zeros((1, 1), np.uint16))
    w = oracle.tq1_pack(np.zeros((1, 256), np.int8), np.zeros((1, 1), np.uint16))
    bad = w.copy()
    bad[0, 7] = 243
    with pytest.raises(oracle.OracleError):
        oracle.tq1_unpack(bad, 1, 256)
    bad = w.copy()
    bad[0, 50] = 81
    with pytest.raises(oracle.OracleError):
        oracle.tq1_unpack(bad, 1, 256)
    a = oracle.q8_1_quantize(np.ones((1, 256), np.float32))
    with pytest.raises(oracle.OracleError):
        oracle.mmvq(bad, a, 1, 256, 1)
    with pytest.raises(oracle.OracleError):
        oracle.block_isums(bad, a, 1, 256, 1, method="bytes")
    with pytest.raises(oracle.OracleError):
        oracle.mmvq_id(w, a, np.array([[1]], np.int32), 1, 1, 256, 1, 1)


# ---------------------------------------------------------------------------
# Q8_1 quantization: properties that characterize the rule.
# ---------------------------------------------------------------------------

def _q8_fields(x):
    T, K = x.shape
    a = oracle.q8_1_quantize(x)
    q, d16, s16 = oracle.q8_1_fields(a, T, K)
    return a, q.astype(np.int64), d16, s16


def test_q8_1_rule_characterized_on_random_data():
    rng = np.random.default_rng(11)
    x = synth.activations(rng, 4, 2048, outlier_frac=0.01)
    x[0, :32] = 0.0                                   # amax = 0 block
    x[1, 32:64] = np.float32(1e-6) * rng.standard_normal(32).astype(np.float32)  # subnormal fp16 d
    T, K = x.shape
    a, q, d16, s16 = _q8_fields(x)
    xb = x.reshape(T, K // 32, 32)
    qb = q.reshape(T, K // 32, 32)
    amax = np.abs(xb).max(axis=2).astype(np.float32)
    d = (amax / np.float32(127.0)).astype(np.float32)          # IEEE fp32 division
    inv = np.where(d != 0, np.float32(1.0) / np.where(d != 0, d, 1), 0).astype(np.float32)
    v = (xb * inv[:, :, None]).astype(np.float32).astype(np.float64)  # exact product rounded once
    diff = np.abs(v - qb)
    # q is the nearest integer to x/d, ties away from zero, and |q| <= 127
    assert np.all(np.abs(qb) <= 127)
    assert np.all(diff <= 0.5)
    tie = diff == 0.5
    assert np.all(np.abs(qb[tie]) > np.abs(v[tie]))
    # the element of largest magnitude maps to +-127 (unless the block is 0)
    arg = np.abs(xb).argmax(axis=2)
    top = np.take_along_axis(qb, arg[:, :, None], axis=2)[:, :, 0]
    nz = amax > 0
    assert np.all(np.abs(top[nz]) == 127)
    assert np.all(qb[~nz] == 0)
    # stored d and s are the fp16 roundings of d and d * sum(q)
    assert np.array_equal(d16, d.astype(np.float16).view(np.uint16))
    sq = qb.sum(axis=2).astype(np.float32)
    assert np.array_equal(s16, (d * sq).astype(np.float32).astype(np.float16).view(np.uint16))
    # reconstruction error bound |x - d q| <= d/2 (plus fp32 rounding of d)
    err = np.abs(xb.astype(np.float64) - d[:, :, None].astype(np.float64) * qb)
    assert np.all(err <= d[:, :, None].astype(np.float64) * (0.5 + 1e-6) + 1e-30)


def test_q8_1_ties_round_away_from_zero():
    # amax = 127 gives d = 1 and 1/d = 1 exactly, so x * (1/d) = x
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, :8] = [127.0, 2.5, -2.5, 0.5, -0.5, 1.5, -126.5, 3.49999976]
    _, q, d16, s16 = _q8_fields(x)
    assert q[0, :8].tolist() == [127, 3, -3, 1, -1, 2, -127, 3]
    assert d16[0, 0] == 0x3C00
    assert s16[0, 0] == np.float16(127 + 3 - 3 + 1 - 1 + 2 - 127 + 3).view(np.uint16)


# ---------------------------------------------------------------------------
# Integer sums and the mat-vec.
# ---------------------------------------------------------------------------

def _case(N, K, T, seed, p_zero=1 / 3):
    rng = np.random.default_rng(seed)
    trits = synth.ternary(rng, (N, K), p_zero)
    d16 = synth.block_scales_f16(rng, (N, K // 256), 0.01, 0.1)
    x = synth.activations(rng, T, K, outlier_frac=0.01)
    return trits, d16, x


def _isums_numpy(trits, q):
    # int64 contraction per 32-element sub-block, a library routine
    N, K = trits.shape
    T = q.shape[0]
    tb = trits.astype(np.int64).reshape(N, K // 32, 32)
    qb = q.astype(np.int64).reshape(T, K // 32, 32)
    return np.einsum("njk,tjk->tnj", tb, qb)


@pytest.mark.parametrize("N,K,T,seed", [(7, 256, 1, 1), (16, 1024, 3, 2), (5, 2304, 2, 3)])
def test_isums_both_methods_equal_numpy_int_contraction(N, K, T, seed):
    trits, d16, x = _case(N, K, T, seed)
    w = oracle.tq1_pack(trits, d16)
    a = oracle.q8_1_quantize(x)
    q, _, _ = oracle.q8_1_fields(a, T, K)
    ref = _isums_numpy(trits, q)
    assert np.array_equal(oracle.block_isums(w, a, N, K, T, "elem"), ref)
    assert np.array_equal(oracle.block_isums(w, a, N, K, T, "bytes"), ref)


def test_isums_closed_forms():
    K = 512
    rng = np.random.default_rng(5)
    x = synth.activations(rng, 2, K)
    a = oracle.q8_1_quantize(x)
    q, _, _ = oracle.q8_1_fields(a, 2, K)
    sq = q.astype(np.int64).reshape(2, K // 32, 32).sum(axis=2)
    d = np.full((3, 2), 0x3C00, np.uint16)
    trits = np.stack([np.full(K, 1), np.full(K, -1), np.zeros(K)]).astype(np.int8)
    w = oracle.tq1_pack(trits, d)
    for method in ("elem", "bytes"):
        s = oracle.block_isums(w, a, 3, K, 2, method)
        assert np.array_equal(s[:, 0], sq)
        assert np.array_equal(s[:, 1], -sq)
        assert np.all(s[:, 2] == 0)
    # the largest possible sum: q = 127 everywhere against t = +1
    qa = synth.q8_1_blocks_from_fields(np.full((1, K), 127, np.int8),
                                       np.full((1, K // 32), 0x3C00, np.uint16),
                                       np.zeros((1, K // 32), np.uint16))
    for method in ("elem", "bytes"):
        s = oracle.block_isums(w[:1], qa, 1, K, 1, method)
        assert np.all(s == 127 * 32)


@pytest.mark.parametrize("N,K,T,seed", [(9, 256, 1, 10), (32, 1024, 4, 11), (3, 4096, 2, 12)])
def test_mmvq_equals_dequantize_then_dot(N, K, T, seed):
    """Blockwise factorization vs the plain product of dequantized operands."""
    trits, d16, x = _case(N, K, T, seed)
    w = oracle.tq1_pack(trits, d16)
    a = oracle.q8_1_quantize(x)
    q, da16, _ = oracle.q8_1_fields(a, T, K)
    W = trits.astype(np.float64) * np.repeat(d16.view(np.float16).astype(np.float64), 256, axis=1)
    A = q.astype(np.float64) * np.repeat(da16.view(np.float16).astype(np.float64), 32, axis=1)
    ref = A @ W.T                                               # [T, N]
    y, y64, ab = oracle.mmvq(w, a, N, K, T)
    assert np.all(np.abs(y64 - ref) <= 1e-12 * ab + 1e-300)
    assert np.array_equal(y, y64.astype(np.float32))
    # sum |terms| bounds |y| and equals the product of |.| factors when all t >= 0
    assert np.all(np.abs(y64) <= ab * (1 + 1e-12))


def test_mmvq_unit_scales_is_integer_matvec_exactly():
    N, K, T = 24, 1536, 3
    rng = np.random.default_rng(21)
    trits = synth.ternary(rng, (N, K))
    q = rng.integers(-127, 128, (T, K)).astype(np.int8)
    a = synth.q8_1_blocks_from_fields(q, np.full((T, K // 32), 0x3C00, np.uint16),
                                      np.zeros((T, K // 32), np.uint16))
    w = oracle.tq1_pack(trits, np.full((N, K // 256), 0x3C00, np.uint16))
    y, y64, _ = oracle.mmvq(w, a, N, K, T)
    ref = q.astype(np.int64) @ trits.astype(np.int64).T
    assert np.array_equal(y64, ref.astype(np.float64))
    assert np.array_equal(y, ref.astype(np.float32))


def test_mmvq_scale_and_sign_invariants():
    N, K, T = 6, 768, 2
    trits, d16, x = _case(N, K, T, 31)
    a = oracle.q8_1_quantize(x)
    y1, y64, _ = oracle.mmvq(oracle.tq1_pack(trits, d16), a, N, K, T)
    d2 = (d16.view(np.float16).astype(np.float32) * 2).astype(np.float16).view(np.uint16)
    y2, _, _ = oracle.mmvq(oracle.tq1_pack(trits, d2), a, N, K, T)
    assert np.array_equal(y2, 2 * y1)                            # exact power-of-two scaling
    yn, _, _ = oracle.mmvq(oracle.tq1_pack(-trits, d16), a, N, K, T)
    assert np.array_equal(yn, -y1)
    # rows are independent: permuting rows permutes outputs
    perm = np.random.default_rng(1).permutation(N)
    yp, _, _ = oracle.mmvq(oracle.tq1_pack(trits[perm], d16[perm]), a, N, K, T)
    assert np.array_equal(yp, y1[:, perm])


def test_mmvq_add_unit_scales_is_integer_matvec_plus_residual_exactly():
    """Unit scales and an integer residual: y is the int64 product t @ q plus
    r, exactly, with r laid out [T][N] (T != N, so a transposed residual or
    a dropped or negated one fails)."""
    N, K, T = 5, 768, 3
    rng = np.random.default_rng(41)
    trits = synth.ternary(rng, (N, K))
    q = rng.integers(-127, 128, (T, K)).astype(np.int8)
    a = synth.q8_1_blocks_from_fields(q, np.full((T, K // 32), 0x3C00, np.uint16),
                                      np.zeros((T, K // 32), np.uint16))
    w = oracle.tq1_pack(trits, np.full((N, K // 256), 0x3C00, np.uint16))
    r = rng.integers(-5000, 5000, (T, N)).astype(np.float32)
    y, y64, ab = oracle.mmvq_add(w, a, r, N, K, T)
    ref = q.astype(np.int64) @ trits.astype(np.int64).T + r.astype(np.int64)
    assert np.array_equal(y64, ref.astype(np.float64))
    assert np.array_equal(y, ref.astype(np.float32))
    # the tolerance scale: sum |term| over the 32-element sub-block terms
    # (unit scales: |sub-block integer sum|) plus |r|
    prod = trits.astype(np.int64)[None, :, :] * q.astype(np.int64)[:, None, :]
    sub = np.abs(prod.reshape(T, N, K // 32, 32).sum(axis=3)).sum(axis=2)
    assert np.array_equal(ab, sub + np.abs(r))


def test_mmvq_add_zero_residual_is_mmvq():
    N, K, T = 12, 1024, 2
    trits, d16, x = _case(N, K, T, 42)
    w = oracle.tq1_pack(trits, d16)
    a = oracle.q8_1_quantize(x)
    y0, y640, ab0 = oracle.mmvq(w, a, N, K, T)
    y, y64, ab = oracle.mmvq_add(w, a, np.zeros((T, N), np.float32), N, K, T)
    assert np.array_equal(y, y0) and np.array_equal(y64, y640) and np.array_equal(ab, ab0)


def test_mmvq_id_equals_gathered_mmvq():
    E, N, K, T, n_used = 6, 10, 512, 4, 3
    rng = np.random.default_rng(41)
    trits = synth.ternary(rng, (E * N, K))
    d16 = synth.block_scales_f16(rng, (E * N, K // 256), 0.01, 0.1)
    x = synth.activations(rng, T, K)
    ids = synth.zipf_routing(rng, T, E, n_used)
    w = oracle.tq1_pack(trits, d16)
    a = oracle.q8_1_quantize(x)
    y, y64, ab = oracle.mmvq_id(w, a, ids, E, N, K, T, n_used)
    rb = w.reshape(E, N, -1)
    for t in range(T):
        for s in range(n_used):
            yr, yr64, abr = oracle.mmvq(rb[ids[t, s]], a[t:t + 1], N, K, 1)
            assert np.array_equal(y[t, s], yr[0])
            assert np.array_equal(y64[t, s], yr64[0])
            assert np.array_equal(ab[t, s], abr[0])


def test_mmvq_id_slots_equals_dequantize_then_dot():
    """Per-slot activations (one Q8_1 column per (token, slot) pair) against
    numpy's plain product of the dequantized expert matrix and that pair's
    dequantized column, in fp64."""
    E, N, K, T, n_used = 5, 9, 768, 3, 2
    rng = np.random.default_rng(43)
    trits = synth.ternary(rng, (E * N, K))
    d16 = synth.block_scales_f16(rng, (E * N, K // 256), 0.01, 0.1)
    x = synth.activations(rng, T * n_used, K)
    ids = synth.zipf_routing(rng, T, E, n_used)
    w = oracle.tq1_pack(trits, d16)
    a = oracle.q8_1_quantize(x)
    q, da16, _ = oracle.q8_1_fields(a, T * n_used, K)
    W = trits.astype(np.float64) * np.repeat(d16.view(np.float16).astype(np.float64), 256, axis=1)
    A = q.astype(np.float64) * np.repeat(da16.view(np.float16).astype(np.float64), 32, axis=1)
    y, y64, ab = oracle.mmvq_id(w, a, ids, E, N, K, T, n_used, per_slot=True)
    for t in range(T):
        for s in range(n_used):
            e, p = ids[t, s], t * n_used + s
            ref = W[e * N:(e + 1) * N] @ A[p]
            assert np.all(np.abs(y64[t, s] - ref) <= 1e-12 * ab[t, s] + 1e-300)
    assert np.array_equal(y, y64.astype(np.float32))


def test_mmvq_id_slots_with_shared_columns_is_mmvq_id():
    """Repeating each token's column over its slots turns the per-slot
    product into the shared-column one, bit for bit."""
    E, N, K, T, n_used = 4, 7, 512, 3, 3
    rng = np.random.default_rng(44)
    trits = synth.ternary(rng, (E * N, K))
    d16 = synth.block_scales_f16(rng, (E * N, K // 256), 0.01, 0.1)
    x = synth.activations(rng, T, K)
    ids = synth.zipf_routing(rng, T, E, n_used)
    w = oracle.tq1_pack(trits, d16)
    a = oracle.q8_1_quantize(x)
    a_slots = np.repeat(a.reshape(T, 1, -1), n_used, axis=1).reshape(T * n_used, -1)
    y1, y64a, ab1 = oracle.mmvq_id(w, a, ids, E, N, K, T, n_used)
    y2, y64b, ab2 = oracle.mmvq_id(w, a_slots, ids, E, N, K, T, n_used, per_slot=True)
    assert np.array_equal(y64a, y64b) and np.array_equal(ab1, ab2) and np.array_equal(y1, y2)


def test_zipf_routing_has_no_repeats_per_token():
    ids = synth.zipf_routing(np.random.default_rng(0), 64, 128, 8)
    assert ids.shape == (64, 8)
    for row in ids:
        assert len(set(row.tolist())) == 8
    assert ids.min() >= 0 and ids.max() < 128


# ---------------------------------------------------------------------------
# Dequantization and row gather
# ---------------------------------------------------------------------------

def test_bf16_rounding_matches_torch():
    """The oracle's fp32 -> bfloat16 rounding against torch's CPU conversion
    (round to nearest even), on random values, exact ties and neighbours."""
    import torch
    rng = np.random.default_rng(41)
    bits = rng.integers(0, 2**32, 20000, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 2**16, 2000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    x = np.concatenate([bits, ties, ties + 1, ties - 1]).view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < 3e38)]
    got = oracle.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("name,trits,expect", _parse_golden_blocks(), ids=lambda v: v if isinstance(v, str) else "")
def test_dequantize_hand_worked_blocks(name, trits, expect):
    """Pack the hand-worked blocks with a scale of -1.5 and dequantize: every
    element is -1.5 * trit (fp16 -1.5 = 0xBE00)."""
    w = oracle.tq1_pack(trits.reshape(1, 256), np.array([[0xBE00]], np.uint16))
    v = oracle.tq1_dequantize(w, 1, 256, "f32")
    assert np.array_equal(v[0], np.float32(-1.5) * trits.astype(np.float32)), name
    # a zero trit under a negative scale is the fp32 product, -0
    zeros = trits == 0
    assert np.all(np.signbit(v[0][zeros]))


def test_dequantize_then_dot_is_the_unit_scale_mat_vec():
    """Dequantized weights times integer activations equal the oracle mat-vec
    with unit activation scales (itself pinned to the integer mat-vec)."""
    N, K, T = 20, 1280, 3
    rng = np.random.default_rng(43)
    trits = synth.ternary(rng, (N, K))
    d16 = synth.block_scales_f16(rng, (N, K // 256), 0.01, 0.1)
    w = oracle.tq1_pack(trits, d16)
    q = rng.integers(-127, 128, (T, K)).astype(np.int8)
    a = synth.q8_1_blocks_from_fields(q, np.full((T, K // 32), 0x3C00, np.uint16),
                                      np.zeros((T, K // 32), np.uint16))
    _, y64, ab = oracle.mmvq(w, a, N, K, T)
    W = oracle.tq1_dequantize(w, N, K, "f32").astype(np.float64)
    ref = q.astype(np.float64) @ W.T
    assert np.all(np.abs(ref - y64) <= 1e-12 * ab + 1e-300)


def test_dequantize_dtypes_and_row_gather():
    N, K = 7, 768
    rng = np.random.default_rng(44)
    trits = synth.ternary(rng, (N, K))
    d16 = synth.block_scales_f16(rng, (N, K // 256), 0.01, 0.1)
    d16[3, 1] = 0xB800                      # a negative scale (-0.5)
    w = oracle.tq1_pack(trits, d16)
    f32 = oracle.tq1_dequantize(w, N, K, "f32")
    assert np.array_equal(oracle.tq1_dequantize(w, N, K, "f16"),
                          f32.astype(np.float16).view(np.uint16))
    assert np.array_equal(oracle.tq1_dequantize(w, N, K, "bf16"), oracle.f32_to_bf16_bits(f32))
    rows = np.array([6, 0, 3, 3, 1], np.int32)
    for dt in ("f32", "f16", "bf16"):
        full = oracle.tq1_dequantize(w, N, K, dt)
        assert np.array_equal(oracle.tq1_dequantize(w, N, K, dt, rows=rows), full[rows])
    with pytest.raises(oracle.OracleError):
        oracle.tq1_dequantize(w, N, K, "f32", rows=np.array([0, 7], np.int32))


# ---------------------------------------------------------------------------
# TQ2_0: the 2-bit layout read from "Upstream state" (the page names the type
# and prints no layout; the reading is stated in tests/golden/tq2_blocks.txt).
# ---------------------------------------------------------------------------

def test_tq2_element_map_is_a_bijection_and_agrees_with_tq1_first_chunks():
    slots = [oracle.tq2_element_slot(e) for e in range(256)]
    assert len(set(slots)) == 256
    assert all(0 <= b < 64 and 0 <= f < 4 for b, f in slots)
    # the first four 32-element chunks sit where TQ1_0 puts them (byte e % 32,
    # digit / field e / 32), and chunk c + 4 is chunk c moved 32 bytes on
    for e in range(128):
        assert oracle.tq2_element_slot(e) == oracle.element_slot(e)
        b, f = oracle.tq2_element_slot(e + 128)
        assert (b - 32, f) == oracle.element_slot(e)


def _parse_tq2_golden():
    cases = []
    with open(os.path.join(GOLDEN, "tq2_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, pat, exp = [s.strip() for s in line.split("|")]
            trits = np.zeros(256, dtype=np.int8)
            for tok in pat.split():
                if tok.startswith("all="):
                    trits[:] = int(tok[4:])
                else:
                    e, t = tok[1:].split("=")
                    trits[int(e)] = int(t)
            expect = np.zeros(64, dtype=np.int64)
            for tok in exp.split():
                k, val = tok.split("=")
                if k == "qs*":
                    expect[:] = int(val)
                else:
                    expect[int(k[3:-1])] = int(val)
            cases.append((name, trits, expect))
    return cases


@pytest.mark.parametrize("name,trits,expect", _parse_tq2_golden(), ids=lambda v: v if isinstance(v, str) else "")
def test_tq2_pack_hand_worked_blocks(name, trits, expect):
    w = oracle.tq2_pack(trits.reshape(1, 256), np.array([[0xBC00]], np.uint16))
    assert w.shape == (1, 66)
    assert np.array_equal(w[0, :64].astype(np.int64), expect), name
    assert w[0, 64] == 0x00 and w[0, 65] == 0xBC  # little-endian fp16 -1.0
    back, dback = oracle.tq2_unpack(w, 1, 256)
    assert np.array_equal(back[0], trits)
    assert dback[0, 0] == 0xBC00


def test_tq2_every_valid_byte_roundtrips_and_field_3_is_rejected():
    # the 81 bytes whose four fields are digits, at every byte position
    vals = [v for v in range(256) if all((v >> (2 * f)) & 3 != 3 for f in range(4))]
    assert len(vals) == 81
    rows = np.zeros((81, 64), np.uint8)
    for i, v in enumerate(vals):
        rows[i, :] = v
    w = np.concatenate([rows, np.zeros((81, 2), np.uint8)], axis=1)
    trits, d = oracle.tq2_unpack(w, 81, 256)
    assert np.array_equal(oracle.tq2_pack(trits, d), w)
    # all 256 trits of a block decode from digits 0..2, so each byte's four
    # trits are base-4 digits of v - 85 shifted: sum_f (t_f + 1) 4^f = v
    for i, v in enumerate(vals):
        for p in (0, 17, 40, 63):
            s = sum((int(trits[i, 128 * (p // 32) + 32 * f + p % 32]) + 1) * 4 ** f
                    for f in range(4))
            assert s == v
    for v in (3, 12, 48, 192, 255):
        bad = w[:1].copy()
        bad[0, 9] = v
        with pytest.raises(oracle.OracleError):
            oracle.tq2_unpack(bad, 1, 256)
        a = oracle.q8_1_quantize(np.ones((1, 256), np.float32))
        with pytest.raises(oracle.OracleError):
            oracle.tq2_mmvq(bad, a, 1, 256, 1)
        for method in ("elem", "bytes"):
            with pytest.raises(oracle.OracleError):
                oracle.tq2_block_isums(bad, a, 1, 256, 1, method)
    t = np.zeros((1, 256), np.int8)
    t[0, 77] = -2
    with pytest.raises(oracle.OracleError):
        oracle.tq2_pack(t, np.zeros((1, 1), np.uint16))


@pytest.mark.parametrize("N,K,T,seed", [(7, 256, 1, 61), (16, 1024, 3, 62), (5, 2304, 2, 63)])
def test_tq2_isums_both_methods_equal_numpy_int_contraction(N, K, T, seed):
    trits, d16, x = _case(N, K, T, seed)
    w = oracle.tq2_pack(trits, d16)
    a = oracle.q8_1_quantize(x)
    q, _, _ = oracle.q8_1_fields(a, T, K)
    ref = _isums_numpy(trits, q)
    assert np.array_equal(oracle.tq2_block_isums(w, a, N, K, T, "elem"), ref)
    assert np.array_equal(oracle.tq2_block_isums(w, a, N, K, T, "bytes"), ref)


@pytest.mark.parametrize("N,K,T,seed", [(9, 256, 1, 64), (32, 1024, 4, 65), (3, 4096, 2, 66)])
def test_tq2_mmvq_equals_tq1_mmvq_of_the_same_trits(N, K, T, seed):
    """One matrix, two packings: both products sum the same exact terms in
    the same order, so they agree bit for bit; and both match the plain
    product of dequantized operands."""
    trits, d16, x = _case(N, K, T, seed)
    a = oracle.q8_1_quantize(x)
    y1, y1_64, ab1 = oracle.mmvq(oracle.tq1_pack(trits, d16), a, N, K, T)
    y2, y2_64, ab2 = oracle.tq2_mmvq(oracle.tq2_pack(trits, d16), a, N, K, T)
    assert np.array_equal(y2_64, y1_64) and np.array_equal(ab2, ab1)
    assert np.array_equal(y2, y1)
    q, da16, _ = oracle.q8_1_fields(a, T, K)
    W = trits.astype(np.float64) * np.repeat(d16.view(np.float16).astype(np.float64), 256, axis=1)
    A = q.astype(np.float64) * np.repeat(da16.view(np.float16).astype(np.float64), 32, axis=1)
    assert np.all(np.abs(y2_64 - A @ W.T) <= 1e-12 * ab2 + 1e-300)


def test_tq2_mmvq_unit_scales_is_integer_matvec_exactly():
    N, K, T = 24, 1536, 3
    rng = np.random.default_rng(67)
    trits = synth.ternary(rng, (N, K))
    q = rng.integers(-127, 128, (T, K)).astype(np.int8)
    a = synth.q8_1_blocks_from_fields(q, np.full((T, K // 32), 0x3C00, np.uint16),
                                      np.zeros((T, K // 32), np.uint16))
    w = oracle.tq2_pack(trits, np.full((N, K // 256), 0x3C00, np.uint16))
    y, y64, _ = oracle.tq2_mmvq(w, a, N, K, T)
    ref = q.astype(np.int64) @ trits.astype(np.int64).T
    assert np.array_equal(y64, ref.astype(np.float64))
    assert np.array_equal(y, ref.astype(np.float32))


def test_tq2_mmvq_scale_index_and_row_order():
    """A scale change in one block moves only that block's terms; permuted
    rows permute the outputs."""
    N, K, T = 6, 768, 2
    trits, d16, x = _case(N, K, T, 68)
    a = oracle.q8_1_quantize(x)
    _, y64, _ = oracle.tq2_mmvq(oracle.tq2_pack(trits, d16), a, N, K, T)
    d2 = d16.copy()
    d2[2, 1] = 0
    _, z64, _ = oracle.tq2_mmvq(oracle.tq2_pack(trits, d2), a, N, K, T)
    t0 = trits.copy()
    t0[2, 256:512] = 0
    _, r64, _ = oracle.tq2_mmvq(oracle.tq2_pack(t0, d16), a, N, K, T)
    assert np.array_equal(z64, r64)
    assert not np.array_equal(z64[:, 2], y64[:, 2])
    perm = np.random.default_rng(2).permutation(N)
    _, p64, _ = oracle.tq2_mmvq(oracle.tq2_pack(trits[perm], d16[perm]), a, N, K, T)
    assert np.array_equal(p64, y64[:, perm])


# The logistic function sigma(x) = e^x / (1 + e^x) at x = 1 and 2, with
# e = 2.718281828459045: e / (1 + e) and e^2 / (1 + e^2). silu(x) = x sigma(x),
# and sigma(-x) = 1 - sigma(x).
SIGMA_1 = 0.7310585786300049
SIGMA_2 = 0.8807970779778823


def test_mmvq_glu_unit_scales_against_logistic_values():
    """Unit scales and an all-ones activation column make the gate and up
    products small integers g, u (g ones or minus ones in the gate row, u in
    the up row); y = silu(g) * u is checked against the logistic function's
    values, silu(0) = 0, silu(40) = 40 in fp64 and silu(-40) ~ -40 e^-40. The
    gate and up rows differ, so swapped operands or a dropped factor fail."""
    K, T = 256, 1
    cases = [(1, 2), (2, 1), (-1, 3), (2, -1), (0, 5), (-2, -2), (40, 1), (-40, 1), (3, 0)]
    N = len(cases)
    gate = np.zeros((N, K), np.int8)
    up = np.zeros((N, K), np.int8)
    for n, (g, u) in enumerate(cases):
        gate[n, :abs(g)] = np.sign(g)
        up[n, :abs(u)] = np.sign(u)
    unit = np.full((N, K // 256), 0x3C00, np.uint16)
    wg, wu = oracle.tq1_pack(gate, unit), oracle.tq1_pack(up, unit)
    a = synth.q8_1_blocks_from_fields(np.ones((T, K), np.int8),
                                      np.full((T, K // 32), 0x3C00, np.uint16),
                                      np.zeros((T, K // 32), np.uint16))
    y, y64, g64, u64, absg, absu = oracle.mmvq_glu(wg, wu, a, N, K, T)
    assert g64[0].tolist() == [float(c[0]) for c in cases]
    assert u64[0].tolist() == [float(c[1]) for c in cases]
    assert absg[0].tolist() == [float(abs(c[0])) for c in cases]
    expect = [SIGMA_1 * 2, 2 * SIGMA_2, -(1 - SIGMA_1) * 3, -2 * SIGMA_2, 0.0,
              -2 * (1 - SIGMA_2) * -2, 40.0, -40 * np.exp(-40.0), 0.0]
    assert np.allclose(y64[0], expect, rtol=1e-13, atol=0)
    assert y64[0, 4] == 0.0 and y64[0, 6] == 40.0
    assert np.array_equal(y, y64.astype(np.float32))


def test_mmvq_glu_products_are_the_two_matvecs():
    N, K, T = 9, 1024, 2
    tg, d16g, x = _case(N, K, T, 51)
    tu, d16u, _ = _case(N, K, T, 52)
    wg, wu = oracle.tq1_pack(tg, d16g), oracle.tq1_pack(tu, d16u)
    a = oracle.q8_1_quantize(x)
    y, y64, g64, u64, absg, absu = oracle.mmvq_glu(wg, wu, a, N, K, T)
    _, gy64, gab = oracle.mmvq(wg, a, N, K, T)
    _, uy64, uab = oracle.mmvq(wu, a, N, K, T)
    assert np.array_equal(g64, gy64) and np.array_equal(absg, gab)
    assert np.array_equal(u64, uy64) and np.array_equal(absu, uab)
