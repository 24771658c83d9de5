"""CPU check of the integer arithmetic the gfx950 kernels use to expand
base-3 digits (bit_quantized_mat_amd/csrc/tq1_decode.hpp): the multiply-shift
constants are read from the header and the two-bytes-per-register lane
arithmetic is emulated for every qs byte (0..242) and qh byte (0..80), against
Python's own integer division."""
import os
import re

import numpy as np

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "bit_quantized_mat_amd", "csrc", "tq1_decode.hpp")


def _constants():
    text = open(HDR).read()
    def get(name):
        m = re.search(r"\b%s\s*=\s*(\d+)u(?:\s*\*\s*0x00010001u)?" % name, text)
        assert m, name
        return int(m.group(1))
    return {k: get(k) for k in ("kQsMul", "kQsAdd", "kQsShift", "kQhMul", "kQhAdd", "kQhShift")}


C = _constants()
M16 = 0xFFFF


def _lane_chain(v, mul, add, shift, mults):
    """Emulate one 16-bit lane: X1 = (mul*v + add) >> shift, then X1 * m."""
    x1 = (mul * v + add) & M16
    assert mul * v + add <= M16, "lane overflow in the first product"
    x1 >>= shift
    xs = [x1]
    for m in mults:
        assert x1 * m <= M16, "lane overflow"
        xs.append((x1 * m) & M16)
    return xs


def test_qs_digit_chain_exhaustive():
    for v in range(243):
        x1, x2, x3, x4 = _lane_chain(v, C["kQsMul"], C["kQsAdd"], C["kQsShift"], (3, 9, 27))
        floors = [(x >> 8) & 0xFF for x in (x1, x2, x3, x4)]
        assert floors == [v // 81, v // 27, v // 9, v // 3], v
        # the lowest digit as the byte's value minus 3 floor(v / 3), which
        # never goes below zero (no borrow into the next byte of the dword)
        assert 0 <= v - 3 * floors[3] == v % 3, v
        # the unsigned digits recovered as F_m - 3 F_(m+1) match base 3
        f = [v // 3 ** m for m in range(6)]
        digits = [f[m] - 3 * f[m + 1] for m in range(5)]
        assert int("".join(str(d) for d in reversed(digits)), 3) == v


def test_qh_digit_chain_exhaustive():
    for v in range(81):
        x1, x2, x3 = _lane_chain(v, C["kQhMul"], C["kQhAdd"], C["kQhShift"], (3, 9))
        floors = [(x >> 8) & 0xFF for x in (x1, x2, x3)]
        assert floors == [v // 27, v // 9, v // 3], v
        assert 0 <= v - 3 * floors[2] == v % 3, v


def _qh_lane_multipliers():
    """The per-lane multipliers 3^(3-c) of qh_lane_muls, read from the header."""
    text = open(HDR).read()
    m = re.search(r"c == 0 \? (\d+)u : c == 1 \? (\d+)u : c == 2 \? (\d+)u : (\d+)u", text)
    assert m, "qh_lane_muls"
    return [int(g) for g in m.groups()]


def test_qh_lane_digit_exhaustive():
    # qh_digit_lane: digit c of a qh byte from F_c - 3 F_(c+1), where F_m is
    # byte 1 of X1 * 3^(3-m) and the next multiplier is the current one / 3
    # (0 for c = 3)
    muls = _qh_lane_multipliers()
    assert muls == [27, 9, 3, 1]
    for v in range(81):
        (x1,) = _lane_chain(v, C["kQhMul"], C["kQhAdd"], C["kQhShift"], ())
        for c in range(4):
            cur, nxt = muls[c], muls[c] // 3
            assert x1 * cur <= M16 and x1 * nxt <= M16
            fc = ((x1 * cur) >> 8) & 0xFF
            fn = ((x1 * nxt) >> 8) & 0xFF
            assert fc == v // 3 ** c and fn == (v // 3 ** (c + 1) if c < 3 else 0), (v, c)
            assert 3 * fn <= fc and fc - 3 * fn == (v // 3 ** c) % 3, (v, c)


def test_two_lanes_share_a_register_without_crosstalk():
    # the first step is one 24-bit multiply-add on bytes 0 and 2 of a dword
    rng = np.random.default_rng(0)
    for _ in range(2000):
        b0, b2 = (int(t) for t in rng.integers(0, 243, 2))
        e = b0 | (b2 << 16)
        r = (e * C["kQsMul"] + C["kQsAdd"] * 0x00010001) & 0xFFFFFFFF
        assert e < (1 << 24)
        assert r & M16 == C["kQsMul"] * b0 + C["kQsAdd"]
        assert r >> 16 == C["kQsMul"] * b2 + C["kQsAdd"]


def _perm(s0, s1, sel):
    """v_perm_b32: selector bytes 0-3 pick bytes of s1, 4-7 bytes of s0, 12 -> 0."""
    src = [(s1 >> (8 * i)) & 0xFF for i in range(4)] + [(s0 >> (8 * i)) & 0xFF for i in range(4)]
    out = 0
    for i in range(4):
        s = (sel >> (8 * i)) & 0xFF
        b = src[s] if s < 8 else (0 if s == 12 else 0xFF)
        out |= b << (8 * i)
    return out


def test_byte_split_and_merge_selectors():
    w = 0x44332211
    assert w & 0x00FF00FF == 0x00330011
    assert _perm(0, w, 0x0C030C01) == 0x00440022          # bytes 1, 3 into lanes
    e, o = 0xAA01BB02, 0xCC03DD04                          # byte 1/3 of each lane
    assert _perm(o, e, 0x07030501) == 0xCCAADDBB          # [e.b1, o.b1, e.b3, o.b3]


def test_single_level_digit_extraction_exhaustive():
    """Dequantization extracts one digit level per lane: floor(v / 3^c) is
    byte 1 of X1 * 3^(k - c) in each 16-bit lane (k = 4 for qs bytes, 3 for
    qh), and the digit is that floor minus 3 times the next one. Every byte
    value, every level, against Python's base-3 digits."""
    for qh, nbytes_max, k in ((False, 243, 4), (True, 81, 3)):
        mul = C["kQhMul"] if qh else C["kQsMul"]
        add = C["kQhAdd"] if qh else C["kQsAdd"]
        shift = C["kQhShift"] if qh else C["kQsShift"]
        for v in range(nbytes_max):
            x1 = ((mul * v + add) & M16) >> shift
            for c in range(k + 1):
                m_c = 3 ** (k - c)
                m_n = 3 ** (k - c - 1) if c + 1 <= k else 0
                assert x1 * m_c <= M16
                f_c = ((x1 * m_c) & M16) >> 8
                f_n = ((x1 * m_n) & M16) >> 8
                assert f_c == v // 3 ** c, (qh, v, c)
                assert f_c - 3 * f_n == (v // 3 ** c) % 3, (qh, v, c)


DEQ = os.path.join(os.path.dirname(HDR), "dequant.hip")


def _dequant_level_multipliers():
    """The multipliers 3^p of level_consts in dequant.hip, read from the source."""
    text = open(DEQ).read()
    m = re.search(r"p == 0 \? (\d+)u : p == 1 \? (\d+)u : p == 2 \? (\d+)u : (\d+)u", text)
    assert m, "level_consts"
    return [int(g) for g in m.groups()]


def test_dequant_digit_from_low_byte_exhaustive():
    # digit_lanes in dequant.hip: below the top level c < k, the digit is byte 1
    # of 3 * ((X1 * 3^(k-c-1)) & 0xff) (mod 2^16 per lane); at c = k, byte 1 of
    # X1. Checked for every qs byte (k = 4) and qh byte (k = 3) at every level
    # against Python's base-3 digits.
    pw = _dequant_level_multipliers()
    assert pw == [1, 3, 9, 27]
    for k, n, mul, add, shift in ((4, 243, C["kQsMul"], C["kQsAdd"], C["kQsShift"]),
                                   (3, 81, C["kQhMul"], C["kQhAdd"], C["kQhShift"])):
        for v in range(n):
            (x1,) = _lane_chain(v, mul, add, shift, ())
            for c in range(k + 1):
                p = k - c - 1
                if p < 0:
                    y = x1
                else:
                    x = (x1 * pw[p]) & M16
                    y = ((x & 0xFF) * 3) & M16
                assert (y >> 8) & 0xFF == (v // 3 ** c) % 3, (k, v, c)
