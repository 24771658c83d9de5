"""Seeded synthetic inputs for the TQ1_0 x Q8_1 mat-vec.

This module only draws random inputs (ternary weights, fp16 block scales,
fp32 activations, expert ids) and lays given fields out in the block byte
layouts. It holds none of the method's arithmetic: no packing, no
quantization, no products. Both the CPU oracle and the HIP path take their
inputs from here, so neither has to trust the other's data.

Draw order per workload: weights' trits, then block scales (one generator),
activations (second generator), expert ids (third generator). A sweep over T
draws the widest T once; narrower T uses the leading columns, so every
narrower input is a prefix of the wider one.

The workloads follow the shapes the pages measure on: a 4096 x 4096 decode
mat-vec, the N=5120 / K=6144 shape and its 1,2,3,4,5,8 column widths ("ops::linear
q5: one Capacity=32 K-split rung ..." and "cuda: opt-in MMVQ activation reuse
across output rows"), and a Zipf-routed MoE with weights drawn distinctly per
expert ("tools: add mmq-tune ...", section "How the measurement is set up").
"""
from dataclasses import dataclass, field
from typing import Tuple

import numpy as np

TQ1_BLOCK = 256
Q81_BLOCK = 32


@dataclass(frozen=True)
class Workload:
    name: str
    N: int
    K: int
    Ts: Tuple[int, ...]
    p_zero: float = 1.0 / 3.0          # probability of trit 0; +-1 share the rest
    d_lo: float = 0.01                 # block scale ~ U[d_lo, d_hi] (fp32 draw, then fp16)
    d_hi: float = 0.1
    outlier_frac: float = 0.0          # fraction of activation entries scaled by outlier_scale
    outlier_scale: float = 20.0
    seeds: Tuple[int, ...] = (0, 0)    # (weights, activations[, ids, per-slot activations])
    experts: int = 0                   # > 0: MoE with this many experts
    n_used: int = 0                    # experts per token
    zipf_s: float = 1.1
    note: str = field(default="", compare=False)


WORKLOADS = {
    "tiny": Workload("tiny", N=256, K=1024, Ts=(1,), seeds=(101, 102),
                     note="tiny mat-vec, 4 blocks per row"),
    "decode": Workload("decode", N=4096, K=4096, Ts=(1,), seeds=(201, 202),
                       note="decode-shaped mat-vec"),
    "multicol": Workload("multicol", N=5120, K=6144, Ts=(1, 2, 3, 4, 5, 8), seeds=(301, 302),
                         note="multi-column activation reuse"),
    "ffn": Workload("ffn", N=14336, K=4096, Ts=(1, 2, 4, 8, 16, 32), p_zero=0.4,
                    d_lo=0.005, d_hi=0.05, outlier_frac=0.01, seeds=(401, 402),
                    note="FFN-shaped small batch with 1% x20 activation outliers"),
    "moe": Workload("moe", N=1536, K=4096, Ts=(1, 8, 64), seeds=(501, 502, 503, 504),
                    experts=128, n_used=8, note="MoE expert-routed mat-vec, top-8 Zipf(1.1)"),
}


def ternary(rng, shape, p_zero=1.0 / 3.0):
    """int8 trits in {-1, 0, +1}; P(0) = p_zero, P(-1) = P(+1) = (1 - p_zero) / 2."""
    if abs(p_zero - 1.0 / 3.0) < 1e-12:
        return (rng.integers(0, 3, size=shape, dtype=np.int8) - 1).astype(np.int8)
    u = rng.random(shape, dtype=np.float32)
    lo = np.float32((1.0 - p_zero) / 2.0)
    hi = np.float32(lo + p_zero)
    return ((u >= lo).astype(np.int8) + (u >= hi).astype(np.int8) - 1).astype(np.int8)


def block_scales_f16(rng, shape, lo, hi):
    """fp16 bit patterns of scales drawn U[lo, hi] in fp32 and rounded to fp16."""
    d = rng.uniform(lo, hi, size=shape).astype(np.float32)
    return d.astype(np.float16).view(np.uint16)


def activations(rng, T, K, outlier_frac=0.0, outlier_scale=20.0):
    """fp32 [T, K] standard normal; each entry independently scaled by
    outlier_scale with probability outlier_frac."""
    x = rng.standard_normal((T, K), dtype=np.float32)
    if outlier_frac > 0:
        mask = rng.random((T, K)) < outlier_frac
        x[mask] *= np.float32(outlier_scale)
    return x


def zipf_routing(rng, T, E, n_used, s=1.1):
    """int32 [T, n_used] expert ids: ranks drawn without repeats per token with
    weight rank^-s over a seeded permutation of the experts; the order of the
    draws is the slot order."""
    perm = rng.permutation(E)
    w = np.arange(1, E + 1, dtype=np.float64) ** (-s)
    p = w / w.sum()
    ids = np.empty((T, n_used), dtype=np.int32)
    for t in range(T):
        ids[t] = perm[rng.choice(E, size=n_used, replace=False, p=p)]
    return ids


@dataclass
class Inputs:
    workload: Workload
    trits: np.ndarray        # int8 [N, K] or [E*N, K] for MoE (expert-major)
    d16: np.ndarray          # uint16 [N, K/256] or [E*N, K/256]
    x: np.ndarray            # float32 [Tmax, K]
    ids: np.ndarray = None   # int32 [Tmax, n_used] for MoE


def make_inputs(wl: Workload, T: int = None, N: int = None, K: int = None, E: int = None):
    """Draw the workload's inputs. N, K, E may be overridden to shrink a case
    (same recipe, smaller shape); T defaults to the widest of the sweep."""
    N = wl.N if N is None else N
    K = wl.K if K is None else K
    T = max(wl.Ts) if T is None else T
    E = (wl.experts if E is None else E) if wl.experts else 0
    rows = N * E if E else N
    rng_w = np.random.default_rng(wl.seeds[0])
    trits = ternary(rng_w, (rows, K), wl.p_zero)
    d16 = block_scales_f16(rng_w, (rows, K // TQ1_BLOCK), wl.d_lo, wl.d_hi)
    rng_a = np.random.default_rng(wl.seeds[1])
    x = activations(rng_a, T, K, wl.outlier_frac, wl.outlier_scale)
    ids = None
    if E:
        rng_i = np.random.default_rng(wl.seeds[2])
        ids = zipf_routing(rng_i, T, E, wl.n_used, wl.zipf_s)
    return Inputs(wl, trits, d16, x, ids)


def slot_activations(wl: Workload, T: int = None, K: int = None):
    """One fp32 activation column per (token, slot) pair of an MoE workload,
    float32 [T * n_used, K], for the per-slot product (the down-projection
    shape); same law as the workload's token activations, own seed."""
    K = wl.K if K is None else K
    T = max(wl.Ts) if T is None else T
    rng = np.random.default_rng(wl.seeds[3])
    return activations(rng, T * wl.n_used, K, wl.outlier_frac, wl.outlier_scale)


def q8_1_blocks_from_fields(q, d16, s16):
    """Lay out given Q8_1 fields as 36-byte blocks: int8 q[32], fp16 d, fp16 s.

    q int8 [T, K]; d16, s16 uint16 [T, K/32]. Used to hand-build activations
    with exact unit scales; nothing is computed here."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    T, K = q.shape
    nb = K // Q81_BLOCK
    out = np.empty((T, nb, 36), dtype=np.uint8)
    out[:, :, :32] = q.reshape(T, nb, 32).view(np.uint8)
    out[:, :, 32:34] = np.ascontiguousarray(d16, dtype=np.uint16).reshape(T, nb, 1).view(np.uint8)
    out[:, :, 34:36] = np.ascontiguousarray(s16, dtype=np.uint16).reshape(T, nb, 1).view(np.uint8)
    return out.reshape(T, nb * 36)
