"""The allocation-free expert-routed entry point (mmvq_id_tq1_0_noalloc)
against the allocating one (mmvq_id_tq1_0), through the C ABI: two calls in
a row that both route through the library's device scratch, the second
smaller than the first, then one routed inside the wave; every output bitwise
equal, and the smaller call also against the oracle."""
import sys

import numpy as np
import pytest

import oracle
from bit_quantized_mat_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _inputs(E, N, K, T, n_used, seed):
    rng = np.random.default_rng(seed)
    trits = synth.ternary(rng, (E * N, K))
    d16 = synth.block_scales_f16(rng, (E * N, K // 256), 0.01, 0.1)
    x = synth.activations(rng, T, K)
    ids = synth.zipf_routing(rng, T, E, n_used)
    return trits, d16, x, ids


def test_noalloc_equals_workspace_call():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_mat_amd as bqm
    bqm.library()
    # (E, N, K, T, n_used): 512 pairs over 128 experts (pre-pass, narrow and
    # matrix-core items), then 160 pairs over 20 experts (pre-pass again, on
    # the scratch the first call left behind), then 24 pairs (routed in the
    # wave: the scratch is not used)
    cases = [(128, 1536, 4096, 64, 8, 1), (20, 100, 4096, 40, 4, 2), (6, 40, 512, 8, 3, 3)]
    for (E, N, K, T, n_used, seed) in cases:
        print("noalloc case", E, N, K, T, n_used, file=sys.stderr, flush=True)
        trits, d16, x, ids = _inputs(E, N, K, T, n_used, seed)
        w = bqm.tq1_pack(_dev(trits), _dev(d16.view(np.int16)))
        a = bqm.q8_1_quantize(_dev(x))
        ids_d = _dev(ids)
        ref = _host(bqm.mmvq_id_tq1_0(w, a, ids_d, E, N, K, T, n_used))
        out = torch.full((T, n_used, N), float("nan"), dtype=torch.float32, device=w.device)
        got = _host(bqm.mmvq_id_tq1_0_noalloc(w, a, ids_d, E, N, K, T, n_used, out=out))
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (E, T, n_used)
        if E * N <= 4096:
            w_ref = oracle.tq1_pack(trits, d16)
            a_ref = oracle.q8_1_quantize(x)
            _, y64, ab = oracle.mmvq_id(w_ref, a_ref, ids, E, N, K, T, n_used)
            err = np.abs(got.astype(np.float64) - y64)
            assert np.all(err <= 1e-5 * ab)
