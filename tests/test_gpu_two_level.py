"""Two-level group scales on the device (a power of two per (chunk, head)
times the E4M3 group scale), against the oracle through the C ABI: the
second-level exponents, codes, scales and centroids bit for bit, and the
decode (both decode kernels) of the result."""
import numpy as np
import pytest

import oracle
import synthkv
from gpu_util import check_chunk, fetch, gcfg, gpu_encode_chunks, lib, ocfg, say, to_np


def _values(heads, n, boost):
    """Value rows of the single-head workload, scaled by a power of two so that
    residual groups exceed E4M3's range (exact in bf16)."""
    return synthkv.gen_numpy(synthkv.PRESETS[2], "V", heads=heads, n_tokens=n) * np.float32(boost)


pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,boost,dtype", [(2, 8.0, "bf16"), (0, 1.0, "bf16"), (5, 512.0, "bf16"), (1, 4.0, "f32")])
def test_two_level_encode_and_decode_match_oracle(T, boost, dtype):
    say(f"two-level scales T={T} boost={boost} {dtype}")
    p = synthkv.PRESETS[2]
    oc = ocfg(p, "V", n_stages=T, n_centroids=64, iters_cold=3, iters_warm=2, scale_mode="two_level", dtype=dtype)
    X = _values(2, 2000, boost)
    if dtype == "bf16":
        X = oracle.bf16_round(X).astype(np.float32)
    dst, _ = gpu_encode_chunks(oc, X, 1000)
    q = lib()
    y = to_np(q.decode(gcfg(oc), dst, 0, 2000, out_dtype="f32"))
    cache, any_f = {}, 0
    for c in range(2):
        b, e = c * 1000, (c + 1) * 1000
        g = fetch(dst, c, oc)
        for h in range(2):
            ora = oracle.encode_chunk(X[h:h + 1, b:e], oc, cache=cache.get(h), head_offset=h)
            cache[h] = ora.cache
            assert int(g["scale_exp"][h]) == int(ora.scale_exp[0])
            any_f = max(any_f, int(ora.scale_exp[0]))
            if T:
                assert check_chunk(oc, X[:, b:e], g, ora, 0, h, f"chunk {c}") == 0
            else:
                np.testing.assert_array_equal(g["codes"][h], ora.codes[0])
                np.testing.assert_array_equal(g["scales"][h], ora.scales[0])
            np.testing.assert_array_equal(y[h, b:e], oracle.decode(ora, oc.group_size, "f32")[0])
    say(f"  largest second-level exponent {any_f}")
    if boost > 1:
        assert any_f >= 1


def test_saturating_groups_error_report():
    """Printed: on boosted value rows, the worst error inside groups that would
    saturate, and the MSE, with and without the second level."""
    p = synthkv.PRESETS[2]
    X = oracle.bf16_round(_values(2, 4680, 8.0)).astype(np.float32)
    q = lib()
    res = {}
    for mode in ("e4m3", "two_level"):
        oc = ocfg(p, "V", scale_mode=mode, iters_cold=4)
        dst, _ = gpu_encode_chunks(oc, X, 4680)
        res[mode] = to_np(q.decode(gcfg(oc), dst, 0, 4680, out_dtype="f32"))
    err0 = np.abs(res["e4m3"] - X)
    err2 = np.abs(res["two_level"] - X)
    sat = err0.reshape(2, 4680, -1, 64).max(axis=3) > 224          # groups whose error exceeds the step 448 / 2
    say(f"  groups with saturation-sized errors: {int(sat.sum())}; worst error there "
        f"{err0.reshape(2, 4680, -1, 64).max(axis=3)[sat].max() if sat.any() else 0:.4g} -> "
        f"{err2.reshape(2, 4680, -1, 64).max(axis=3)[sat].max() if sat.any() else 0:.4g}; "
        f"MSE {oracle.mse(res['e4m3'], X):.4g} -> {oracle.mse(res['two_level'], X):.4g}")
    assert err2.max() <= err0.max()
