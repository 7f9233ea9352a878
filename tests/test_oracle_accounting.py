"""Closed-form byte accounting: the memory formula, the per-chunk byte counts
and compression ratios, checked against actual array sizes and the pages'
round-to-nearest figure."""
import numpy as np
import pytest

import synthkv
from conftest import golden
from oracle import (CodecConfig, bits_per_value_ratio, chunk_bytes, compression_ratio,
                    encode_chunk, kv_cache_bytes)


def _cfg(p, tensor="K"):
    return CodecConfig(d=p.d, n_centroids=p.n_centroids, n_stages=p.n_stages,
                       group_size=p.group_size, iters_cold=1, iters_warm=1,
                       seed=p.codec_seed(tensor), dtype=p.dtype)


def test_kv_memory_formula_matches_an_allocation():
    # K and V for L layers of (H*W*T) tokens with hidden size d
    for L, Hh, W, T, d, b in [(2, 3, 4, 5, 8, 2), (1, 30, 52, 3, 128, 2), (4, 8, 8, 2, 64, 4)]:
        dt = {2: np.float16, 4: np.float32}[b]
        kv = np.zeros((2, L, Hh * W * T, d), dtype=dt)
        assert kv_cache_bytes(L, Hh, W, T, d, b) == kv.nbytes


def test_token_count_of_a_five_second_clip_fits_the_layer_preset():
    pf = golden("pages_figures.json")
    assert synthkv.PRESETS[3].n_tokens == pf["latent_tokens_5s_480p"]["value"]
    assert synthkv.PRESETS[3].n_centroids == pf["centroids"]["value"]


@pytest.mark.parametrize("idx", [1, 2])
def test_chunk_bytes_match_encoded_arrays(idx):
    p = synthkv.PRESETS[idx]
    X = synthkv.gen_numpy(p, "K", n_tokens=min(p.n_tokens, 600))
    cfg = _cfg(p)
    enc = encode_chunk(X, cfg)
    b = chunk_bytes(cfg, X.shape[0], X.shape[1])
    assert b["codes"] == enc.codes.nbytes
    assert b["scales"] == enc.scales.nbytes
    assert b["assign"] == enc.assign.nbytes
    assert b["centroids"] == enc.centroids.size * (2 if p.dtype == "bf16" else 4)


def test_chunk_bytes_closed_form_values():
    assert sum(chunk_bytes(_cfg(synthkv.PRESETS[2]), 1, 4680).values()) == 299552
    assert sum(chunk_bytes(_cfg(synthkv.PRESETS[1]), 1, 128).values()) == 6784
    assert chunk_bytes(_cfg(synthkv.PRESETS[2]), 1, 4680) == {
        "codes": 149760, "scales": 9360, "assign": 9360, "centroids": 131072}


def test_compression_ratios():
    c2 = _cfg(synthkv.PRESETS[2])
    assert compression_ratio(c2, 1, 4680) == pytest.approx(1198080 / 299552)
    assert compression_ratio(c2, 40, 4680) == pytest.approx(4.000, abs=5e-3)
    assert compression_ratio(c2, 1, 4680, include_centroids=False) == pytest.approx(2048 / 288)
    c4 = _cfg(synthkv.PRESETS[4])
    assert compression_ratio(c4, 24, 4680) == pytest.approx(2.56, abs=5e-3)
    assert compression_ratio(c2, 40, 560) < 1.0                  # ragged chunk: centroids dominate


def test_round_to_nearest_figure_is_two_and_a_half_bits():
    rtn = golden("pages_figures.json")["rtn_compression"]["value"]
    assert bits_per_value_ratio(2, 16, 32) == pytest.approx(rtn)      # fp16 scale per 32 values
    assert bits_per_value_ratio(2, 32, 64) == pytest.approx(rtn)      # fp16 scale + zero per 64
    assert bits_per_value_ratio(2, 8, 64) == pytest.approx(16 / 2.125)  # E4M3 scale per 64
