"""The synthetic inputs have the statistics the pages describe (input recipe checks)."""
import numpy as np

import synthkv


def test_magnitudes_and_outlier_channels():
    p = synthkv.PRESETS[2]
    K = synthkv.gen_numpy(p, "K")[0]
    V = synthkv.gen_numpy(p, "V")[0]
    assert 80 < np.abs(K).max() < 200 and 800 < np.abs(V).max() < 2000
    # two dominant channels per token, mostly the same two, sometimes others
    top = np.argsort(-np.abs(K), axis=1)[:, :2]
    fixed = np.bincount(top.ravel(), minlength=p.d).argsort()[-2:]
    moved = ~np.isin(top, fixed).all(axis=1)
    assert 0.002 < moved.mean() < 0.05


def test_adjacent_frames_are_similar():
    p = synthkv.PRESETS[2]
    X = synthkv.gen_numpy(p, "K")[0].astype(np.float64)
    top = np.bincount(np.argsort(-np.abs(X), axis=1)[:, :2].ravel(), minlength=p.d).argsort()[-2:]
    keep = np.setdiff1d(np.arange(p.d), top)
    f = X[:, keep].reshape(3, p.frame_tokens, -1)
    cos = []
    for i in range(2):
        # leave out the ~1% of tokens whose outliers moved into these channels
        ok = (np.abs(f[i]).max(1) < 20) & (np.abs(f[i + 1]).max(1) < 20)
        a, b = f[i][ok], f[i + 1][ok]
        cos.append((a * b).sum() / np.linalg.norm(a) / np.linalg.norm(b))
    assert all(0.9 < c < 0.99 for c in cos), cos


def test_bf16_values_and_prefix_consistency():
    p = synthkv.PRESETS[2]
    a = synthkv.gen_numpy(p, "V", n_tokens=2000)
    b = synthkv.gen_numpy(p, "V")
    np.testing.assert_array_equal(a, b[:, :2000])
    bits = a.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0)
    w = synthkv.gen_numpy(p, "V", n_tokens=1560, frame_begin=1)
    np.testing.assert_array_equal(w, b[:, 1560:3120])


def test_presets_chunking():
    p3 = synthkv.PRESETS[3]
    assert p3.chunk_tokens == 4680 and p3.n_chunks == 9 and p3.chunk_range(8) == (37440, 38000)
    p5 = synthkv.PRESETS[5]
    assert p5.n_chunks == 234 and p5.chunk_range(233)[1] - p5.chunk_range(233)[0] == 1560
    assert synthkv.PRESETS[1].chunk_tokens == 128
