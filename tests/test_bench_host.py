"""Host-side checks of bench.py (no GPU): the multi-GPU refusal and the closed
forms it reports against."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_decode_bytes_closed_form():
    # 13B layer, K and V as 80 heads, 38,000 tokens in 9 chunks: codes d/4, scales d/G,
    # labels T, bf16 output 2d per vector, plus every chunk's bf16 tables once
    assert bench.decode_bytes(80, 38000, 128, 64, 2, 256, 9) == 982051840
    # long-horizon cache: 24 heads, 1,092,000 tokens in 234 chunks
    assert bench.decode_bytes(24, 1092000, 128, 64, 2, 256, 234) == 8388836352


def test_traffic_follows_the_kernel_source(tmp_path, monkeypatch):
    """hbm_traffic gives the committed counters' bytes only while the kernel
    source hashes to the one they were taken on, else None."""
    import hashlib
    import json
    rec = json.load(open(os.path.join(ROOT, "profiles", "hbm_traffic.json")))
    src = os.path.join(ROOT, "bit_vector_quantization_amd", "csrc", "qvg_kernels.hip")
    same = hashlib.sha256(open(src, "rb").read()).hexdigest() == rec["kernels_source_sha256"]
    t = bench.hbm_traffic("decode")
    assert (t is not None and t > 0) if same else t is None
    assert bench.hbm_traffic("no_such_kernel") is None
    # a copy of the repository whose kernel source differs reports None
    root = tmp_path / "r"
    (root / "profiles").mkdir(parents=True)
    (root / "bit_vector_quantization_amd" / "csrc").mkdir(parents=True)
    (root / "profiles" / "hbm_traffic.json").write_text(json.dumps(rec))
    (root / "bit_vector_quantization_amd" / "csrc" / "qvg_kernels.hip").write_text("// changed\n")
    monkeypatch.setattr(bench.os.path, "abspath", lambda p, _a=os.path.abspath: str(root / "bench.py")
                        if p == bench.__file__ else _a(p))
    assert bench.hbm_traffic("decode") is None
