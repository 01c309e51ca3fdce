"""Host-side checks of the benchmark script (no GPU): the multi-GPU refusal and the
rule that a profiled traffic figure is reported only while its kernel source is the
one the counters were taken on."""
import hashlib
import importlib.util
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused_before_any_device_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


def test_profiled_traffic_follows_the_code_hash(tmp_path):
    bench = _bench_module()
    csrc = tmp_path / "block_scaled_fp8_linear_amd" / "csrc"
    csrc.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    src = csrc / "k.hip"
    src.write_text("// kernel v1\n__global__ void k(float* y) { y[0] = 1.0f; }  /* one store */\n")
    digest = bench.code_digest(str(src))
    # the digest is that of the code alone: comments and whitespace removed
    assert digest == hashlib.sha256(b"__global__ void k(float* y) { y[0] = 1.0f; }").hexdigest()[:16]
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(
        {"k_case": {"source": "k.hip", "code_sha256_16": digest, "traffic_bytes": 1234.5},
         "stale": {"source": "k.hip", "code_sha256_16": "0" * 16, "traffic_bytes": 99.0}}))
    bench.ROOT = str(tmp_path)
    assert bench.profiled_traffic("k_case") == 1234.5
    assert bench.profiled_traffic("stale") is None          # counters taken on other code
    assert bench.profiled_traffic("missing") is None
    src.write_text("// kernel v1, comment reworded\n__global__ void k(float* y) {\n  y[0] = 1.0f;\n}\n")
    assert bench.profiled_traffic("k_case") == 1234.5       # only comments and layout changed
    src.write_text("__global__ void k(float* y) { y[0] = 2.0f; }\n")   # the kernel changed since
    assert bench.profiled_traffic("k_case") is None

