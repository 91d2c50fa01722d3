"""Host-side logic of bench.py, checked without a GPU: the one-GPU guard, the algorithmic
byte and flop counts the roofline divides by, the profile-traffic gate and the trace-region
parser that matches bench's event figures to the rocprofv3 dispatch trace."""
import csv
import json
import os
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import mla_inputs as mi  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _shape(B, q_len, H, L, dtype):
    return types.SimpleNamespace(B=B, q_len=q_len, H=H, dtype=dtype, page_size=64,
                                 seq_lens=__import__("numpy").array(L, dtype="int32"))


def test_algorithmic_counts_of_the_batch4_agentic_step():
    """B=4, q_len=4, H=32, E4M3, 81,920 keys each: the KV stream is B*L*576 bytes (188.7 MB), and the
    causal rule leaves L-3, L-2, L-1, L keys visible to the four tokens of each sequence."""
    L = 81920
    alg = bench.algorithmic(_shape(4, 4, 32, [L] * 4, mi.FP8_E4M3))
    assert alg["kv_bytes"] == 4 * L * 576
    assert alg["flops"] == 2 * (576 + 512) * 32 * 4 * (4 * L - 6)
    # everything else (q, out, lse, block table, lengths) is under 1% of the KV stream
    assert alg["kv_bytes"] < alg["bytes"] < 1.01 * alg["kv_bytes"]


def test_algorithmic_counts_with_sequences_shorter_than_the_query():
    # L=2 with q_len=4: tokens 0 and 1 see nothing, tokens 2 and 3 see 1 and 2 keys; L=0 sees nothing
    alg = bench.algorithmic(_shape(2, 4, 16, [2, 0], mi.BF16))
    assert alg["flops"] == 2 * (576 + 512) * 16 * 3
    assert alg["kv_bytes"] == 2 * 576 * 2


def test_code_hash_ignores_comments_and_whitespace_only():
    a = bench.code_hash("int a = 1; // one\n/* block\ncomment */ float b;")
    assert a == bench.code_hash("int  a = 1;\n\nfloat   b;  // other words")
    assert a != bench.code_hash("int a = 2; float b;")


def test_traffic_is_reported_only_for_the_current_kernel_code(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    path = tmp_path / "profiles" / "mla_split_kv_partial_w_traffic.json"
    path.write_text(json.dumps({"kernel_code_sha256_16": bench.kernel_hash(), "hbm_bytes_per_launch": 123}))
    assert bench.load_traffic("w") == 123
    path.write_text(json.dumps({"kernel_code_sha256_16": "0" * 16, "hbm_bytes_per_launch": 123}))
    assert bench.load_traffic("w") is None
    assert bench.load_traffic("absent") is None


def _write_trace(path, events):
    path.mkdir(parents=True)
    with open(path / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        t = 1000
        for name, dur in events:
            w.writerow({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + dur})
            t += dur + 100


def test_trace_regions_average_only_the_timed_launches(tmp_path):
    """bench runs warm-up steps, K timed steps, then each kernel alone (a few untimed launches that
    marshal the calls, then K timed ones); only the last K launches of each region count."""
    P, M = "void mla::mla_split_kv_partial<2, true, false, true>", "mla::mla_combine(mla::CombineParams)"
    K = 50
    ev = [("copyBuffer", 500)]
    ev += [(P, 9000), (M, 3000)] * 30  # warm-up: slower, as at cold clocks
    ev += [(P, 5000), (M, 1000)] * K
    ev += [(P, 7000)] * 5 + [(P, 4000)] * K
    ev += [(M, 2500)] * 5 + [(M, 800)] * K
    _write_trace(tmp_path / "trace", ev)
    reg = bench._trace_regions(str(tmp_path / "trace"), steps=K)
    assert reg["steps"]["split_kv_us"] == 5.0 and reg["steps"]["merge_us"] == 1.0
    assert reg["steps"]["step_period_us"] == pytest.approx(6.2)  # 5 + 1 us of kernels, two 0.1 us gaps
    assert reg["split_kv_alone"]["duration_us"] == 4.0
    assert reg["merge_alone"]["duration_us"] == 0.8
