"""Host-side checks of bench.py (no GPU): the algorithmic byte counts behind
the roofline figures, the counter-summary lookup and the one-GPU guard.

The expected byte totals are the per-workload figures stated with the
workload definitions (DeepSeek-V3-shaped, skewed and large batches), in MB
of 10^6 bytes rounded to 0.1 MB; the test recomputes nothing from bench.py's
own formulas."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from permute_ep_layout_amd import profiling, workloads  # noqa: E402


def mb(x):
    return round(x / 1e6, 1)


# (workload, routed rows N, tokens with a slot, layout MB, scatter MB,
#  combine MB with fp32 y, combine MB with bf16 y, scatter + combine MB)
STATED = [
    ("dsv3", 32768, 4096, 0.39, 537.3, 587.5, 528.7, 1124.7),
    ("skew", 131072, 16384, 1.57, 2149.1, 2349.9, 2115.0, 4498.9),
    ("large", 524288, 65536, 8.39, 8464.1, 9399.4, 8459.9, 17863.5),
]


@pytest.mark.parametrize("case", STATED, ids=[c[0] for c in STATED])
def test_algorithmic_bytes_match_the_stated_totals(case):
    name, N, T_any, layout, scatter, comb32, comb16, both = case
    w = workloads.get(name)
    b32 = bench.algorithmic_bytes(w, N, T_any, 4)
    b16 = bench.algorithmic_bytes(w, N, T_any, 2)
    # the stated layout figure has no per-node column; those add 4 bytes each
    assert abs(b32["layout"] / 1e6 - layout) < 0.01
    assert mb(b32["scatter"]) == scatter
    assert mb(b32["combine"]) == comb32
    assert mb(b16["combine"]) == comb16
    assert mb(b32["scatter"] + b32["combine"]) == both


def test_fp8_scatter_bytes_halve_the_rows():
    """FP8 rows are H bytes and the UE8M0 scales ceil(S/4) = 14 words:
    at DeepSeek-V3 shape 29.4 + 0.2 + 0.3 MB read (rows, scales, ids) and
    234.9 + 1.8 + 0.3 MB written (rows, scales, m_indices + output_index),
    266.8 MB against 537.3 MB for bf16 rows with fp32 scales."""
    w = workloads.get("dsv3_fp8")
    assert w.scale_words == 14
    assert mb(bench.algorithmic_bytes(w, 32768, 4096)["scatter"]) == 266.8


def test_low_latency_bytes():
    """Low-latency dispatch at DeepSeek-V3 shape: bf16 rows in, FP8 rows and
    fp32 scales out for 32768 routed rows, plus the small per-slot arrays."""
    w = workloads.get("dsv3_ll")
    b = bench.ll_algorithmic_bytes(w, 32768, 4096)
    assert mb(b["ll_dispatch"]) == 301.7
    assert mb(b["combine"]) == 587.5


def test_padding_rows_cost_one_index_each():
    w = workloads.get("dsv3")
    a = bench.algorithmic_bytes(w, 32768, 4096, 4, pad_rows=0)
    b = bench.algorithmic_bytes(w, 32768, 4096, 4, pad_rows=1000)
    assert b["scatter"] - a["scatter"] == 4000
    assert b["combine"] == a["combine"]


def test_traffic_lookup_requires_the_profiled_sources(monkeypatch):
    """roofline.traffic comes from the committed counter summary only while
    the kernel sources match the digest it was taken on, and only for the
    options it was taken with."""
    path = bench.TRAFFIC_FILE.format(workload="dsv3")
    data = profiling.read_traffic(path)
    assert data and "combine" in data["kernels"]
    if data["source_digest"] == profiling.source_digest():
        got = bench.measured_traffic("dsv3", "combine")
        assert got == data["kernels"]["combine"]["bytes_per_launch"]
    # the summaries were taken with the default options only
    assert bench.measured_traffic("dsv3", "combine", out_dtype="bf16") is None
    assert bench.measured_traffic("dsv3", "combine", alignment=128) is None
    monkeypatch.setattr(profiling, "source_digest", lambda root=None: "0" * 16)
    assert bench.measured_traffic("dsv3", "combine") is None
    assert bench.measured_traffic("no_such_workload", "combine") is None


def test_digest_ignores_comments_only():
    a = "int f(int x) { return x + 1; } // add one\n/* block */"
    b = "int f(int x)\n{\n    return x + 1;   /* other words */\n}\n"
    c = "int f(int x) { return x + 2; }"
    assert profiling._code_only(a) == profiling._code_only(b)
    assert profiling._code_only(a) != profiling._code_only(c)
    # string literals keep their comment-like text
    assert "//" in profiling._code_only('const char *s = "a // b";')


def test_more_than_one_gpu_is_refused():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert proc.returncode == 2
    assert "one GPU" in proc.stdout + proc.stderr
    # nothing that looks like a result line
    for line in proc.stdout.splitlines():
        with pytest.raises(ValueError):
            json.loads(line)


def test_probe_library_exports_and_checks_arguments():
    """The streaming probes behind bench.py --ceilings: every entry point
    exists and rejects bad arguments on the host (no GPU call is made)."""
    import ctypes

    import bench_probe

    lib = ctypes.CDLL(bench_probe.ensure_built())
    for name in ("epl_probe_mix", "epl_probe_fan"):
        f = getattr(lib, name)
        f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                      ctypes.c_int, ctypes.c_int, ctypes.c_uint, ctypes.c_void_p]
        assert f(None, None, 16, 16, 1, 0, 64, None) == -1      # null buffers
        assert f(16, 32, 0, 0, 1, 0, 64, None) == -1            # no words
        assert f(16, 32, 16, 8, 1, 0, 64, None) == -1           # streams overlap
        assert f(16, 32, 16, 16, 3, 0, 64, None) == -1          # unsupported mix
        assert f(8, 32, 16, 16, 1, 0, 64, None) == -1           # misaligned
        assert f(16, 32, 16, 16, 1, 0, 0, None) == -1           # empty grid
    pieces = lib.epl_probe_pieces
    pieces.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                       ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    assert pieces(None, 256, 256, 256, 0, 0, None) == -1        # null buffer
    assert pieces(16, 0, 256, 256, 0, 0, None) == -1            # no words
    assert pieces(16, 256, 0, 256, 0, 0, None) == -1            # empty pieces
    assert pieces(16, 256, 256, 96, 0, 0, None) == -1           # not whole waves
    assert pieces(16, 256, 256, 2048, 0, 0, None) == -1         # above 1024 threads
    assert pieces(8, 256, 256, 256, 0, 0, None) == -1           # misaligned
    assert pieces(16, 1 << 40, 1, 64, 0, 0, None) == -1         # grid above 2^22
    fill = lib.epl_probe_fill32
    fill.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p]
    assert fill(None, 16, 7, None) == -1
    assert fill(16, 0, 7, None) == -1
    assert fill(2, 16, 7, None) == -1


def test_host_cpu_description():
    h = bench.host_cpu()
    assert isinstance(h["model"], str) and h["model"]
    assert h["logical_cpus"] >= 1
