"""bench.py's command line on the CPU: more than one GPU is refused with a
message before any GPU is touched (the library is single-GPU)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""


def test_bench_help_lists_launch_modes():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0
    for opt in ("--launch", "--streams", "--workload", "--steps", "--warmup", "--extras"):
        assert opt in r.stdout


def test_traffic_key_ignores_comments_only(tmp_path):
    """The key of the stored HBM counters survives comment and blank-line edits
    and changes with any edit of the code itself."""
    sys.path.insert(0, ROOT)
    from ternary_weight_linear_tern_amd.rocprof_summary import kernel_code_hash
    base = "// header\n__global__ void k(int *p) {\n    p[0] = 1;   // store\n}\n"
    variants = {
        "comments": "// other header\n/* block\n   comment */\n__global__ void k(int *p) {\n\n    p[0] = 1;\n}\n",
        "code": "// header\n__global__ void k(int *p) {\n    p[0] = 2;   // store\n}\n",
    }
    f = tmp_path / "a.hip"
    f.write_text(base)
    h0 = kernel_code_hash(str(f))
    f.write_text(variants["comments"])
    assert kernel_code_hash(str(f)) == h0
    f.write_text(variants["code"])
    assert kernel_code_hash(str(f)) != h0
