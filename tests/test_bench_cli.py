"""bench.py's command-line contract on the host (no GPU needed)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_help_lists_the_contract_flags():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup"):
        assert flag in r.stdout


def _bench_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_counter_records_attach_only_to_their_own_kernel_and_run(tmp_path, monkeypatch):
    """A counter record reaches the bench line only for the step kind, token count and id rotation it was taken on,
    and only while the kernel's code (comments aside) is the code it was taken on."""
    import json
    b = _bench_module()
    src = tmp_path / "kernel.hip"
    src.write_text("int f() {\n    return 1;  // one\n}\n")
    rec_path = tmp_path / "rec.json"
    rec = {"n_tok": 1000, "id_batches": 4, "kernel_source_sha256": b.source_sha256([str(src)]),
           "hbm_bytes_per_launch": 7.0, "request_sizes": {"bytes_exact": 5.0}}
    rec_path.write_text(json.dumps(rec))
    monkeypatch.setattr(b, "PMC_RECORDS", {(5, "direct"): (str(rec_path), [str(src)])})
    assert b._traffic_exact((5, "direct"), 1000, 4) == 5.0
    assert b._traffic((5, "direct"), 1000, 4) == 7.0
    assert b._traffic_exact((5, "direct"), 1001, 4) is None  # another token count
    assert b._traffic_exact((5, "direct"), 1000, 1) is None  # another id rotation
    assert b._traffic_exact((5, "dedup"), 1000, 4) is None  # another step kind
    assert b._traffic_exact((4, "direct"), 1000, 4) is None  # another workload
    src.write_text("int f() {\n        return 1;  // a different comment, other indentation\n\n}\n")
    assert b._traffic_exact((5, "direct"), 1000, 4) == 5.0  # comments and layout do not count
    src.write_text("int f() {\n    return 2;\n}\n")
    assert b._traffic_exact((5, "direct"), 1000, 4) is None  # code does
    rec_path.write_text("not json")
    assert b._traffic_exact((5, "direct"), 1000, 4) is None
