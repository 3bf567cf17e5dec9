"""bench.py on the host (no GPU): the one-GPU guard and the kernel-code hash
that keys the committed HBM counter data."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("_bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_exits_with_2():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_code_hash_ignores_comments_and_blank_lines(tmp_path):
    b = _bench()
    assert any(p.endswith("reduce.hip") for p in b.KERNEL_SOURCES)
    assert any(p.endswith("device.h") for p in b.KERNEL_SOURCES)
    assert not any(p.endswith("probe.hip") for p in b.KERNEL_SOURCES)
    base = b.kernel_source_sha()
    copies = []
    for path in b.KERNEL_SOURCES:
        c = tmp_path / os.path.basename(path)
        src = open(path, encoding="utf-8").read()
        if path.endswith("device.h"):
            src = "// a new comment\n\n" + src.replace("\n{\n", "\n{   /* note */\n", 1) + "\n\n"
        c.write_text(src)
        copies.append(str(c))
    b.KERNEL_SOURCES = copies
    assert b.kernel_source_sha() == base
    dev = next(c for c in copies if c.endswith("device.h"))
    text = open(dev, encoding="utf-8").read()
    open(dev, "w", encoding="utf-8").write(text.replace("kThreads = 64", "kThreads = 128", 1))
    assert b.kernel_source_sha() != base


def test_traffic_is_reported_only_for_the_hashed_code(tmp_path):
    b = _bench()
    import json
    rec = {"resnet50/ring": {"kernel_source_sha": b.kernel_source_sha(), "hbm_bytes_per_launch": 123}}
    f = tmp_path / "t.json"
    f.write_text(json.dumps(rec))
    b.TRAFFIC_FILE = str(f)
    assert b.measured_traffic("resnet50", "ring", 1) == 123
    assert b.measured_traffic("resnet50", "seq", 1) is None
    rec["resnet50/ring"]["kernel_source_sha"] = "0" * 16
    f.write_text(json.dumps(rec))
    assert b.measured_traffic("resnet50", "ring", 1) is None


def test_parser_defaults_and_layouts(monkeypatch):
    b = _bench()
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    a = b.parse_args()
    assert (a.gpus, a.steps, a.warmup, a.workload, a.layout) == (1, 200, 20, "resnet50", "bucket-view")
    assert a.order is None and a.settle_seconds == 20.0
    monkeypatch.setattr(sys, "argv", ["bench.py", "--layout", "per-parameter", "--settle-seconds", "0",
                                      "--workload", "tiny", "--order", "seq"])
    a = b.parse_args()
    assert (a.layout, a.settle_seconds, a.workload, a.order) == ("per-parameter", 0.0, "tiny", "seq")
