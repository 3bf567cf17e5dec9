"""bench.py on the host (no GPU): the one-GPU guard and the kernel-code hashes
that key the committed HBM counter data."""
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
    rec = {"resnet50/ring": {"kernel_source_sha": b.kernel_source_sha(), "hbm_bytes_per_launch": 123,
                             "profile": "profiles/x.md", "taken": "2026-12-02"}}
    f = tmp_path / "t.json"
    f.write_text(json.dumps(rec))
    b.TRAFFIC_FILE = str(f)
    nbytes, src = b.measured_traffic("resnet50", "ring")
    assert nbytes == 123 and src["profile"] == "profiles/x.md" and src["taken"] == "2026-12-02"
    nbytes, why = b.measured_traffic("resnet50", "seq")
    assert nbytes is None and "no counter run" in why
    rec["resnet50/ring"]["kernel_source_sha"] = "0" * 16
    f.write_text(json.dumps(rec))
    nbytes, why = b.measured_traffic("resnet50", "ring")
    assert nbytes is None and "0" * 16 in why


def test_per_parameter_traffic_has_its_own_key_and_hash(tmp_path):
    """The per-parameter sync's counters are keyed apart from the flat
    reduce's and checked against the hash of its own sources."""
    b = _bench()
    import json
    assert any(p.endswith("params.hip") for p in b.PARAMS_KERNEL_SOURCES)
    assert not any(p.endswith("reduce.hip") for p in b.PARAMS_KERNEL_SOURCES)
    assert b.kernel_source_sha("per-parameter") != b.kernel_source_sha()
    assert b.traffic_key("gpt1p3b", "ring", "per-parameter") == "gpt1p3b:per-parameter/ring"
    rec = {"gpt1p3b/ring": {"kernel_source_sha": b.kernel_source_sha(), "hbm_bytes_per_launch": 1},
           "gpt1p3b:per-parameter/ring": {"kernel_source_sha": b.kernel_source_sha("per-parameter"),
                                          "hbm_bytes_per_launch": 2}}
    f = tmp_path / "t.json"
    f.write_text(json.dumps(rec))
    b.TRAFFIC_FILE = str(f)
    assert b.measured_traffic("gpt1p3b", "ring")[0] == 1
    assert b.measured_traffic("gpt1p3b", "ring", "per-parameter")[0] == 2
    nbytes, why = b.measured_traffic("gpt1p3b", "seq", "per-parameter")
    assert nbytes is None and "gpt1p3b:per-parameter/seq" in why
    # a record taken on the flat reduce's hash does not serve the per-parameter sync
    rec["gpt1p3b:per-parameter/ring"]["kernel_source_sha"] = b.kernel_source_sha()
    f.write_text(json.dumps(rec))
    assert b.measured_traffic("gpt1p3b", "ring", "per-parameter")[0] is None


def test_parser_defaults_and_layouts(monkeypatch):
    b = _bench()
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    a = b.parse_args()
    assert (a.gpus, a.steps, a.warmup, a.workload, a.layout) == (1, 50, 10, "gpt1p3b", "bucket-view")
    assert a.order is None and a.settle_seconds == 20.0 and not a.child
    assert a.configs.split(",") == ["resnet50", "many_small", "tiny", "gpt1p3b_two_bucket",
                                    "gpt1p3b:per-parameter", "llama7b"]
    monkeypatch.setattr(sys, "argv", ["bench.py", "--layout", "per-parameter", "--settle-seconds", "0",
                                      "--workload", "tiny", "--order", "seq", "--child"])
    a = b.parse_args()
    assert (a.layout, a.settle_seconds, a.workload, a.order, a.child) == \
        ("per-parameter", 0.0, "tiny", "seq", True)


def test_dtype_label_follows_the_workload():
    b = _bench()
    import workloads as W
    assert b.dtype_label(W.workload("gpt1p3b")) == "f32"
    assert b.dtype_label(W.workload("llama7b")) == "bf16->bf16 (f32 accumulate)"


def test_cpu_sample_is_bounded_and_keeps_bucket_positions():
    """The CPU oracle's sample of a multi-GB workload: leading buckets up to
    4 GiB of inputs, the last one cut short at its own position 0."""
    b = _bench()
    import types
    import workloads as W
    import oracle
    for name in ("gpt1p3b", "gpt1p3b_two_bucket", "resnet50"):
        wl = W.workload(name)
        c = types.SimpleNamespace(wl=wl, N=wl.n_ranks, P=wl.total)
        runs, sampled = b.oracle_sample(c, oracle)
        n = sum(r[3] for r in runs)
        assert n * wl.n_ranks * wl.in_bytes <= b.SAMPLE_INPUT_BYTES
        assert sampled == (n < wl.total)
        assert all(pos == 0 and 0 < cnt <= ln for _, ln, pos, cnt in runs)
        starts = [a for a, _, _, _ in runs]
        assert starts == sorted(starts)
    assert not sampled           # resnet50: the whole synchronisation
