"""Host logic of bench.py that needs no GPU: the one-GPU guard, the option
rules and the traffic record lookup (reported only for the profiled kernel
source)."""
import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          cwd=ROOT, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("workload", ["ulysses", "plain"])
def test_auxiliary_workloads_refuse_more_than_one_gpu(workload):
    r = _run("--workload", workload, "--gpus", "2", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_option_rules(monkeypatch):
    mod = _bench_module()
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    a = mod.parse()
    assert a.gpus == 1 and a.fuse_merge and not a.fuse_q
    monkeypatch.setattr(sys, "argv", ["bench.py", "--separate-merge"])
    assert not mod.parse().fuse_merge
    monkeypatch.setattr(sys, "argv", ["bench.py", "--fuse-q"])
    a = mod.parse()
    assert a.fuse_q and not a.fuse_merge          # the merging epilogue has no fused-Q form


def test_traffic_record_follows_the_kernel_source(tmp_path, monkeypatch):
    mod = _bench_module()
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    e = rec["attn_fwd"]["wan"]
    src = os.path.join(ROOT, "attention_qk_norm_rope_amd", "csrc", e["source"])
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    got = mod.traffic_entry("attn_fwd", "wan")
    assert got == (e["bytes_per_launch"] if digest == e["sha256"] else None)
    assert e["bytes_per_launch"] == round(sum(e["hbm_bytes_per_launch"]) / len(e["hbm_bytes_per_launch"]))
    # a record taken on other source bytes is not reported
    fake = tmp_path / "repo"
    (fake / "profiles").mkdir(parents=True)
    (fake / "attention_qk_norm_rope_amd" / "csrc").mkdir(parents=True)
    (fake / "attention_qk_norm_rope_amd" / "csrc" / e["source"]).write_text("// other source\n")
    json.dump(rec, open(fake / "profiles" / "traffic.json", "w"))
    monkeypatch.setattr(mod, "ROOT", str(fake))
    assert mod.traffic_entry("attn_fwd", "wan") is None
    assert mod.traffic_entry("attn_fwd", "qwen") is None
