"""Host-side behaviour of bench.py, the binding and the entry module (CPU only):
the one-GPU contract, loud failures without a GPU or without the library, the
algorithmic byte counts and the staleness check of the recorded HBM traffic."""
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run_bench(*args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300, env=env)


def test_bench_refuses_more_than_one_gpu():
    r = _run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""


def test_bench_refuses_a_multi_rank_launch():
    r = _run_bench(env_extra={"WORLD_SIZE": "2"})
    assert r.returncode == 2
    assert "WORLD_SIZE=2" in r.stderr


def _gpu_present():
    torch = pytest.importorskip("torch")
    return torch.cuda.is_available()


def test_bench_without_gpu_fails_loudly():
    if _gpu_present():
        pytest.skip("a GPU is present")
    for extra in ([], ["--decode", "d1"]):
        r = _run_bench("--steps", "1", "--warmup", "0", *extra)
        assert r.returncode == 1, r.stderr
        assert "needs a GPU" in r.stderr
        assert not any(l.startswith("{") for l in r.stdout.splitlines())


def test_algorithmic_bytes():
    """Forward: Q, K, V read and O written (bf16) plus the fp32 LSE. Backward:
    Q, K, V, O, dO read, LSE and D (fp32) read, D written, dQ, dK, dV written."""
    sys.path.insert(0, ROOT)
    import bench
    from exact_io_aware_12_amd import inputs as fi
    w = fi.WORKLOADS[5]
    n = w.B * w.H * w.N
    assert bench.fwd_bytes(w) == 4 * n * w.d * 2 + 4 * n
    assert bench.bwd_bytes(w) == (5 * n * w.d * 2) + 4 * n + 8 * n + 3 * n * w.d * 2
    assert bench.fwd_bytes(w) == 2 * 16 * 2048 * (4 * 128 * 2 + 4)


def test_recorded_traffic_is_dropped_when_sources_change(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import hashlib
    import bench
    csrc = tmp_path / "exact_io_aware_12_amd" / "csrc"
    csrc.mkdir(parents=True)
    names = ("fa_common.h", "fa_fwd.hip", "fa_bwd.hip")
    for f in names:
        shutil.copy(os.path.join(ROOT, "exact_io_aware_12_amd", "csrc", f), csrc / f)
    h = hashlib.sha256("".join((csrc / f).read_text() for f in names).encode()).hexdigest()[:16]
    (tmp_path / "profiles").mkdir()
    rec = {"sources_sha256_16": h, "read_bytes": 1000.0, "write_bytes": 24.0}
    (tmp_path / "profiles" / "fa_fwd_workload3_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.recorded_traffic(3, "fa_fwd") == 1024.0
    assert bench.recorded_traffic(4, "fa_fwd") is None      # no record
    with open(csrc / "fa_fwd.hip", "a") as f:
        f.write("\n// edited\n")
    assert bench.recorded_traffic(3, "fa_fwd") is None      # stale record


def test_binding_without_library_raises(monkeypatch):
    sys.path.insert(0, ROOT)
    from exact_io_aware_12_amd import fa
    monkeypatch.setattr(fa, "_LIB_PATH", os.path.join(ROOT, "no_such_dir", "libfa355.so"))
    monkeypatch.setattr(fa, "_lib", None)
    with pytest.raises(ImportError, match="no CPU fallback"):
        fa.library()
    with pytest.raises(ImportError):
        fa.fa_bwd_workspace_bytes(1, 1, 16, 64)


def test_entry_module_has_build_and_smoke():
    sys.path.insert(0, ROOT)
    import __graft_entry__ as g
    assert callable(g.build) and callable(g.smoke)
    if not _gpu_present():
        with pytest.raises(AssertionError, match="needs a GPU"):
            g.smoke()


def test_autograd_wrapper_refuses_cpu_tensors():
    # fa.attention checks its inputs like fwd: CPU tensors never reach the
    # library (and there is no CPU path to fall back to).
    torch = pytest.importorskip("torch")
    from exact_io_aware_12_amd import fa
    q = torch.zeros((1, 1, 8, 64), dtype=torch.bfloat16, requires_grad=True)
    with pytest.raises(ValueError, match="must be on a GPU"):
        fa.attention(q, q, q, causal=True)
