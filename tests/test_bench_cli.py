"""bench.py's command-line contract on the host: it measures one GPU only, so a request for more
GPUs (flag or torchrun environment) exits with status 2 and a message, before touching a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True,
                          text=True, env=env, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_world_size_above_one_is_refused():
    r = _run([], {"WORLD_SIZE": "4"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_counter_figures_follow_the_kernel_hash(tmp_path, monkeypatch):
    """The traffic and ALU figures come from the committed counter summaries only while the kernel
    source hashes to the value recorded with them; another hash, or no summary, gives None."""
    sys.path.insert(0, ROOT)
    import bench

    digest = bench.kernel_code_digest()
    good = tmp_path / "good.md"
    good.write_text(f"text\nkernel_code_sha256: {digest}\ntraffic_bytes_per_launch: 123\n"
                    "valu_lane_instr_per_weight: 4.5\nlds_lane_instr_per_weight: 1.25\nvalu_bound_us: 40\n")
    stale = tmp_path / "stale.md"
    stale.write_text(good.read_text().replace(digest, "0" * 64))
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(good))
    monkeypatch.setattr(bench, "SQ_PROFILE", str(good))
    assert bench.measured_traffic() == 123.0
    assert bench.measured_alu() == {"valu_lane_instr_per_weight": 4.5, "lds_lane_instr_per_weight": 1.25,
                                    "valu_bound_us": 40.0}
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(stale))
    monkeypatch.setattr(bench, "SQ_PROFILE", str(tmp_path / "missing.md"))
    assert bench.measured_traffic() is None
    assert bench.measured_alu() is None
