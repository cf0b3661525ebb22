"""CPU checks of bench.py: a run on more than one GPU is refused with a message before
anything touches a device (the library has no multi-GPU path), and the HBM traffic it
reports comes from the committed counter summary only while the kernel sources match."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          env=env, capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_a_multi_rank_launch_is_refused():
    r = _run([], {"WORLD_SIZE": "2", "RANK": "0", "LOCAL_RANK": "0"})
    assert r.returncode == 2
    assert "WORLD_SIZE 2" in r.stderr


def test_traffic_is_read_only_for_matching_kernel_sources(tmp_path, monkeypatch):
    """bench.py takes a launch's HBM bytes from the committed counter summary only while
    the kernel sources still hash to the digest recorded with the counters."""
    import hashlib
    import shutil
    sys.path.insert(0, ROOT)
    import bench
    csrc = tmp_path / "pseudo_random_weight_amd" / "csrc"
    csrc.mkdir(parents=True)
    h = hashlib.sha256()
    for f in ("seedmm.hip", "seed_decode.hpp"):
        shutil.copy(os.path.join(ROOT, "pseudo_random_weight_amd", "csrc", f), csrc / f)
        h.update((csrc / f).read_bytes())
    (tmp_path / "profiles").mkdir()
    summary = tmp_path / "profiles" / "hbm_traffic.txt"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    summary.write_text(f"# test\nsource_sha256_16 = {h.hexdigest()[:16]}\n"
                       "gateup_T64_P4.bytes_per_launch = 1.5e+08\n")
    assert bench.read_traffic("gateup_T64_P4") == 1.5e8
    assert bench.read_traffic("down_T64_P4") is None
    summary.write_text("source_sha256_16 = 0000000000000000\n"
                       "gateup_T64_P4.bytes_per_launch = 1.5e+08\n")
    assert bench.read_traffic("gateup_T64_P4") is None
