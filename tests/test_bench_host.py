"""Host-side parts of bench.py (no GPU): the shader-clock table parser, the
check that the committed counter summaries match the sources, and the
refusal of runs on more than one GPU."""

import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
bench = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(bench)


def test_current_sclk_active_level():
    assert bench.current_sclk_mhz("0: 500Mhz\n1: 2309Mhz *\n2: 2400Mhz\n") == 2309


def test_current_sclk_deep_sleep_level():
    assert bench.current_sclk_mhz("S: 95Mhz *\n0: 500Mhz\n1: 2400Mhz\n") == 95


def test_current_sclk_no_marked_level():
    assert bench.current_sclk_mhz("0: 500Mhz\n1: 2400Mhz\n") is None
    assert bench.current_sclk_mhz("") is None


def test_committed_counter_summaries_match_current_sources():
    """Every HBM-traffic and SQ-counter summary under profiles/ records the hash
    of the kernel sources it was measured on; a kernel edit must come with
    fresh counters (the bench reads the tile kernel's traffic only when its
    hash matches, the other summaries are cited as they stand)."""
    import glob
    import os
    from fp8_block_scaled_03_amd import profiling
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    files = sorted(glob.glob(os.path.join(root, "profiles", "traffic_*.txt")) +
                   glob.glob(os.path.join(root, "profiles", "counters_*.txt")))
    assert files
    for path in files:
        fields = {}
        with open(path, encoding="utf-8") as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip()
        sources = fields.get("sources", " ".join(profiling.GEMM_SOURCES)).split()
        assert fields.get("source_sha") == profiling.source_sha(sources), os.path.basename(path)


def test_bench_refuses_more_than_one_gpu():
    """The bench measures one GPU's share; any other --gpus (or a launcher's
    WORLD_SIZE above 1) ends with a message and status 2 before any GPU work."""
    import subprocess
    import sys
    env = dict(os.environ)
    env.pop("WORLD_SIZE", None)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, env=env, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    env["WORLD_SIZE"] = "4"
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True, text=True, env=env,
                       timeout=120)
    assert r.returncode == 2
