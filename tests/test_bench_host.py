"""Host-side helpers of bench.py (no GPU): the shader-clock table parser."""

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
