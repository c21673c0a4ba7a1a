"""The optional roctx ranges of the round loop: off by default (a no-op), and
with SPEC_ROCTX=1 the ROCm marker library loads and ranges nest (no GPU and
no profiler needed: without a profiler the markers do nothing)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_ranges_are_a_no_op_when_disabled():
    from layer_speculative_decoding_amd import trace
    if os.environ.get("SPEC_ROCTX") == "1":
        return
    with trace.rng("round"):
        with trace.rng("draft"):
            pass
    assert not trace.enabled()


def test_ranges_load_the_marker_library_when_enabled():
    code = ("import sys; from layer_speculative_decoding_amd import trace\n"
            "with trace.rng('round'):\n    with trace.rng('draft'):\n        pass\n"
            "print('enabled', trace.enabled())")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=dict(os.environ, SPEC_ROCTX="1"),
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    if not os.path.exists("/opt/rocm/lib"):
        return
    assert "enabled True" in r.stdout, (r.stdout, r.stderr[-1000:])
