"""The cross-workgroup protocols (generation-counted join, tagged-slot exchanges, launch joins) as a
host thread model, built with ThreadSanitizer and run on the CPU (tests/join_model.cpp).

[sass2mlir] "Counter-based mini-joins" and "Grid-barrier synthesis" (arrival counters, self-cleaning
state, coherent cross-workgroup reads); [AStitch] "What it costs" (the exchange needs every member
resident: a member that never arrives must end in the error word, never in a hang).
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("g++ is not available")
    out = str(tmp_path_factory.mktemp("join_model") / "join_model")
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-pthread", "-fsanitize=thread", os.path.join(HERE, "join_model.cpp"),
           "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return out


@pytest.mark.parametrize("scenario", ["gen", "split", "ln", "missing"])
def test_protocol_under_thread_sanitizer(model, scenario):
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1 exitcode=66")
    r = subprocess.run([model, scenario], capture_output=True, text=True, timeout=300, env=env)
    assert "ThreadSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, (r.stdout, r.stderr[-2000:])
    assert r.stdout.strip() == f"OK {scenario}"


@pytest.mark.parametrize("mutant", ["mutant-nowait", "mutant-noawait", "mutant-oneparity"])
def test_planted_protocol_mistakes_are_caught(model, mutant):
    """Reading partials without the join (a data race the sanitizer reports), taking slots before
    the launch join (stale slots of the previous launch carry the first row's tag: wrong merges),
    and one slot set for every row (a fast member's next row hides the tag a slow one waits for:
    the waits give up): each must fail."""
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1 exitcode=66")
    r = subprocess.run([model, mutant], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode != 0 or "ThreadSanitizer" in r.stderr, (r.stdout, r.stderr[-2000:])
