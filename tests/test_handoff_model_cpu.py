"""Host-thread model of a workgroup-to-workgroup record handoff (a ring of
chunk records with per-slot flags), the protocol a fused prefill would use.
Built with g++ (and once with ThreadSanitizer), run on the CPU only.

It pins the two properties such a handoff needs on the GPU:
  - publication by a release store and observation by an acquire load of
    the same word deliver every record intact (normal mode, TSan clean);
  - with a wait that can never succeed (a poll served by a stale private copy
    of the flag, or a role no workgroup took) every thread still ends, within
    about ONE wait bound, because the first timed-out wait sets a shared abort
    word that every other wait checks;
and it shows the failure mechanism without that abort word: each wait bounded
on its own, the run time grows as (number of waits) x (bound).
"""
import os
import shutil
import subprocess
import time

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "handoff_model", "ring_model.cpp")


@pytest.fixture(scope="module")
def model(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("ring") / "ring_model")
    subprocess.run(["g++", "-std=c++17", "-O2", "-pthread", "-Wall", "-Wextra", "-Werror", SRC,
                    "-o", exe], check=True)
    return exe


def run(exe, *args, timeout=60):
    t0 = time.perf_counter()
    r = subprocess.run([exe] + [str(a) for a in args], capture_output=True, text=True,
                       timeout=timeout)
    return r, time.perf_counter() - t0


@pytest.mark.parametrize("producers,ring", [(1, 2), (3, 4), (8, 16)])
def test_every_record_arrives_intact(model, producers, ring):
    r, _ = run(model, "normal", 2048, 8, producers, ring, 5000)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
    assert "checked 16384 bad 0" in r.stdout


@pytest.mark.parametrize("mode", ["stale", "missing_producer"])
def test_a_broken_handoff_ends_within_one_bound(model, mode):
    # 2048 chunk steps x 8 consumers: without the shared abort this would be
    # thousands of bounds; with it, about one.
    r, wall = run(model, mode, 2048, 8, 3, 4, 200)
    assert r.returncode == 0 and r.stdout.startswith("aborted"), r.stdout + r.stderr
    assert wall < 5.0


def test_bounded_waits_without_abort_add_up(model):
    r, wall = run(model, "stale_no_abort", 200, 4, 2, 4, 5)
    assert r.returncode == 0, r.stdout + r.stderr
    assert wall >= 0.5                  # 200 waits x 5 ms, not one bound


def test_protocol_is_race_free_under_thread_sanitizer(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "ring_tsan")
    b = subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=thread", "-pthread", SRC,
                        "-o", exe], capture_output=True, text=True)
    if b.returncode != 0:
        pytest.skip("ThreadSanitizer build not available: " + b.stderr[-200:])
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1:exitcode=66")
    r = subprocess.run([exe, "normal", "512", "8", "3", "4", "10000"], capture_output=True,
                       text=True, timeout=120, env=env)
    assert r.returncode == 0 and "checked 4096 bad 0" in r.stdout, r.stdout + r.stderr
