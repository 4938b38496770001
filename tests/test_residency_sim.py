"""The arena's residency protocol on the CPU (EStream section 3.3: no expert
executes before its parameters are ready; no slot is overwritten while a
queued invocation still references it).

tests/residency_sim.cpp runs the library's own residency table
(routed_expert_ffn_top_amd/csrc/residency.h) on a fake copy backend: worker
threads play the copy and compute streams, copies and invocations proceed
in chunks with random pauses, and every invocation checks each byte of the
slots it reads. The paged layer's schedule (banks loaded before routing,
groups skipped, banks reused longest-released first) runs over many layer
calls on two compute streams. With the protocol no invocation sees a partly
loaded or overwritten slot; with its waits dropped (the control) the same
check sees violations. The protocol run is also built with ThreadSanitizer:
its copies and reads are ordered by the events alone, with no data race.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "residency_sim.cpp")
INC = [f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.join(ROOT, 'routed_expert_ffn_top_amd', 'csrc')}"]


def _build(tmp_path, name, extra):
    exe = str(tmp_path / name)
    subprocess.run(["g++", "-std=c++17", "-pthread", "-Wall", *extra, *INC, SRC, "-o", exe], check=True)
    return exe


@pytest.fixture(scope="module")
def sim(tmp_path_factory):
    return _build(tmp_path_factory.mktemp("rsim"), "residency_sim", ["-O2"])


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_protocol_has_no_violation(sim, seed):
    r = subprocess.run([sim, "correct", "60", str(seed)], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert " 0 violations" in r.stdout


def test_dropped_waits_are_detected(sim):
    r = subprocess.run([sim, "control", "20", "4"], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, "the check saw no violation with the waits dropped: " + r.stdout + r.stderr


def test_protocol_under_thread_sanitizer(tmp_path):
    exe = _build(tmp_path, "residency_sim_tsan", ["-O1", "-g", "-fsanitize=thread"])
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1 exitcode=66")
    r = subprocess.run([exe, "correct", "20", "5"], capture_output=True, text=True, timeout=300, env=env)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr[-3000:]
    assert "ThreadSanitizer" not in r.stderr
