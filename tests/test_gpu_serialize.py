"""Stream-ordering races: every schedule gives the same bits when the runtime serialises
kernels and copies (AMD_SERIALIZE_KERNEL=3, AMD_SERIALIZE_COPY=3) as when it overlaps them.
Each run is a child process (tests/serialize_child.py) that prints one digest per output."""

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

CHILD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "serialize_child.py")


def _run(extra_env):
    env = dict(os.environ, **extra_env)
    r = subprocess.run([sys.executable, "-u", CHILD], capture_output=True, text=True, timeout=240, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    lines = [ln for ln in r.stdout.splitlines() if ln and not ln.startswith("[")]
    return dict(ln.rsplit(" ", 1) for ln in lines)


def test_serialised_runs_match_overlapped():
    print("[serialize] overlapped run", flush=True)
    free = _run({})
    print("[serialize] serialised run", flush=True)
    ser = _run({"AMD_SERIALIZE_KERNEL": "3", "AMD_SERIALIZE_COPY": "3"})
    assert free["timeouts"] == "0" and ser["timeouts"] == "0"
    assert len(free) == 9 and free == ser, (free, ser)
