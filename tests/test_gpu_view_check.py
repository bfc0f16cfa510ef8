"""The debug mode that checks views on the host (SE_CHECK_VIEWS=1) rejects views
whose entries fall outside the cache before launching anything.  The environment
switch is read once per process, so the case runs in a child process."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu


def test_view_checks_in_a_child_process(se):
    script = os.path.join(os.path.dirname(os.path.abspath(__file__)), "view_check_case.py")
    env = dict(os.environ, SE_CHECK_VIEWS="1")
    r = subprocess.run([sys.executable, script], capture_output=True, text=True, env=env, timeout=240)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "view checks ok" in r.stdout
