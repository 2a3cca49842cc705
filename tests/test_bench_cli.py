"""bench.py's command line on a host without a GPU: it measures one GPU only,
so a request for more (a flag, or a launcher's WORLD_SIZE) ends with status
2 and a message before anything touches a device."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("argv,env", [
    (["--gpus", "2"], {}),
    (["--gpus", "8", "--steps", "1"], {}),
    ([], {"WORLD_SIZE": "4"}),
])
def test_more_than_one_gpu_is_refused(argv, env):
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], cwd=ROOT, env=e,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""   # no JSON line for a refused run
