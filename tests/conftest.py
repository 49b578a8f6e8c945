import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload cases")


def read_golden(name):
    """Rows of a whitespace-separated fixture, comments stripped."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


@pytest.fixture(scope="session")
def rocrand_kat(tmp_path_factory):
    """Philox4x32-10 block outputs from rocRAND's header implementation of
    the published generator (Salmon et al., SC'11), compiled here as a
    host-only helper (tests/philox_kat/): an independent source of known
    answers for the oracle's generator and of SR draws for the brute-force
    checks.  Takes rows (key, c0, c1, c2, c3) and returns the four words of
    each."""
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand"):
        pytest.skip("rocRAND headers / hipcc not available")
    exe = str(tmp_path_factory.mktemp("kat") / "kat")
    src = os.path.join(ROOT, "tests", "philox_kat", "rocrand_philox_kat.cpp")
    subprocess.run([hipcc, "--offload-host-only", "-O1", src, "-o", exe], check=True,
                   capture_output=True)

    def run(rows):
        inp = "".join("%d %d %d %d %d\n" % tuple(r) for r in rows)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True)
        return [list(map(int, line.split())) for line in out.stdout.strip().splitlines()]
    return run
