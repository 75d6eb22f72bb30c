import os
import shutil
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

FULL_TESTS = "test_gpu_zfull_configs.py"


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload (minutes of CPU oracle time)")
    _start_oracle_worker(config)


def _gpu_run_selected(config) -> bool:
    mark = (config.getoption("markexpr", "") or "").replace(" ", "")
    if "gpu" not in mark or "notgpu" in mark:
        return False
    if not os.path.exists("/dev/kfd"):          # no GPU on this host
        return False
    here = os.path.dirname(os.path.abspath(__file__))
    for a in [a.split("::")[0] for a in config.args] or ["."]:
        p = os.path.abspath(a)
        if p == os.path.join(here, FULL_TESTS) or (os.path.isdir(p) and (here + os.sep).startswith(p.rstrip(os.sep) + os.sep)):
            return True
    return False


def _start_oracle_worker(config):
    """The full-size workloads' oracle results, computed by a separate process
    while the other GPU tests run; started here, before any test touches the
    device (tests/full_parity.py explains)."""
    config._lopt_oracle = None
    if os.environ.get("LOPT_FULL_PARITY_INLINE") or not _gpu_run_selected(config):
        return
    base = "/dev/shm" if os.path.isdir("/dev/shm") and os.access("/dev/shm", os.W_OK) else None
    root = tempfile.mkdtemp(prefix="lopt_full_parity_", dir=base)
    log = open(os.path.join(root, "worker.log"), "w")
    proc = subprocess.Popen([sys.executable, os.path.join(ROOT, "tests", "full_parity_worker.py"), root],
                            stdout=log, stderr=subprocess.STDOUT, cwd=ROOT)
    config._lopt_oracle = (proc, root, log)
    os.environ["LOPT_FULL_PARITY_DIR"] = root


def pytest_unconfigure(config):
    job = getattr(config, "_lopt_oracle", None)
    if not job:
        return
    proc, root, log = job
    if proc.poll() is None:
        proc.terminate()
        try:
            proc.wait(timeout=30)
        except subprocess.TimeoutExpired:
            proc.kill()
            proc.wait()
    log.close()
    shutil.rmtree(root, ignore_errors=True)
