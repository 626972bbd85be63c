"""The C interface from a plain C caller (tests/c_abi/ob_c_driver.c: no
Python, no torch, device memory from hipMalloc): warm-up and compressed steps
for the few-worker, generic and subtree-table server forms, every field read
back through ob_adam_get_state and compared with the CPU oracle; error paths
and the workspace guards; then a 0/1 Adam handle through local steps,
synchronizations and a variance refresh, every field (the open period's local
ones too) bit-identical to the oracle's.  The driver runs as a child process."""
import os
import subprocess

import pytest

from gpu_common import log

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "c_abi", "ob_c_driver")


@pytest.mark.parametrize("d,n", [(4 * 3392, 4), (5 * 2112, 5), (8 * 3392, 8), (16 * 448, 16)])
def test_c_caller_matches_oracle(d, n):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(DRIVER):
        raise RuntimeError("the C driver is not built: run __graft_entry__.build()")
    log("c driver d=%d n=%d" % (d, n))
    r = subprocess.run([DRIVER, str(d), str(n)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c driver ok" in r.stdout
