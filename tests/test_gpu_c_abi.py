"""The C ABI from plain C on the GPU: tests/c/abi_demo (built by build())
runs a three-step constrained search with device logits it allocates through
the HIP runtime -- no Python or torch in that process -- and checks each
step against the C oracle."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEMO = os.path.join(ROOT, "tests", "c", "abi_demo")


def test_plain_c_search_matches_oracle():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(DEMO):
        pytest.fail("tests/c/abi_demo is not built (run __graft_entry__.build())")
    r = subprocess.run([DEMO], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout
    assert "ok: C ABI search matches the oracle" in r.stdout
