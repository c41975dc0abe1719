"""The plain-C example of the ABI (contextual_head_sparsity_amd/examples/
decode_c.c) runs on the GPU: hipMalloc'd buffers, a head-indexed call whose
keys the library splits (its own workspace, then the combine) and a
group-indexed call, each checked against the closed form for q = 0 (outputs
equal the mean of V) with unselected slots untouched; then the router on
unit-vector weights (known scores and top-k) feeding a decode call, the
router's K-split form with a caller workspace on f16 small integers, and the
union + selective MLP on small integers, checked for exact equality."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "contextual_head_sparsity_amd", "examples", "decode_c")


def test_c_example_runs_and_passes():
    if not os.path.exists(EXE):
        raise RuntimeError(f"{EXE} is not built (run __graft_entry__.build())")
    print("[example] decode_c", flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().splitlines()[-1] == "PASS"
    assert r.stdout.count("unselected slots untouched: yes") == 3
    assert "scores exact: yes" in r.stdout
    assert "split scores exact: yes" in r.stdout
    assert "y exact" in r.stdout and "union: 5 neurons [3 7 12 30 39]" in r.stdout
