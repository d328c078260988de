"""The C ABI used from C++ with plain HIP device buffers: the client in
tests/c_client (built by __graft_entry__.build()) calibrates, writes and
decodes, plain and with the newest tokens appended, through libkvq, and checks
every result against the C oracle itself (scales and cache bytes bit-exact,
attention within 2e-3 globally and per row, the append identical to
write-then-decode), plus two host-side refusals.  One run per cache format."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

CLIENT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_client", "kvq_c_client")


@pytest.mark.parametrize("fmt", [0, 1, 2])  # E4M3, E5M2, INT8
def test_c_client(fmt):
    assert os.path.exists(CLIENT), "the C client is not built: run __graft_entry__.build()"
    r = subprocess.run([CLIENT, str(fmt)], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stdout[-2000:]
    assert "all checks passed" in r.stdout
