"""The library driven from plain C (tests/c_client/tp_c_client.c): the header,
the enums, struct tp_plan and every entry point, with device memory from the
HIP runtime's C API, results compared bit for bit with the oracle."""
import os

import pytest

from software_pipelining_amd import tilepipe
from tests import c_client


@pytest.fixture(scope="module")
def client():
    if not os.path.exists(tilepipe.library_path()):
        pytest.skip("libtilepipe.so is not built")
    if not os.path.exists(c_client.LIB) or (
            os.path.getmtime(c_client.LIB) < os.path.getmtime(c_client.SRC)):
        c_client.build()
    return c_client


def test_c_client_host_mode(client):
    """Planning, argument errors, status strings and workspace sizes from C;
    no device is touched."""
    st, msg = client.run("host")
    assert st == 0, msg


def test_c_client_rejects_unknown_mode(client):
    st, msg = client.run("neither")
    assert st == 2 and "unknown mode" in msg


@pytest.mark.gpu
def test_c_client_gpu_mode(client):
    """Every entry point from C on device 0: the row exchange, the 1-D map (three
    ops, a source off its 16-byte boundary, in place with the 4-byte fallback,
    argument errors), the 2-D map, chunk copies of 16, 8 and 4 bytes, and both
    copies between workgroups, each against the oracle."""
    st, msg = client.run("gpu")
    assert st == 0, msg
