"""The fp64 oracle against facts the pages and mathematics fix (CPU only)."""
import pytest

import oracle
from pins import PINS


@pytest.mark.parametrize("name,pin", PINS, ids=[n for n, _ in PINS])
def test_pin(name, pin):
    pin(oracle.load())


def test_tiny_workload_matches_bruteforce():
    """The tiny fp32 workload (B1 Hq2 Hkv1 T64 d32 L4) through both formulations."""
    import numpy as np
    from bruteforce import moda_bruteforce
    from synth import WORKLOADS, numpy_inputs
    x = numpy_inputs(WORKLOADS["tiny"])
    out, lse = oracle.moda_forward(x["q"], x["k"], x["v"], x["kd"], x["vd"])
    ref, rlse = moda_bruteforce(*(x[n].astype(np.float64) for n in ("q", "k", "v", "kd", "vd")))
    assert np.max(np.abs(out - ref)) <= 1e-12
    assert np.max(np.abs(lse - rlse)) <= 1e-12


def test_rejects_bad_shapes():
    import numpy as np
    lib = oracle.load()
    z = np.zeros(8)
    # Hq not a multiple of Hkv
    assert lib.oracle_moda_fwd(1, 3, 2, 1, 0, 4, oracle.F64, z.ctypes.data, z.ctypes.data,
                               z.ctypes.data, None, None, z.ctypes.data, None) != 0
    # T = 0
    assert lib.oracle_moda_fwd(1, 2, 1, 0, 0, 4, oracle.F64, z.ctypes.data, z.ctypes.data,
                               z.ctypes.data, None, None, z.ctypes.data, None) != 0
