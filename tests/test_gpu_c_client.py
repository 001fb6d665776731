"""The C ABI from a plain C program (tests/c_client.c, built by build()):
current per-tensor E4M3 scaling of the 65,536-element fp32 workload --
amax, scale update, cast -- with no Python between the caller and the
library, against the oracle."""

import os
import struct
import subprocess
from fractions import Fraction

import numpy as np
import pytest

import workloads
from oracle import E4M3, bulk
from oracle.cast import scale_exponent

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "c_client")


def test_c_client_current_scaling(tmp_path):
    if not os.path.exists(EXE):
        pytest.fail("tests/c_client is not built (run __graft_entry__.build())")
    x = workloads.per_tensor_small()
    x[3], x[4] = np.float32(1e-30), np.float32(-2.5e3)      # an underflow and the amax
    inp, codes_p, counts_p, state_p = (str(tmp_path / f) for f in ("x.bin", "codes.bin", "counts.bin", "st.bin"))
    x.tofile(inp)
    r = subprocess.run([EXE, inp, codes_p, counts_p, state_p], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    x64 = x.astype(np.float64)
    k = scale_exponent(E4M3, Fraction(float(np.max(np.abs(x64)))))
    want_codes, clip, uf, nf = bulk.cast_f64(E4M3, x64, k)
    codes = np.fromfile(codes_p, dtype=np.uint8)
    assert np.array_equal(codes, want_codes)
    n_finite, n_clip, n_uf, n_nf, amax_bits, _ = struct.unpack("<4Q2I", open(counts_p, "rb").read())
    assert (n_finite, n_clip, n_uf, n_nf) == (x.size, int(np.count_nonzero(clip)), int(np.count_nonzero(uf)), 0)
    assert amax_bits == int(np.max(np.abs(x)).view(np.uint32))
    st = struct.unpack("<i5i", open(state_p, "rb").read())
    assert st[0] == k
