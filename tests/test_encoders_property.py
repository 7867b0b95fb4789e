"""Property-based check (hypothesis, derandomized) that the library's host
encoders and the independent numpy encoders agree byte for byte on random
inputs: shapes with ragged edges, both tile widths the kernels use, masks of
any density, +0 / -0 entries kept by the mask, and values drawn from a small
pool so that equal magnitudes are common.  Covers the tiled format and the
column-run encoding derived from it."""
import numpy as np
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
import sparse_weight_matmul_amd as swm

POOL = np.array([0.0, -0.0, 0.5, -0.5, 1.0, -1.0, 0.015625, -0.015625, 6.0e-5, -6.0e-5, 2.0],
                dtype=np.float16)


@st.composite
def cases(draw):
    M = draw(st.integers(1, 300))
    K = draw(st.integers(1, 200))
    tk = draw(st.sampled_from([32, 64]))
    density = draw(st.sampled_from([0.0, 0.05, 0.5, 0.95, 1.0]))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    null_mask = draw(st.booleans())
    g = np.random.default_rng(seed)
    W = POOL[g.integers(0, len(POOL), size=(M, K))]
    mask = None if null_mask else g.random((M, K)) < density
    return W, mask, tk


@settings(max_examples=60, deadline=None, derandomize=True, suppress_health_check=[HealthCheck.too_slow])
@given(cases())
def test_encoders_agree_byte_for_byte(case):
    W, mask, tk = case
    blob = swm.encode_blob(W, mask, tile=(16, tk))
    assert blob == oracle.tcb_encode(W, mask, TK=tk).blob()
    assert swm.validate_blob(blob) == 0
    assert swm.colruns_encode_blob(blob) == oracle.colruns_encode(W, mask).blob()
