"""The stored tuner references (tests/golden/tune_refs_*.npz)
are what the oracle computes on the seeded reference inputs: the small
context's terms are recomputed here and compared (fp32-rounded fp64 values;
a BLAS summation order may move the last bit), the large ones checked for
shape and finiteness."""

import os

import numpy as np

from tests.golden import make_tune_refs as mk


def test_stored_tuner_references_match_the_oracle():
    z = np.load(mk.OUT)                  # allow_pickle=False (the default)
    dec, ver, sigma = mk.reference_terms("small")
    np.testing.assert_allclose(z["decode_small"], dec, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(z["verify_small"], ver, rtol=1e-6, atol=1e-6)
    assert np.array_equal(z["sigma_small"], sigma.astype(np.float32))
    assert z["decode_large"].shape == (32, 128) and z["verify_large"].shape == (8, 32, 128)
    assert np.all(np.isfinite(z["decode_large"])) and np.all(np.isfinite(z["verify_large"]))
    # the verify term's last draft sees everything; its first draft sees the decode term's
    # context plus itself, so the two differ
    assert not np.allclose(z["decode_small"], z["verify_small"][0])


def test_stored_session_references_match_the_oracle():
    """The multi-session terms (tests/golden/tune_refs_32q4kv_d128_s16.npz):
    the small one recomputed, the large one checked for shape and
    finiteness."""
    z = np.load(mk.SESSIONS_OUT)
    out, sigma = mk.session_terms("small")
    np.testing.assert_allclose(z["multi_session_small"], out, rtol=1e-6, atol=1e-6)
    assert np.array_equal(z["sigma_small"], sigma.astype(np.float32))
    assert z["multi_session_large"].shape == (16, 32, 128)
    assert np.all(np.isfinite(z["multi_session_large"]))
    # the sessions share a prefix but not their suffixes or queries
    assert not np.allclose(z["multi_session_small"][0], z["multi_session_small"][1])
