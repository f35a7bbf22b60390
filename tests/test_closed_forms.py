"""The closed forms used at full length (tests/closed_forms.py) against the
oracle on a small case (CPU only): q = 0, one causal document, chunks and
blocks smaller than the sequence so that every carry is exercised."""
import numpy as np
import pytest


@pytest.mark.parametrize("theta", [0.0, 5e7])
def test_zero_query_closed_forms_match_oracle(oracle, theta):
    from closed_forms import zero_query_closed_forms

    rng = np.random.Generator(np.random.PCG64(12))
    S, D = 700, 16
    k, v, do = (rng.standard_normal((S, D)) for _ in range(3))
    q = np.zeros((1, 1, S, D))
    scale = 1.0 / np.sqrt(D)
    ro, rlse = oracle.attn_fwd(q, k[None, None], v[None, None], None, None, theta=theta)
    rdq, rdk, rdv = oracle.attn_bwd(q, k[None, None], v[None, None], do[None, None], None, None, theta=theta)
    assert np.allclose(rlse[0, 0], np.log(np.arange(1, S + 1)), rtol=0, atol=1e-12)
    assert np.array_equal(rdk, np.zeros_like(rdk))
    seen = 0
    for sl, o_ref, dv_ref, dq_ref in zero_query_closed_forms(oracle, k, v, do, theta, scale, chunk_rows=256,
                                                             block=100):
        assert np.allclose(o_ref, ro[0, 0, sl], rtol=0, atol=1e-12)
        assert np.allclose(dv_ref, rdv[0, 0, sl], rtol=0, atol=1e-12)
        assert np.allclose(dq_ref, rdq[0, 0, sl], rtol=0, atol=1e-11)
        seen += sl.stop - sl.start
    assert seen == S
