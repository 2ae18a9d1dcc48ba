"""CPU pins of the rounding models the GPU tests compare the kernels with
(tests/_util.py): each is held to closed forms and to the fp64 oracle."""
import numpy as np

import oracle
import synthdata
from _util import attention_fwd_rounding_model, attention_bwd_rounding_model, max_rel_err


def test_attention_rounding_model_pins():
    """The attention rounding model (tests/_util.py, used to check the
    matrix-core kernels bit for bit) is pinned to closed forms and to the
    fp64 oracle: with q = 0 every score is 0, so every weight is exactly 1
    and row i averages v over keys 0..i -- with v = 1 the output is exactly
    1 and the log-sum-exp ln(i + 1); on random bf16 inputs it stays within
    the bf16 bars the kernels meet against the oracle."""
    T, Q = 192, 128
    o, lse = attention_fwd_rounding_model(np.zeros((T, Q)), np.ones((T, Q)), np.ones((T, Q)))
    assert np.all(o == 1.0)
    np.testing.assert_allclose(lse, np.log(np.arange(1, T + 1)), rtol=1e-6, atol=1e-6)
    rng = np.random.default_rng(5)
    q, k, v, do = (synthdata.round_to_bf16(rng.standard_normal((T, Q)).astype(np.float32)).astype(np.float64)
                   for _ in range(4))
    o, lse = attention_fwd_rounding_model(q, k, v)
    assert max_rel_err(o, oracle.causal_attention(q[:, None], k[:, None], v[:, None])[:, 0]) <= 1e-2
    got = attention_bwd_rounding_model(q, k, v, o, lse, do)
    want = oracle.causal_attention_bwd(q[:, None], k[:, None], v[:, None], do[:, None])
    for g, w in zip(got, want):
        assert max_rel_err(g, w[:, 0]) <= 2e-2
