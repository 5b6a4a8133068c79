"""The chunkwise form the kernels implement equals the oracle's token recurrence in fp64."""
import numpy as np
import pytest

import oracle
from chunk_form import chunked_forward


@pytest.mark.parametrize("C", [16, 64])
def test_chunked_form_is_exact(C):
    rng = np.random.default_rng(3)
    ntok, H, dk, dv = 300, 2, 32, 24
    q = rng.standard_normal((ntok, H, dk))
    k = rng.standard_normal((ntok, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((ntok, H, dv))
    g = -np.exp(rng.uniform(0, np.log(16), H)) * np.log1p(np.exp(rng.standard_normal((ntok, H)) - 4.6))
    beta = 1 / (1 + np.exp(-rng.standard_normal((ntok, H))))
    S0 = rng.standard_normal((3, H, dk, dv)) * 0.1
    cu = [0, 130, 131, 300]           # ragged: partial chunks, a one-token sequence
    y_ref, s_ref = oracle.recurrence(q, k, v, np.exp(g), beta, S0, cu)
    y, s = chunked_forward(q, k, v, g, beta, S0, cu, C=C)
    assert np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref) < 1e-12
    assert np.linalg.norm(s - s_ref) / np.linalg.norm(s_ref) < 1e-12


@pytest.mark.parametrize("C", [16, 64])
def test_chunked_backward_is_exact(C):
    from chunk_form import chunked_backward
    rng = np.random.default_rng(4)
    ntok, H, dk, dv = 200, 2, 16, 12
    q = rng.standard_normal((ntok, H, dk))
    k = rng.standard_normal((ntok, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((ntok, H, dv))
    g = -np.exp(rng.uniform(0, np.log(16), H)) * np.log1p(np.exp(rng.standard_normal((ntok, H)) - 4.6))
    beta = 1 / (1 + np.exp(-rng.standard_normal((ntok, H))))
    S0 = rng.standard_normal((3, H, dk, dv)) * 0.1
    dy = rng.standard_normal((ntok, H, dv))
    dST = rng.standard_normal((3, H, dk, dv))
    cu = [0, 90, 91, 200]
    ref = oracle.recurrence_backward(q, k, v, np.exp(g), beta, dy, S0, dST, cu)
    got = chunked_backward(q, k, v, g, beta, dy, S0, dST, cu, C=C)
    for key in ("dq", "dk", "dv", "dg", "dbeta", "dS0"):
        err = np.linalg.norm(got[key] - ref[key]) / np.linalg.norm(ref[key])
        assert err < 1e-11, (key, err)


@pytest.mark.parametrize("C", [16, 64])
def test_chunked_kda_form_is_exact(C):
    from chunk_form import chunked_forward_kda
    rng = np.random.default_rng(5)
    ntok, H, dk, dv = 150, 2, 12, 10
    q = rng.standard_normal((ntok, H, dk))
    k = rng.standard_normal((ntok, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((ntok, H, dv))
    g = -5.0 / (1.0 + np.exp(-rng.standard_normal((ntok, H, dk))))     # log-decay in (-5, 0)
    beta = 1 / (1 + np.exp(-rng.standard_normal((ntok, H))))
    S0 = rng.standard_normal((2, H, dk, dv)) * 0.1
    cu = [0, 70, 150]
    y_ref, s_ref = oracle.kda_recurrence(q, k, v, np.exp(g), beta, S0, cu)
    y, s = chunked_forward_kda(q, k, v, g, beta, S0, cu, C=C)
    assert np.linalg.norm(y - y_ref) / np.linalg.norm(y_ref) < 1e-12
    assert np.linalg.norm(s - s_ref) / np.linalg.norm(s_ref) < 1e-12
