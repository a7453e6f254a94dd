"""The chunkwise WY equations (forward and adjoint) reproduce the fp64 oracle.

This pins the chunk algebra the HIP kernels implement, independently of the
GPU, at chunk sizes 1, 4, 16 and 64 (C = 1 is the token loop itself)."""
import numpy as np
import pytest

import oracle
import wy_model


def _case(seed, T=70, dk=6, dv=5):
    r = np.random.default_rng(seed)
    u = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    q, k = u(r.standard_normal((T, dk))), u(r.standard_normal((T, dk)))
    v = r.standard_normal((T, dv))
    la = -np.abs(r.standard_normal((T, dk))) * 0.2
    b = 2 / (1 + np.exp(-r.standard_normal((T, dk))))
    w = 1 / (1 + np.exp(-r.standard_normal((T, dv))))
    S0 = r.standard_normal((dk, dv)) * 0.3
    dO = r.standard_normal((T, dv))
    dSf = r.standard_normal((dk, dv)) * 0.1
    return q, k, v, la, b, w, S0, dO, dSf


def _o(x):
    return x[None, :, None, :]


@pytest.mark.parametrize("C", [1, 4, 16, 64])
def test_chunk_forward_equals_oracle(C):
    q, k, v, la, b, w, S0, _, _ = _case(C)
    O, S, _ = wy_model.fwd(q, k, v, la, b, w, S0, C)
    o_ref, s_ref = oracle.fwd(_o(q), _o(k), _o(v), _o(la), _o(b), _o(w), S0[None, None])
    np.testing.assert_allclose(O, o_ref[0, :, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(S, s_ref[0, 0], rtol=0, atol=1e-12)


@pytest.mark.parametrize("C", [1, 4, 16, 64])
def test_chunk_adjoint_equals_oracle_backward(C):
    q, k, v, la, b, w, S0, dO, dSf = _case(100 + C)
    g = wy_model.bwd(q, k, v, la, b, w, S0, dO, dSf, C)
    ref = oracle.bwd(_o(q), _o(k), _o(v), _o(la), _o(b), _o(w), S0[None, None], _o(dO), dSf[None, None])
    for n in ("dq", "dk", "dv", "dlog_alpha", "db", "dw"):
        np.testing.assert_allclose(g[n], ref[n][0, :, 0], rtol=0, atol=1e-11, err_msg=n)
    np.testing.assert_allclose(g["dS0"], ref["dS0"][0, 0], rtol=0, atol=1e-11)
