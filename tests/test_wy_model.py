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


def test_factored_reverse_step_equals_the_chunk_adjoint():
    """The reverse sweep's factored form: with W = T Et, the state gradient passed to the
    previous chunk, Qt^T dO + diag(gamma) dS' - Et^T T^T (P^T dO + Kh dS'), equals
    R dS' + Q2^T dO with R = (I - W^T Kt) diag(gamma) and Q2 = Qt - P W."""
    q, k, v, la, b, w, S0, dO, dSf = _case(11, T=64)
    G, gC, Et, Kt, Qt, Kh, A, P, T, Z = wy_model._chunk_quantities(q, k, v, la, b, w)
    gam = np.exp(gC)
    dU = P.T @ dO + Kh @ dSf
    dX = T.T @ dU
    recurrence = Qt.T @ dO + gam[:, None] * dSf - Et.T @ dX
    W = T @ Et
    R = (np.eye(len(gam)) - W.T @ Kt) * gam[None, :]
    Q2 = Qt - P @ W
    factored = R @ dSf + Q2.T @ dO
    assert np.max(np.abs(factored - recurrence)) <= 1e-12 * np.max(np.abs(recurrence))
    # and the chunk adjoint of the model itself hands the same gradient to the previous chunk
    g = wy_model.bwd(q, k, v, la, b, w, S0, dO, dSf, C=64)
    assert np.max(np.abs(g["dS0"] - factored)) <= 1e-12 * np.max(np.abs(factored))


def test_chunk_map_is_affine_in_the_start_state():
    """S' = M S + N with M = diag(gamma) - Kh^T T Et and N = Kh^T T Z: the composite a
    sequence split across devices would exchange (two chunks compose by M2 M1, M2 N1 + N2)."""
    q, k, v, la, b, w, S0, dO, dSf = _case(12, T=128)
    mats = []
    for sl in (slice(0, 64), slice(64, 128)):
        G, gC, Et, Kt, Qt, Kh, A, P, T, Z = wy_model._chunk_quantities(q[sl], k[sl], v[sl], la[sl], b[sl], w[sl])
        mats.append((np.diag(np.exp(gC)) - Kh.T @ T @ Et, Kh.T @ T @ Z))
    (M1, N1), (M2, N2) = mats
    _, S_final, _ = wy_model.fwd(q, k, v, la, b, w, S0, C=64)
    composed = M2 @ (M1 @ S0 + N1) + N2
    assert np.max(np.abs(composed - S_final)) <= 1e-12 * np.max(np.abs(S_final))
    # the same through the oracle's token loop
    _, S_ref = oracle.fwd(*[_o(x) for x in (q, k, v, la, b, w)], S0[None, None])
    assert np.max(np.abs(composed - S_ref[0, 0])) <= 1e-12 * np.max(np.abs(S_ref))
