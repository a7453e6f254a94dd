"""Pins for the fp64 oracle: each test checks it against something other than itself.

Sources (Gated DeltaNet-2 pages):
* the per-token rule and its two reductions -- iplexlaw.co.kr blog, section
  "Independent control on two axes" (decay first, read through e = b*k, write
  along k, query reads the updated state; equal scalar gates give KDA, a scalar
  decay as well gives Gated DeltaNet); the paper abstract (OpenAlex record)
  states the same two reductions.
* the gate-aware backward -- same blog, section "Token path and parallel
  training"; pinned here by central finite differences.

A plausible slip in the oracle (a dropped term, a wrong sign, the wrong gate on
the wrong axis, reading the state before instead of after the write, decaying
after the read, a missing checkpoint) fails at least one of these tests; see
test_planted_mistakes_are_caught, which plants such slips in a copy of the rule
and checks that the pins notice.
"""
import numpy as np
import pytest

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _case(seed, B=2, T=12, H=2, dk=6, dv=5, s0=0.3, la_scale=0.3):
    r = _rng(seed)
    q = _unit(r.standard_normal((B, T, H, dk)))
    k = _unit(r.standard_normal((B, T, H, dk)))
    v = r.standard_normal((B, T, H, dv))
    la = -np.abs(r.standard_normal((B, T, H, dk))) * la_scale
    b = 1 / (1 + np.exp(-r.standard_normal((B, T, H, dk))))
    w = 1 / (1 + np.exp(-r.standard_normal((B, T, H, dv))))
    S0 = r.standard_normal((B, H, dk, dv)) * s0
    return q, k, v, la, b, w, S0


# ---------------------------------------------------------------------------
# forward pins
# ---------------------------------------------------------------------------

def _kda_matrix_form(q, k, v, la, beta, S0):
    """KDA: S_t = (I - beta k k^T) diag(alpha_t) S_{t-1} + beta k v^T, o_t = S_t^T q_t.
    Written with dense dk x dk transition matrices (a different evaluation order
    from the oracle's per-channel loops)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    SF = np.zeros((B, H, dk, dv))
    I = np.eye(dk)
    for bb in range(B):
        for h in range(H):
            S = S0[bb, h].copy()
            for t in range(T):
                kk = k[bb, t, h][:, None]
                be = beta[bb, t, h]
                S = (I - be * kk @ kk.T) @ np.diag(np.exp(la[bb, t, h])) @ S + be * kk @ v[bb, t, h][None, :]
                o[bb, t, h] = S.T @ q[bb, t, h]
            SF[bb, h] = S
    return o, SF


def test_reduces_to_kda_when_gates_share_a_scalar():
    q, k, v, la, _, _, S0 = _case(1)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    beta = 1 / (1 + np.exp(-_rng(2).standard_normal((B, T, H))))
    b = np.broadcast_to(beta[..., None], (B, T, H, dk)).copy()
    w = np.broadcast_to(beta[..., None], (B, T, H, dv)).copy()
    o, sf = oracle.fwd(q, k, v, la, b, w, S0)
    o_ref, sf_ref = _kda_matrix_form(q, k, v, la, beta, S0)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(sf, sf_ref, rtol=0, atol=1e-13)


def test_reduces_to_gated_deltanet_when_decay_is_scalar_too():
    q, k, v, _, _, _, S0 = _case(3)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    r = _rng(4)
    beta = 1 / (1 + np.exp(-r.standard_normal((B, T, H))))
    alpha = 1 / (1 + np.exp(-(r.standard_normal((B, T, H)) + 3)))
    la = np.broadcast_to(np.log(alpha)[..., None], (B, T, H, dk)).copy()
    b = np.broadcast_to(beta[..., None], (B, T, H, dk)).copy()
    w = np.broadcast_to(beta[..., None], (B, T, H, dv)).copy()
    o, sf = oracle.fwd(q, k, v, la, b, w, S0)
    # Gated DeltaNet: S_t = alpha_t (I - beta k k^T) S_{t-1} + beta k v^T
    o_ref = np.zeros_like(o)
    sf_ref = np.zeros_like(sf)
    I = np.eye(dk)
    for bb in range(B):
        for h in range(H):
            S = S0[bb, h].copy()
            for t in range(T):
                kk = k[bb, t, h][:, None]
                S = alpha[bb, t, h] * (I - beta[bb, t, h] * kk @ kk.T) @ S + beta[bb, t, h] * kk @ v[bb, t, h][None, :]
                o_ref[bb, t, h] = S.T @ q[bb, t, h]
            sf_ref[bb, h] = S
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(sf, sf_ref, rtol=0, atol=1e-13)


def test_read_after_write_returns_the_written_value():
    """b = 1 and unit k: S_t^T k_t = z_t = w_t * v_t for any decay, write gate and
    start state.  Querying with q_t = k_t exposes S_t^T k_t as the output."""
    q, k, v, la, _, w, S0 = _case(5, T=40, la_scale=1.5, s0=2.0)
    b = np.ones_like(k)
    o, _ = oracle.fwd(k, k, v, la, b, w, S0)
    np.testing.assert_allclose(o, w * v, rtol=0, atol=1e-13)


def _brute_force(q, k, v, la, b, w, S0):
    """S_t = (M_t ... M_1) S0 + sum_j (M_t ... M_{j+1}) k_j z_j^T with dense
    M_s = (I - k_s e_s^T) diag(alpha_s); evaluated from scratch for every t."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    SF = np.zeros((B, H, dk, dv))
    I = np.eye(dk)
    for bb in range(B):
        for h in range(H):
            M = [(I - np.outer(k[bb, s, h], b[bb, s, h] * k[bb, s, h])) @ np.diag(np.exp(la[bb, s, h]))
                 for s in range(T)]
            for t in range(T):
                prod = I.copy()
                for s in range(t + 1):
                    prod = M[s] @ prod
                S = prod @ S0[bb, h]
                for j in range(t + 1):
                    P = I.copy()
                    for s in range(j + 1, t + 1):
                        P = M[s] @ P
                    S = S + P @ np.outer(k[bb, j, h], w[bb, j, h] * v[bb, j, h])
                o[bb, t, h] = S.T @ q[bb, t, h]
                if t == T - 1:
                    SF[bb, h] = S
    return o, SF


@pytest.mark.parametrize("T", [1, 2, 5, 8])
def test_brute_force_unrolled_products(T):
    args = _case(10 + T, B=1, T=T, H=2, dk=5, dv=4, la_scale=0.8, s0=1.0)
    # gates in [0, 2] as in the pages' erase-range ablation
    q, k, v, la, b, w, S0 = args
    b = 2 * b
    o, sf = oracle.fwd(q, k, v, la, b, w, S0)
    o_ref, sf_ref = _brute_force(q, k, v, la, b, w, S0)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(sf, sf_ref, rtol=0, atol=1e-13)


def test_no_erase_no_decay_is_causal_linear_attention():
    q, k, v, _, _, _, S0 = _case(20, T=30, dk=7, dv=9)
    zeros = np.zeros_like(k)
    o, sf = oracle.fwd(q, k, v, zeros, zeros, np.ones_like(v), S0)
    B, T, H, _ = q.shape
    for bb in range(B):
        for h in range(H):
            Q, K, V = q[bb, :, h], k[bb, :, h], v[bb, :, h]
            ref = Q @ S0[bb, h] + np.tril(Q @ K.T) @ V
            np.testing.assert_allclose(o[bb, :, h], ref, rtol=0, atol=1e-12)
            np.testing.assert_allclose(sf[bb, h], S0[bb, h] + K.T @ V, rtol=0, atol=1e-12)


def test_zero_keys_leave_pure_channel_decay():
    q, k, v, la, b, w, S0 = _case(21, T=25, la_scale=0.5, s0=1.0)
    o, sf = oracle.fwd(q, np.zeros_like(k), v, la, b, w, S0)
    cum = np.cumsum(la, axis=1)  # [B,T,H,dk]
    B, T, H, _ = q.shape
    for bb in range(B):
        for h in range(H):
            for t in range(T):
                St = np.exp(cum[bb, t, h])[:, None] * S0[bb, h]
                np.testing.assert_allclose(o[bb, t, h], St.T @ q[bb, t, h], rtol=0, atol=1e-13)
            np.testing.assert_allclose(sf[bb, h], np.exp(cum[bb, -1, h])[:, None] * S0[bb, h],
                                       rtol=0, atol=1e-13)


def test_chaining_two_calls_equals_one():
    q, k, v, la, b, w, S0 = _case(22, T=37)
    o, sf = oracle.fwd(q, k, v, la, b, w, S0)
    c = 15
    o1, s1 = oracle.fwd(q[:, :c], k[:, :c], v[:, :c], la[:, :c], b[:, :c], w[:, :c], S0)
    o2, s2 = oracle.fwd(q[:, c:], k[:, c:], v[:, c:], la[:, c:], b[:, c:], w[:, c:], s1)
    np.testing.assert_allclose(np.concatenate([o1, o2], 1), o, rtol=0, atol=1e-14)
    np.testing.assert_allclose(s2, sf, rtol=0, atol=1e-14)


def test_value_channel_permutation_equivariance():
    q, k, v, la, b, w, S0 = _case(23, T=20)
    perm = _rng(0).permutation(v.shape[-1])
    o, sf = oracle.fwd(q, k, v, la, b, w, S0)
    o2, sf2 = oracle.fwd(q, k, v[..., perm], la, b, w[..., perm], S0[..., perm])
    np.testing.assert_allclose(o2, o[..., perm], rtol=0, atol=1e-14)
    np.testing.assert_allclose(sf2, sf[..., perm], rtol=0, atol=1e-14)


def test_none_start_state_means_zeros():
    q, k, v, la, b, w, S0 = _case(24, T=9)
    o1, s1 = oracle.fwd(q, k, v, la, b, w, None)
    o2, s2 = oracle.fwd(q, k, v, la, b, w, np.zeros_like(S0))
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


# ---------------------------------------------------------------------------
# backward pins: central finite differences of the forward
# ---------------------------------------------------------------------------

NAMES = ["q", "k", "v", "log_alpha", "b", "w", "S0"]


def _loss(args, dO, dSf):
    o, sf = oracle.fwd(*args, nthreads=1)
    return float(np.sum(o * dO) + np.sum(sf * dSf))


def _fd_check(args, dO, dSf, idx_sets, tol):
    g = oracle.bwd(*args, dO, dSf, nthreads=1)
    gmap = dict(zip(NAMES, [g["dq"], g["dk"], g["dv"], g["dlog_alpha"], g["db"], g["dw"], g["dS0"]]))
    for ti, name in enumerate(NAMES):
        x = args[ti]
        idxs = idx_sets(x)
        fd = np.empty(len(idxs))
        an = np.empty(len(idxs))
        for n, ix in enumerate(idxs):
            h = 1e-6 * max(1.0, abs(x[ix]))
            xp = [a.copy() for a in args]
            xm = [a.copy() for a in args]
            xp[ti][ix] += h
            xm[ti][ix] -= h
            fd[n] = (_loss(xp, dO, dSf) - _loss(xm, dO, dSf)) / (2 * h)
            an[n] = gmap[name][ix]
        err = np.max(np.abs(fd - an)) / max(np.max(np.abs(fd)), 1e-30)
        assert err < tol, (name, err)


def test_gradients_match_central_differences_tiny():
    """B=1, H=1, T=16, dk=dv=8: every element of every input and of S0."""
    q, k, v, la, b, w, S0 = _case(30, B=1, T=16, H=1, dk=8, dv=8, s0=0.5, la_scale=0.4)
    b = 2 * b  # exercise the [0, 2] erase range
    r = _rng(31)
    dO = r.standard_normal(v.shape)
    dSf = r.standard_normal(S0.shape) * 0.5
    _fd_check([q, k, v, la, b, w, S0], dO, dSf, lambda x: list(np.ndindex(x.shape)), 1e-7)


def test_gradients_across_checkpoint_segments():
    """T = 150 spans three 64-token checkpoint segments with a ragged tail;
    sampled elements near and away from the segment edges."""
    q, k, v, la, b, w, S0 = _case(32, B=1, T=150, H=2, dk=4, dv=3, s0=0.5, la_scale=0.05)
    r = _rng(33)
    dO = r.standard_normal(v.shape)
    dSf = r.standard_normal(S0.shape)
    ts = [0, 1, 63, 64, 65, 127, 128, 149]

    def idx_sets(x):
        if x.ndim == 4 and x.shape[1] == 150:
            return [(0, t, t % 2, t % x.shape[-1]) for t in ts]
        return list(np.ndindex(x.shape))[:6]

    _fd_check([q, k, v, la, b, w, S0], dO, dSf, idx_sets, 1e-6)


def test_backward_none_upstream_state_gradient_means_zeros():
    args = list(_case(34, T=7))
    dO = _rng(35).standard_normal(args[2].shape)
    g1 = oracle.bwd(*args, dO, None)
    g2 = oracle.bwd(*args, dO, np.zeros_like(args[6]))
    for key in g1:
        assert np.array_equal(g1[key], g2[key])


# ---------------------------------------------------------------------------
# the pins have teeth: plant plausible slips in a copy of the rule
# ---------------------------------------------------------------------------

def _mutant(q, k, v, la, b, w, S0, slip):
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    for bb in range(B):
        for h in range(H):
            S = S0[bb, h].copy()
            for t in range(T):
                a = np.exp(la[bb, t, h])
                e = b[bb, t, h] * k[bb, t, h]
                z = w[bb, t, h] * v[bb, t, h]
                if slip == "gate_swap":      # erase gate on the write key instead
                    e = k[bb, t, h]
                    z = w[bb, t, h] * v[bb, t, h]
                    Sb = a[:, None] * S
                    r = Sb.T @ e
                    S = Sb + np.outer(b[bb, t, h] * k[bb, t, h], z - r)
                elif slip == "read_before_decay":
                    r = S.T @ e
                    S = a[:, None] * S + np.outer(k[bb, t, h], z - r)
                elif slip == "query_old_state":
                    Sb = a[:, None] * S
                    o[bb, t, h] = Sb.T @ q[bb, t, h]
                    S = Sb + np.outer(k[bb, t, h], z - Sb.T @ e)
                    continue
                elif slip == "decay_value_axis":
                    Sb = S * a[None, :dv] if dk >= dv else S
                    S = Sb + np.outer(k[bb, t, h], z - Sb.T @ e)
                elif slip == "sign":
                    Sb = a[:, None] * S
                    S = Sb + np.outer(k[bb, t, h], z + Sb.T @ e)
                o[bb, t, h] = S.T @ q[bb, t, h]
    return o


@pytest.mark.parametrize("slip", ["gate_swap", "read_before_decay", "query_old_state",
                                  "decay_value_axis", "sign"])
def test_planted_mistakes_are_caught(slip):
    """Each slip, evaluated on the brute-force pin's inputs, disagrees with the
    brute-force reference (so the same slip in the oracle would fail it)."""
    q, k, v, la, b, w, S0 = _case(40, B=1, T=6, H=1, dk=5, dv=4, la_scale=0.8, s0=1.0)
    o_ref, _ = _brute_force(q, k, v, la, b, w, S0)
    o_bad = _mutant(q, k, v, la, b, w, S0, slip)
    assert np.max(np.abs(o_bad - o_ref)) > 1e-3


def test_golden_regression_fixture():
    """Stored oracle samples (written by tests/golden/make_golden.py, oracle only)."""
    import json
    import os
    from linear_attention_sequence_gdn2_amd.inputs import WORKLOADS, make_workload
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_oracle_samples.json")
    rec = json.load(open(path))
    wl = WORKLOADS[rec["workload"]]
    x = make_workload(wl, grads=True, s0_std=rec["s0_std"])
    args = [x["q32"], x["k32"], x["v32"], x["log_alpha"], x["b"], x["w"], x["S0"]]
    o, sf = oracle.fwd(*args)
    g = oracle.bwd(*args, x["dO"], x["dS_final"])
    arrs = dict(o=o, S_final=sf, **g)
    for name, samples in rec["samples"].items():
        for ix, val in samples:
            assert abs(arrs[name][tuple(ix)] - val) <= 1e-12 * max(1.0, abs(val)), (name, ix)


# ---------------------------------------------------------------------------
# gates given as logits (log_alpha = log sigmoid, b, w = sigmoid)
# ---------------------------------------------------------------------------

def test_logit_gates_closed_forms():
    la, b, w = oracle.gates_from_logits(np.zeros(3), np.zeros(3), np.zeros(3))
    assert np.allclose(la, -np.log(2.0), rtol=0, atol=1e-15)
    assert np.allclose(b, 0.5, rtol=0, atol=1e-15) and np.allclose(w, 0.5, rtol=0, atol=1e-15)
    x = np.array([-60.0, -5.0, 2.0, 60.0])
    la, b, w = oracle.gates_from_logits(x, x, x)
    assert np.all(np.isfinite(la)) and np.all(np.isfinite(b))
    # log sigmoid(x) -> x for x -> -inf and -> -exp(-x) for x -> +inf; sigmoid(-x) = 1 - sigmoid(x)
    assert abs(la[0] - (-60.0)) < 1e-20 and abs(la[3] + np.exp(-60.0)) < 1e-40
    _, bm, _ = oracle.gates_from_logits(x, -x, x)
    assert np.allclose(bm, 1.0 - b, rtol=0, atol=1e-15)
    assert np.allclose(np.exp(la), b, rtol=1e-14, atol=0)


def test_logit_gate_gradients_match_central_differences():
    """Gradients w.r.t. the three logit tensors: the oracle's backward composed with
    the gate activations, against central differences of the composed forward."""
    q, k, v, _, _, _, S0 = _case(34, B=1, T=10, H=1, dk=4, dv=4, s0=0.5)
    r = _rng(35)
    xa = r.standard_normal(q.shape) + 3.0
    xb = r.standard_normal(q.shape)
    xw = r.standard_normal(v.shape)
    dO = r.standard_normal(v.shape)
    dSf = r.standard_normal(S0.shape) * 0.5

    def loss(xa_, xb_, xw_):
        o, sf = oracle.fwd(q, k, v, *oracle.gates_from_logits(xa_, xb_, xw_), S0, nthreads=1)
        return float(np.sum(o * dO) + np.sum(sf * dSf))

    g = oracle.bwd(q, k, v, *oracle.gates_from_logits(xa, xb, xw), S0, dO, dSf, nthreads=1)
    gl = oracle.logit_grads(xa, xb, xw, g)
    for pos, name in ((0, "dlog_alpha"), (1, "db"), (2, "dw")):
        xs = [xa, xb, xw]
        x = xs[pos]
        fd = np.empty(x.size)
        for n, ix in enumerate(np.ndindex(x.shape)):
            h = 1e-6 * max(1.0, abs(x[ix]))
            xp = [t.copy() for t in xs]
            xm = [t.copy() for t in xs]
            xp[pos][ix] += h
            xm[pos][ix] -= h
            fd[n] = (loss(*xp) - loss(*xm)) / (2 * h)
        an = gl[name].reshape(-1)
        err = np.max(np.abs(fd - an)) / max(np.max(np.abs(fd)), 1e-30)
        assert err < 1e-6, (name, err)
    for name in ("dq", "dk", "dv", "dS0"):
        assert gl[name] is g[name]


# ---------------------------------------------------------------------------
# gates given per token (one value per (b, t, h) for all channels of its axis)
# ---------------------------------------------------------------------------

def test_per_token_gates_reduce_to_kda_and_gated_deltanet():
    """beta per token on both gates is KDA; a per-token decay as well is Gated
    DeltaNet: checked against the dense matrix form written independently above."""
    q, k, v, la, _, _, S0 = _case(36, T=9)
    r = _rng(37)
    B, T, H, dk = q.shape
    beta = 1 / (1 + np.exp(-r.standard_normal((B, T, H))))
    la_tok = -np.abs(r.standard_normal((B, T, H))) * 0.3
    g = oracle.gates_per_token(la, beta, beta, dk, v.shape[-1], oracle.SCALAR_ERASE | oracle.SCALAR_WRITE)
    o, sf = oracle.fwd(q, k, v, *g, S0)
    o2, s2 = _kda_matrix_form(q, k, v, la, beta, S0)
    assert np.allclose(o, o2, rtol=0, atol=1e-12) and np.allclose(sf, s2, rtol=0, atol=1e-12)
    g = oracle.gates_per_token(la_tok, beta, beta, dk, v.shape[-1], 7)
    o, sf = oracle.fwd(q, k, v, *g, S0)
    o2, s2 = _kda_matrix_form(q, k, v, np.repeat(la_tok[..., None], dk, axis=-1), beta, S0)
    assert np.allclose(o, o2, rtol=0, atol=1e-12) and np.allclose(sf, s2, rtol=0, atol=1e-12)


@pytest.mark.parametrize("scalar", [1, 2, 4, 6, 7])
def test_per_token_gate_gradients_match_central_differences(scalar):
    """Gradients w.r.t. one scalar per token (perturbing all of its channels at once)."""
    q, k, v, la, b, w, S0 = _case(38, B=1, T=10, H=2, dk=4, dv=3, s0=0.5)
    r = _rng(39)
    tok = {1: la[..., 0].copy(), 2: b[..., 1].copy(), 4: w[..., 2].copy()}
    gates = [tok[1] if scalar & 1 else la, tok[2] if scalar & 2 else b, tok[4] if scalar & 4 else w]
    dO = r.standard_normal(v.shape)
    dSf = r.standard_normal(S0.shape) * 0.5
    dk, dv = q.shape[-1], v.shape[-1]

    def loss(gs):
        o, sf = oracle.fwd(q, k, v, *oracle.gates_per_token(*gs, dk, dv, scalar), S0, nthreads=1)
        return float(np.sum(o * dO) + np.sum(sf * dSf))

    g = oracle.bwd(q, k, v, *oracle.gates_per_token(*gates, dk, dv, scalar), S0, dO, dSf, nthreads=1)
    gt = oracle.per_token_grads(g, scalar)
    for pos, (name, bit) in enumerate((("dlog_alpha", 1), ("db", 2), ("dw", 4))):
        x = gates[pos]
        assert gt[name].shape == x.shape
        if not scalar & bit:
            assert gt[name] is g[name]
            continue
        fd = np.empty(x.size)
        for n, ix in enumerate(np.ndindex(x.shape)):
            h = 1e-6 * max(1.0, abs(x[ix]))
            xp = [t.copy() for t in gates]
            xm = [t.copy() for t in gates]
            xp[pos][ix] += h
            xm[pos][ix] -= h
            fd[n] = (loss(xp) - loss(xm)) / (2 * h)
        err = np.max(np.abs(fd - gt[name].reshape(-1))) / max(np.max(np.abs(fd)), 1e-30)
        assert err < 1e-6, (name, err)


# ---------------------------------------------------------------------------
# output epilogue: RMS normalisation over the value channels, output gate
# ---------------------------------------------------------------------------

def test_output_epilogue_closed_forms():
    r = _rng(40)
    o = r.standard_normal((3, 5, 2, 16))
    ones = np.ones_like(o)
    # eps = 0, unit weight and gate: every row has mean square exactly 1
    y = oracle.output_fwd(o, ones, None, eps=0.0)
    assert np.allclose(np.mean(y * y, axis=-1), 1.0, rtol=0, atol=1e-14)
    # scale invariance of the normalisation (positive scale, eps = 0), sign flip is odd
    assert np.allclose(oracle.output_fwd(7.5 * o, ones, None, 0.0), y, rtol=0, atol=1e-14)
    assert np.allclose(oracle.output_fwd(-o, ones, None, 0.0), -y, rtol=0, atol=1e-14)
    # a constant row c * 1: y = c / sqrt(c^2 + eps) on every channel
    c = np.full((1, 1, 1, 8), 0.01)
    y = oracle.output_fwd(c, np.ones_like(c), None, eps=1e-4)
    assert np.allclose(y, 0.01 / np.sqrt(1e-4 + 1e-4), rtol=1e-14, atol=0)
    # weight and gate act per channel after the normalisation (a zero gate channel is zero)
    wt = r.uniform(0.5, 1.5, 16)
    g = r.uniform(0, 1, o.shape)
    g[..., 3] = 0.0
    y2 = oracle.output_fwd(o, g, wt, eps=0.0)
    assert np.allclose(y2, oracle.output_fwd(o, ones, None, 0.0) * wt * g, rtol=1e-14, atol=1e-14)
    assert np.all(y2[..., 3] == 0.0)
    # the gate is not normalised: scaling it scales y
    assert np.allclose(oracle.output_fwd(o, 3 * g, wt, 1e-6), 3 * oracle.output_fwd(o, g, wt, 1e-6), rtol=1e-14)


def test_output_epilogue_gradients_match_central_differences():
    r = _rng(41)
    o = r.standard_normal((2, 3, 2, 8))
    g = r.uniform(0, 1, o.shape)
    wt = r.uniform(0.5, 1.5, 8)
    dy = r.standard_normal(o.shape)
    eps = 1e-3
    gr = oracle.output_bwd(o, g, wt, eps, dy)

    def loss(o_, g_, w_):
        return float(np.sum(oracle.output_fwd(o_, g_, w_, eps) * dy))

    xs = [o, g, wt]
    for pos, name in enumerate(("do", "dg", "dweight")):
        x = xs[pos]
        fd = np.empty(x.size)
        for n, ix in enumerate(np.ndindex(x.shape)):
            h = 1e-6
            xp = [t.copy() for t in xs]
            xm = [t.copy() for t in xs]
            xp[pos][ix] += h
            xm[pos][ix] -= h
            fd[n] = (loss(*xp) - loss(*xm)) / (2 * h)
        err = np.max(np.abs(fd - gr[name].reshape(-1))) / np.max(np.abs(fd))
        assert err < 1e-7, (name, err)
    # weight None means ones
    g0 = oracle.output_bwd(o, g, None, eps, dy)
    g1 = oracle.output_bwd(o, g, np.ones(8), eps, dy)
    assert all(np.array_equal(g0[n], g1[n]) for n in ("do", "dg", "dweight"))

