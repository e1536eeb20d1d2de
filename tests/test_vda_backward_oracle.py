"""Pins of the VDA-branch gradient oracle (oracle.vda_backward).

The gradient is pinned to the forward oracle (itself pinned in
test_oracle_pins.py) by central finite differences of <d_o, o_l> for every
input, and to invariants of the forward computation that hold exactly:
  * o_l is linear in the RMSNorm weight, so <drms_w, rms_w> = <d_o, o_l>;
  * with eps = 0 each direction's RMSNorm output is invariant to scaling one
    query, so <dq_n, q_n> = 0 per token; scaling every value of a (batch,
    head) scales every state, so sum <dv, v> = 0 per (batch, head);
  * a frame with beta_t = 0 writes nothing, so its dk and dv vanish;
  * reversing the frame order swaps the two scan directions, so the gradient
    of the reversed inputs is the reversed gradient.
A dropped term, a wrong sign, index or transposed operand in any adjoint step
fails the finite-difference test of the input it feeds.
"""
import numpy as np
import pytest

from oracle import vdn_oracle as O
from oracle.vda_backward import vda_branch_backward


def _inputs(seed, B=1, H=2, T=5, N=3, d=4):
    g = np.random.default_rng(seed)
    q = g.normal(0, 1, (B, H, T, N, d))
    k = g.normal(0, 1, (B, H, T, N, d))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = g.normal(0, 1, (B, H, T, N, d))
    gamma = g.uniform(0.3, 0.95, (B, H, T))
    beta = g.uniform(0.2, 1.5, (B, H, T))
    rms_w = g.uniform(0.5, 1.5, H * d)
    d_o = g.normal(0, 1, (B, H, T, N, d))
    return dict(q=q, k=k, v=v, gamma=gamma, beta=beta, rms_w=rms_w), d_o


def _loss(x, d_o, eps):
    o, _, _ = O.vda_branch(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["rms_w"], eps)
    return float(np.sum(d_o * o))


def _grads(x, d_o, eps):
    return vda_branch_backward(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["rms_w"], eps, d_o)


GRAD_OF = {"q": "dq", "k": "dk", "v": "dv", "gamma": "dgamma", "beta": "dbeta", "rms_w": "drms_w"}


@pytest.mark.parametrize("name", list(GRAD_OF))
def test_directional_finite_differences(name):
    eps = 1e-3
    x, d_o = _inputs(11)
    gr = _grads(x, d_o, eps)[GRAD_OF[name]]
    rng = np.random.default_rng(12)
    h = 1e-6
    for _ in range(3):
        delta = rng.normal(0, 1, x[name].shape)
        xp = dict(x, **{name: x[name] + h * delta})
        xm = dict(x, **{name: x[name] - h * delta})
        fd = (_loss(xp, d_o, eps) - _loss(xm, d_o, eps)) / (2 * h)
        an = float(np.sum(gr * delta))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (name, fd, an)


@pytest.mark.parametrize("name", ["k", "v", "gamma", "beta"])
def test_elementwise_finite_differences_first_and_last_frame(name):
    # single entries in the first, a middle and the last frame: the two scan
    # directions start at opposite ends, so an off-by-one in either shows here
    eps = 1e-6
    x, d_o = _inputs(13, B=2, H=1, T=4, N=2, d=4)
    gr = _grads(x, d_o, eps)[GRAD_OF[name]]
    h = 1e-6
    for t in (0, 2, 3):
        idx = (1, 0, t) + (0,) * (x[name].ndim - 3)
        xp = {kk: vv.copy() for kk, vv in x.items()}
        xm = {kk: vv.copy() for kk, vv in x.items()}
        xp[name][idx] += h
        xm[name][idx] -= h
        fd = (_loss(xp, d_o, eps) - _loss(xm, d_o, eps)) / (2 * h)
        assert abs(fd - gr[idx]) <= 1e-6 * max(1.0, abs(fd)), (name, t, fd, gr[idx])


def test_rms_weight_euler_identity():
    x, d_o = _inputs(14)
    o, _, _ = O.vda_branch(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["rms_w"], 1e-6)
    gr = _grads(x, d_o, 1e-6)
    assert np.isclose(np.dot(gr["drms_w"], x["rms_w"]), np.sum(d_o * o), rtol=1e-12, atol=1e-12)


def test_scale_invariances_at_zero_eps():
    x, d_o = _inputs(15, B=1, H=2, T=6, N=4, d=8)
    gr = _grads(x, d_o, 0.0)
    per_token = np.sum(gr["dq"] * x["q"], axis=-1)
    assert np.max(np.abs(per_token)) < 1e-10 * np.max(np.abs(gr["dq"]))
    per_head = np.sum(gr["dv"] * x["v"], axis=(2, 3, 4))
    assert np.max(np.abs(per_head)) < 1e-10 * np.max(np.abs(gr["dv"]))


def test_zero_beta_frame_has_no_key_value_gradient():
    x, d_o = _inputs(16)
    x["beta"][0, 1, 2] = 0.0
    gr = _grads(x, d_o, 1e-6)
    assert np.all(gr["dk"][0, 1, 2] == 0.0) and np.all(gr["dv"][0, 1, 2] == 0.0)
    assert np.any(gr["dk"][0, 1, 1] != 0.0)
    # the write strength itself still has a gradient at zero (the forward map
    # is smooth through beta = 0, so a central difference applies)
    h = 1e-6
    xp = {kk: vv.copy() for kk, vv in x.items()}
    xm = {kk: vv.copy() for kk, vv in x.items()}
    xp["beta"][0, 1, 2] = h
    xm["beta"][0, 1, 2] = -h
    fd = (_loss(xp, d_o, 1e-6) - _loss(xm, d_o, 1e-6)) / (2 * h)
    assert abs(fd - gr["dbeta"][0, 1, 2]) <= 1e-6 * max(1.0, abs(fd))


def test_frame_reversal_swaps_the_directions():
    x, d_o = _inputs(17, T=6)
    flip = lambda a: np.flip(a, axis=2).copy()
    xr = {kk: (flip(vv) if kk != "rms_w" else vv) for kk, vv in x.items()}
    g0 = _grads(x, d_o, 1e-6)
    g1 = _grads(xr, flip(d_o), 1e-6)
    for name in ("dq", "dk", "dv", "dgamma", "dbeta"):
        np.testing.assert_allclose(g1[name], flip(g0[name]), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g1["drms_w"], g0["drms_w"], rtol=1e-10, atol=1e-12)


def test_all_zero_beta_closed_form():
    """beta = 0 in every frame: every state is zero, so dq, dk, dv and dgamma
    vanish exactly.  dbeta_t has a closed form.  Frame t's write
    Btil_t = V_t^T K_t reaches frame s of the forward scan (s >= t) scaled by
    gamma_{t+1} ... gamma_s, and frame s <= t of the backward scan scaled by
    gamma_s ... gamma_{t-1}.  The readout at zero state is linear,
    r = u / sqrt(eps).  So
        dbeta_t = sum over both scans and reached frames s of
                  (gamma product) * sum_n <w * do_{s,n}, Btil_t q_{s,n}> / sqrt(eps),
    a direct sum, not the adjoint recursion."""
    eps = 1e-4
    x, d_o = _inputs(18, B=1, H=1, T=5, N=3, d=4)
    x["beta"][:] = 0.0
    gr = _grads(x, d_o, eps)
    for name in ("dq", "dk", "dv", "dgamma"):
        assert np.all(gr[name] == 0.0), name
    q, k, v, gam, w = x["q"][0, 0], x["k"][0, 0], x["v"][0, 0], x["gamma"][0, 0], x["rms_w"]
    do = d_o[0, 0]
    T = q.shape[0]
    want = np.zeros(T)
    for t in range(T):
        btil = v[t].T @ k[t]
        for s in range(T):
            if s >= t:      # forward scan
                want[t] += np.prod(gam[t + 1:s + 1]) * np.sum((w * do[s]) * (q[s] @ btil.T))
            if s <= t:      # backward scan
                want[t] += np.prod(gam[s:t]) * np.sum((w * do[s]) * (q[s] @ btil.T))
    want /= np.sqrt(eps)
    np.testing.assert_allclose(gr["dbeta"][0, 0], want, rtol=1e-12, atol=1e-12)


def test_dbeta_term_mass_bounds_dbeta_and_scales_with_the_upstream_gradient():
    """dbeta_mass is a sum of absolute values of the products whose signed sum
    is dbeta: it bounds |dbeta| (triangle inequality), is zero when the
    upstream gradient is zero, and is linear in a positive scaling of it."""
    x, d_o = _inputs(21)
    gr = _grads(x, d_o, 1e-6)
    assert np.all(gr["dbeta_mass"] >= np.abs(gr["dbeta"]) * (1 - 1e-12))
    assert np.all(gr["dbeta_mass"] > 0)
    g0 = _grads(x, np.zeros_like(d_o), 1e-6)
    assert np.all(g0["dbeta_mass"] == 0.0) and np.all(g0["dbeta"] == 0.0)
    g3 = _grads(x, 3.0 * d_o, 1e-6)
    np.testing.assert_allclose(g3["dbeta_mass"], 3.0 * gr["dbeta_mass"], rtol=1e-12)
