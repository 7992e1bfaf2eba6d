"""Pins of the CPU oracle to what the pages and mathematics fix (CPU only).

Each test checks the oracle against something other than itself: hand-worked examples,
closed forms (linear attention, the non-causal one-step solution, the delta-rule
contraction), invariants (perfect write, orthonormal keys, zero tokens, state carry),
central finite differences and torch.autograd.
"""
import json
import os

import numpy as np
import pytest

from oracle import ttt_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")
TOL = 1e-12


def _rng(seed=0):
    return np.random.default_rng(seed)


def _rand_chains(rng, N, T, d, unit=False):
    q = rng.standard_normal((N, T, d))
    k = rng.standard_normal((N, T, d))
    v = rng.standard_normal((N, T, d))
    if unit:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    return q, k, v


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _A(x):
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------- hand-worked examples

def test_golden_delta_rule_by_hand():
    g = _golden()["delta_rule_d2"]
    for fn in ("delta", "linear_b1"):
        if fn == "delta":
            z, w = O.delta_rule(_A(g["q"]), _A(g["k"]), _A(g["v"]), _A(g["w0"]), g["eta"])
        else:
            z, w = O.ttt_linear(_A(g["q"]), _A(g["k"]), _A(g["v"]), _A(g["w0"]), g["eta"], 1)
        np.testing.assert_allclose(z, _A(g["z"]), atol=TOL, rtol=0)
        np.testing.assert_allclose(w, _A(g["w_final"]), atol=TOL, rtol=0)


def test_golden_minibatch_by_hand():
    g = _golden()["minibatch_scalar"]
    args = (_A(g["q"]), _A(g["k"]), _A(g["v"]), _A(g["w0"]), g["eta"])
    z, w = O.ttt_linear(*args, 1)
    np.testing.assert_allclose(z, _A(g["z_b1"]), atol=TOL)
    np.testing.assert_allclose(w, _A(g["w_final_b1"]), atol=TOL)
    z, w = O.ttt_linear(*args, 2)
    np.testing.assert_allclose(z, _A(g["z_b2"]), atol=TOL)
    np.testing.assert_allclose(w, _A(g["w_final_b2"]), atol=TOL)
    z, w = O.ttt_linear(*args, 2, causal=False)
    np.testing.assert_allclose(z, _A(g["z_b2_noncausal"]), atol=TOL)


def test_golden_mlp_by_hand():
    g = _golden()["mlp_scalar"]
    z, w1, w2 = O.ttt_mlp(_A(g["q"]), _A(g["k"]), _A(g["v"]), _A(g["w1"]), _A(g["w2"]),
                          g["eta"], 1)
    np.testing.assert_allclose(z, _A(g["z"]), atol=TOL)
    np.testing.assert_allclose(w1, _A(g["w1_final"]), atol=TOL)
    np.testing.assert_allclose(w2, _A(g["w2_final"]), atol=TOL)


def test_golden_dot_loss_by_hand():
    g = _golden()["dot_loss_linear_attention_scalar"]
    for b in (1, 2):
        z, _ = O.ttt_linear(_A(g["q"]), _A(g["k"]), _A(g["v"]), _A(g["w0"]), g["eta"], b,
                            loss="dot")
        np.testing.assert_allclose(z, _A(g["z"]), atol=TOL)


# ---------------------------------------------------------------- closed forms

def _linear_attention_causal(q, k, v, eta):
    # eta * tril(Q K^T) V, diagonal included (each output sees its own key/value).
    s = np.einsum("ntd,nsd->nts", q, k)
    s = np.tril(s)
    return eta * np.einsum("nts,nsd->ntd", s, v)


@pytest.mark.parametrize("chunk", [1, 3, 16, 37])
def test_dot_loss_equals_linear_attention_for_every_chunk(chunk):
    """Negative dot-product loss, W0 = 0: the gradient -v k^T does not depend on W, so
    every mini-batch size gives the linear-attention cumulative sum."""
    rng = _rng(1)
    q, k, v = _rand_chains(rng, 3, 37, 5)
    w0 = np.zeros((3, 5, 5))
    z, w = O.ttt_linear(q, k, v, w0, 0.3, chunk, loss="dot")
    np.testing.assert_allclose(z, _linear_attention_causal(q, k, v, 0.3), atol=1e-12)
    np.testing.assert_allclose(w, 0.3 * np.einsum("ntd,nte->nde", v, k), atol=1e-12)


def test_theorem1_batch_gd_mse_from_zero_is_linear_attention():
    """Linear inner model, batch GD (one chunk of all T tokens), W0 = 0, reconstruction
    loss: the gradient at W0 = 0 is -v k^T, so the causal outputs are linear attention."""
    rng = _rng(2)
    q, k, v = _rand_chains(rng, 2, 24, 6)
    z, _ = O.ttt_linear(q, k, v, np.zeros((2, 6, 6)), 0.7, 24)
    np.testing.assert_allclose(z, _linear_attention_causal(q, k, v, 0.7), atol=1e-12)
    # non-causal: every query reads the full sum
    z, _ = O.ttt_linear(q, k, v, np.zeros((2, 6, 6)), 0.7, 24, causal=False)
    full = 0.7 * np.einsum("ntd,nsd,nse->nte", q, k, v)
    np.testing.assert_allclose(z, full, atol=1e-12)


def test_noncausal_one_step_closed_form():
    """One full-batch step: W' = W0 - eta (W0 K^T - V^T) K, Z = Q W'^T."""
    rng = _rng(3)
    q, k, v = _rand_chains(rng, 2, 11, 4)
    w0 = 0.3 * rng.standard_normal((2, 4, 4))
    eta = 0.05
    z, w = O.ttt_linear(q, k, v, w0, eta, 11, causal=False)
    Kt = np.swapaxes(k, 1, 2)
    Wp = w0 - eta * (w0 @ Kt - np.swapaxes(v, 1, 2)) @ k
    np.testing.assert_allclose(w, Wp, atol=1e-12)
    np.testing.assert_allclose(z, q @ np.swapaxes(Wp, 1, 2), atol=1e-12)


def test_noncausal_mlp_chunk_T_is_one_full_batch_step():
    """Non-causal MLP with one chunk: W' = W - eta * sum of per-token gradients at W."""
    rng = _rng(4)
    q, k, v = _rand_chains(rng, 2, 9, 3)
    w1 = 0.5 * rng.standard_normal((2, 5, 3))
    w2 = 0.5 * rng.standard_normal((2, 3, 5))
    eta = 0.2
    z, a1, a2 = O.ttt_mlp(q, k, v, w1, w2, eta, 9, causal=False)
    # matrix form of the summed gradient (independent of the per-token loop)
    U = np.einsum("nhd,ntd->nth", w1, k)
    A = U / (1 + np.exp(-U))
    sg = 1 / (1 + np.exp(-U))
    R = np.einsum("ndh,nth->ntd", w2, A) - v
    dU = np.einsum("ntd,ndh->nth", R, w2) * sg * (1 + U * (1 - sg))
    W1p = w1 - eta * np.einsum("nth,ntd->nhd", dU, k)
    W2p = w2 - eta * np.einsum("ntd,nth->ndh", R, A)
    np.testing.assert_allclose(a1, W1p, atol=1e-12)
    np.testing.assert_allclose(a2, W2p, atol=1e-12)
    Aq = np.einsum("nhd,ntd->nth", W1p, q)
    Aq = Aq / (1 + np.exp(-Aq))
    np.testing.assert_allclose(z, np.einsum("ndh,nth->ntd", W2p, Aq), atol=1e-12)


# ---------------------------------------------------------------- finite differences

def _fd_check(loss_fn, params, idx, grad, eps=1e-5):
    """Central difference of loss_fn with respect to params[idx], compared to grad."""
    P = [p.copy() for p in params]
    num = np.zeros_like(P[idx])
    it = np.nditer(P[idx], flags=["multi_index"])
    for _ in it:
        m = it.multi_index
        old = P[idx][m]
        P[idx][m] = old + eps
        fp = loss_fn(*P)
        P[idx][m] = old - eps
        fm = loss_fn(*P)
        P[idx][m] = old
        num[m] = (fp - fm).sum() / (2 * eps)
    scale = max(np.abs(grad).max(), 1e-3)
    assert np.abs(num - grad).max() / scale < 1e-7, (num, grad)


@pytest.mark.parametrize("loss", ["mse", "dot"])
def test_linear_gradient_finite_differences(loss):
    rng = _rng(5)
    W = rng.standard_normal((1, 3, 4))
    k = rng.standard_normal((1, 4))
    v = rng.standard_normal((1, 3))
    g = O.linear_grad(W, k, v, loss)
    _fd_check(lambda W_: O.linear_loss(W_, k, v, loss), [W], 0, g)


@pytest.mark.parametrize("loss", ["mse", "dot"])
def test_mlp_gradient_finite_differences(loss):
    rng = _rng(6)
    W1 = rng.standard_normal((1, 7, 4))
    W2 = rng.standard_normal((1, 4, 7))
    k = rng.standard_normal((1, 4))
    v = rng.standard_normal((1, 4))
    g1, g2 = O.mlp_grad(W1, W2, k, v, loss)
    _fd_check(lambda a, b: O.mlp_loss(a, b, k, v, loss), [W1, W2], 0, g1)
    _fd_check(lambda a, b: O.mlp_loss(a, b, k, v, loss), [W1, W2], 1, g2)


def test_silu_derivative_finite_differences():
    u = np.linspace(-6, 6, 49)
    eps = 1e-6
    num = (O.silu(u + eps) - O.silu(u - eps)) / (2 * eps)
    np.testing.assert_allclose(O.dsilu(u), num, atol=1e-8)
    np.testing.assert_allclose(O.silu(u), u / (1 + np.exp(-u)), atol=1e-15)


# ---------------------------------------------------------------- layer norm, residual, GELU
# The paper's inner models (wmrh.cn summary, section 2.2.1): f(x) = x + LN(f_res(x)), f_res
# linear or a 2-layer MLP with GELU; gamma, beta fixed during the inner loop.

def _ln_args(rng, N, d, eps=1e-5):
    return (1.0 + 0.3 * rng.standard_normal((N, d)), 0.2 * rng.standard_normal((N, d)), eps)


def test_gelu_textbook_values():
    # GELU(u) = u Phi(u); Phi(1), Phi(2) from the standard normal table
    u = np.array([-1.0, 0.0, 1.0, 2.0])
    want = np.array([-0.15865525393145707, 0.0, 0.8413447460685429, 2 * 0.9772498680518208])
    np.testing.assert_allclose(O.gelu(u), want, atol=1e-15)
    np.testing.assert_allclose(O.gelu(np.array([30.0, -30.0])), [30.0, 0.0], atol=1e-12)


def test_gelu_derivative_finite_differences():
    u = np.linspace(-6, 6, 49)
    h = 1e-6
    num = (O.gelu(u + h) - O.gelu(u - h)) / (2 * h)
    np.testing.assert_allclose(O.dgelu(u), num, atol=1e-8)


def test_layer_norm_standardises_and_ignores_shift_and_scale():
    rng = _rng(50)
    y = 3.0 + 2.0 * rng.standard_normal((5, 8))
    one, zero = np.ones((5, 8)), np.zeros((5, 8))
    x = O.layer_norm(y, one, zero, 1e-12)
    np.testing.assert_allclose(x.mean(axis=-1), 0.0, atol=1e-12)
    np.testing.assert_allclose((x ** 2).mean(axis=-1), 1.0, atol=1e-9)   # biased variance
    np.testing.assert_allclose(O.layer_norm(7.0 * y - 4.0, one, zero, 1e-12), x, atol=1e-9)
    g, b = _ln_args(rng, 5, 8)[:2]
    np.testing.assert_allclose(O.layer_norm(y, g, b, 1e-12), g * x + b, atol=1e-12)


def test_layer_norm_vjp_finite_differences():
    rng = _rng(51)
    y = rng.standard_normal((1, 6))
    g, b, eps = _ln_args(rng, 1, 6, eps=0.3)    # a large eps so that it matters
    up = rng.standard_normal((1, 6))
    grad = O.layer_norm_vjp(y, g, eps, up)
    _fd_check(lambda y_: (up * O.layer_norm(y_, g, b, eps)).sum(axis=-1), [y], 0, grad)


@pytest.mark.parametrize("loss", ["mse", "dot"])
def test_linear_ln_gradient_finite_differences(loss):
    rng = _rng(52)
    W = rng.standard_normal((1, 5, 5))
    k, v = rng.standard_normal((1, 5)), rng.standard_normal((1, 5))
    ln = _ln_args(rng, 1, 5, eps=0.05)
    g = O.linear_grad(W, k, v, loss, ln)
    _fd_check(lambda W_: O.linear_loss(W_, k, v, loss, ln), [W], 0, g)


@pytest.mark.parametrize("loss,act,with_ln", [("mse", "gelu", True), ("dot", "gelu", True),
                                              ("mse", "silu", True), ("mse", "gelu", False)])
def test_mlp_ln_gelu_gradient_finite_differences(loss, act, with_ln):
    rng = _rng(53)
    W1 = rng.standard_normal((1, 7, 4))
    W2 = rng.standard_normal((1, 4, 7))
    k, v = rng.standard_normal((1, 4)), rng.standard_normal((1, 4))
    ln = _ln_args(rng, 1, 4, eps=0.05) if with_ln else None
    g1, g2 = O.mlp_grad(W1, W2, k, v, loss, act, ln)
    fn = lambda a, b: O.mlp_loss(a, b, k, v, loss, act, ln)
    _fd_check(fn, [W1, W2], 0, g1)
    _fd_check(fn, [W1, W2], 1, g2)


def test_ln_with_zero_gain_never_learns():
    # gamma = 0 makes LN(.) the constant beta: f(x) = x + beta, every gradient is zero, the
    # state never moves and z_t = q_t + beta
    rng = _rng(54)
    q, k, v = (x[0] for x in _rand_chains(rng, 1, 9, 4))
    w0 = rng.standard_normal((4, 4))
    beta = rng.standard_normal(4)
    z, w = O.ttt_linear(q, k, v, w0, 0.5, 3, ln=(np.zeros(4), beta, 1e-5))
    np.testing.assert_allclose(w, w0, atol=0)
    np.testing.assert_allclose(z, q + beta, atol=1e-15)
    w1, w2 = rng.standard_normal((6, 4)), rng.standard_normal((4, 6))
    z, a1, a2 = O.ttt_mlp(q, k, v, w1, w2, 0.5, 4, act="gelu", ln=(np.zeros(4), beta, 1e-5))
    np.testing.assert_allclose(a1, w1, atol=0)
    np.testing.assert_allclose(a2, w2, atol=0)
    np.testing.assert_allclose(z, q + beta, atol=1e-15)


@pytest.mark.parametrize("model,chunk,causal", [("linear", 1, True), ("linear", 4, True),
                                                ("linear", 5, False), ("mlp", 1, True),
                                                ("mlp", 4, True), ("mlp", 13, False)])
def test_ln_models_match_autograd(model, chunk, causal):
    """Recurrence with f(x) = x + LN(f_res(x)) against torch.autograd through torch's own
    layer_norm and (exact) gelu."""
    import torch
    F = torch.nn.functional
    rng = _rng(55)
    d = 4
    q, k, v = (x[0] for x in _rand_chains(rng, 1, 13, d))
    gam, bet, eps = 1.0 + 0.3 * rng.standard_normal(d), 0.2 * rng.standard_normal(d), 1e-3
    G, Bt = torch.tensor(gam), torch.tensor(bet)
    if model == "linear":
        params = [0.5 * rng.standard_normal((d, d))]
        f = lambda P, x: x + F.layer_norm(P[0] @ x, (d,), G, Bt, eps)
        z, *w = O.ttt_linear(q, k, v, params[0], 0.2, chunk, causal=causal, ln=(gam, bet, eps))
    else:
        params = [0.5 * rng.standard_normal((6, d)), 0.5 * rng.standard_normal((d, 6))]
        f = lambda P, x: x + F.layer_norm(P[1] @ F.gelu(P[0] @ x), (d,), G, Bt, eps)
        z, *w = O.ttt_mlp(q, k, v, params[0], params[1], 0.2, chunk, causal=causal, act="gelu",
                          ln=(gam, bet, eps))
    zr, wr = _autograd_chunked(q, k, v, params, f, 0.2, chunk, causal)
    np.testing.assert_allclose(z, zr, atol=1e-11)
    for a, b in zip(w, wr):
        np.testing.assert_allclose(a, b, atol=1e-11)


# ---------------------------------------------------------------- delta-rule invariants

def test_linear_chunk1_equals_delta_rule():
    """Mini-batch size 1 of the generic recurrence equals the delta rule written in its
    closed form (prediction-error update)."""
    rng = _rng(7)
    q, k, v = _rand_chains(rng, 3, 40, 6)
    w0 = 0.2 * rng.standard_normal((3, 6, 6))
    z1, w1 = O.ttt_linear(q, k, v, w0, 0.05, 1)
    z2, w2 = O.delta_rule(q, k, v, w0, 0.05)
    np.testing.assert_allclose(z1, z2, atol=1e-12)
    np.testing.assert_allclose(w1, w2, atol=1e-12)


def test_perfect_write():
    """Unit keys, eta = 1, one token per step: after writing (k_t, v_t) the state maps k_t
    exactly to v_t, so querying with q_t = k_t returns v_t."""
    rng = _rng(8)
    q, k, v = _rand_chains(rng, 2, 30, 8, unit=True)
    w0 = rng.standard_normal((2, 8, 8))
    for fn in ("delta", "linear"):
        if fn == "delta":
            z, _ = O.delta_rule(k, k, v, w0, 1.0)
        else:
            z, _ = O.ttt_linear(k, k, v, w0, 1.0, 1)
        np.testing.assert_allclose(z, v, atol=1e-10)


@pytest.mark.parametrize("eta", [0.3, 1.0, 1.7])
def test_repeated_write_contracts_geometrically(eta):
    """Writing one unit key n times: W_n k - v = (1 - eta)^n (W_0 k - v)."""
    rng = _rng(9)
    d, n = 5, 12
    kk = rng.standard_normal(d)
    kk /= np.linalg.norm(kk)
    vv = rng.standard_normal(d)
    w0 = rng.standard_normal((d, d))
    k = np.tile(kk, (n, 1))
    v = np.tile(vv, (n, 1))
    q = rng.standard_normal((n, d))
    for fn in ("delta", "linear"):
        if fn == "delta":
            _, w = O.delta_rule(q, k, v, w0, eta)
        else:
            _, w = O.ttt_linear(q, k, v, w0, eta, 1)
        np.testing.assert_allclose(w @ kk - vv, (1 - eta) ** n * (w0 @ kk - vv), atol=1e-10)


def test_predictable_pairs_do_not_write():
    """If every value is already predicted by the state (v = W0 k), no gradient is taken
    and the state stays W0 for every chunk size."""
    rng = _rng(10)
    q, k, _ = _rand_chains(rng, 2, 20, 5)
    w0 = rng.standard_normal((2, 5, 5))
    v = np.einsum("nij,ntj->nti", w0, k)
    for b in (1, 4, 20):
        z, w = O.ttt_linear(q, k, v, w0, 0.4, b)
        np.testing.assert_allclose(w, w0, atol=1e-12)
        np.testing.assert_allclose(z, np.einsum("nij,ntj->nti", w0, q), atol=1e-12)


def test_orthonormal_keys_make_every_chunk_size_exact():
    """With orthonormal keys the gradient of token t at the chunk-start weights equals its
    gradient at W_{t-1}, so every mini-batch size reproduces the b = 1 result."""
    rng = _rng(11)
    d, T = 8, 8
    perm = rng.permutation(d)
    basis, _ = np.linalg.qr(rng.standard_normal((d, d)))
    k = basis[:, perm].T[None]               # rows are orthonormal keys
    q = rng.standard_normal((1, T, d))
    v = rng.standard_normal((1, T, d))
    w0 = rng.standard_normal((1, d, d))
    ref, wref = O.ttt_linear(q, k, v, w0, 0.6, 1)
    for b in (2, 3, 5, 8):
        z, w = O.ttt_linear(q, k, v, w0, 0.6, b)
        np.testing.assert_allclose(z, ref, atol=1e-12)
        np.testing.assert_allclose(w, wref, atol=1e-12)


def test_chunking_matters_for_correlated_keys():
    """Guard against an oracle that silently ignores the chunk size."""
    rng = _rng(12)
    q, k, v = _rand_chains(rng, 1, 16, 4)
    w0 = np.zeros((1, 4, 4))
    z1, _ = O.ttt_linear(q, k, v, w0, 0.2, 1)
    z4, _ = O.ttt_linear(q, k, v, w0, 0.2, 4)
    assert np.abs(z1 - z4).max() > 1e-3


# ---------------------------------------------------------------- state carry / padding

@pytest.mark.parametrize("model", ["linear", "mlp"])
def test_state_carry_at_chunk_boundary(model):
    """Running T tokens in one call equals two calls split at a multiple of the chunk
    size, the second starting from the first call's final state."""
    rng = _rng(13)
    q, k, v = _rand_chains(rng, 2, 40, 4, unit=True)
    if model == "linear":
        w0 = 0.1 * rng.standard_normal((2, 4, 4))
        z, w = O.ttt_linear(q, k, v, w0, 0.3, 8)
        za, wa = O.ttt_linear(q[:, :24], k[:, :24], v[:, :24], w0, 0.3, 8)
        zb, wb = O.ttt_linear(q[:, 24:], k[:, 24:], v[:, 24:], wa, 0.3, 8)
        np.testing.assert_allclose(w, wb, atol=1e-12)
    else:
        w1 = 0.3 * rng.standard_normal((2, 6, 4))
        w2 = 0.3 * rng.standard_normal((2, 4, 6))
        z, a1, a2 = O.ttt_mlp(q, k, v, w1, w2, 0.3, 8)
        za, b1, b2 = O.ttt_mlp(q[:, :24], k[:, :24], v[:, :24], w1, w2, 0.3, 8)
        zb, c1, c2 = O.ttt_mlp(q[:, 24:], k[:, 24:], v[:, 24:], b1, b2, 0.3, 8)
        np.testing.assert_allclose(a1, c1, atol=1e-12)
        np.testing.assert_allclose(a2, c2, atol=1e-12)
    np.testing.assert_allclose(z, np.concatenate([za, zb], axis=1), atol=1e-12)


def test_zero_tokens_change_nothing():
    """Tokens with k = v = 0 have zero gradient (no bias, SiLU(0) = 0), so appending them
    to a full-batch chunk leaves the trained weights and the other outputs unchanged."""
    rng = _rng(14)
    q, k, v = _rand_chains(rng, 2, 10, 4)
    w1 = 0.4 * rng.standard_normal((2, 6, 4))
    w2 = 0.4 * rng.standard_normal((2, 4, 6))
    z, a1, a2 = O.ttt_mlp(q, k, v, w1, w2, 0.5, 10, causal=False)
    pad = np.zeros((2, 3, 4))
    qp = np.concatenate([q, rng.standard_normal((2, 3, 4))], axis=1)
    zp, b1, b2 = O.ttt_mlp(qp, np.concatenate([k, pad], 1), np.concatenate([v, pad], 1),
                           w1, w2, 0.5, 13, causal=False)
    np.testing.assert_allclose(b1, a1, atol=1e-12)
    np.testing.assert_allclose(b2, a2, atol=1e-12)
    np.testing.assert_allclose(zp[:, :10], z, atol=1e-12)
    # same for the linear model
    w0 = rng.standard_normal((2, 4, 4))
    z, w = O.ttt_linear(q, k, v, w0, 0.1, 10, causal=False)
    zp, wp = O.ttt_linear(qp, np.concatenate([k, pad], 1), np.concatenate([v, pad], 1),
                          w0, 0.1, 13, causal=False)
    np.testing.assert_allclose(wp, w, atol=1e-12)
    np.testing.assert_allclose(zp[:, :10], z, atol=1e-12)


def test_state_broadcast_over_batch():
    """A [H, d, d] initial state is shared by every batch element."""
    rng = _rng(15)
    q, k, v = [rng.standard_normal((3, 2, 10, 4)) for _ in range(3)]
    w0 = rng.standard_normal((2, 4, 4))
    z, w = O.ttt_linear(q, k, v, w0, 0.1, 4)
    for b in range(3):
        zb, wb = O.ttt_linear(q[b], k[b], v[b], w0, 0.1, 4)
        np.testing.assert_allclose(z[b], zb, atol=1e-13)
        np.testing.assert_allclose(w[b], wb, atol=1e-13)


# ---------------------------------------------------------------- torch.autograd

def _autograd_chunked(q, k, v, params, f, eta, chunk, causal, epochs=1):
    """Mini-batch GD computed with torch.autograd for the gradients (float64, CPU).  eta is
    a scalar, or one rate per token (each token's gradient scaled by its own rate); the
    non-causal layer may pass over the chunks several times (epochs)."""
    import torch
    T = q.shape[0]
    P = [torch.tensor(p, dtype=torch.float64) for p in params]
    Q, K, V = (torch.tensor(x, dtype=torch.float64) for x in (q, k, v))
    Z = torch.zeros_like(Q)
    per_token = np.ndim(eta) > 0
    starts = []
    for _ in range(epochs):
        starts += list(range(0, T, chunk))
    for c0 in starts:
        Pc = [p.clone().requires_grad_(True) for p in P]
        acc = [torch.zeros_like(p) for p in P]
        cur = P
        for t in range(c0, min(c0 + chunk, T)):
            loss = 0.5 * ((f(Pc, K[t]) - V[t]) ** 2).sum()
            grads = torch.autograd.grad(loss, Pc)
            if per_token:
                acc = [a + float(eta[t]) * g for a, g in zip(acc, grads)]
                cur = [pc.detach() - a for pc, a in zip(Pc, acc)]
            else:
                acc = [a + g for a, g in zip(acc, grads)]
                cur = [pc.detach() - eta * a for pc, a in zip(Pc, acc)]
            if causal:
                with torch.no_grad():
                    Z[t] = f(cur, Q[t])
        P = cur
    if not causal:
        with torch.no_grad():
            for t in range(T):
                Z[t] = f(P, Q[t])
    return Z.numpy(), [p.detach().numpy() for p in P]


def _torch_mlp(P, x):
    import torch
    return P[1] @ torch.nn.functional.silu(P[0] @ x)


def _torch_linear(P, x):
    return P[0] @ x


@pytest.mark.parametrize("chunk,causal", [(1, True), (4, True), (7, True), (13, False),
                                          (5, False)])
def test_mlp_matches_autograd(chunk, causal):
    rng = _rng(16)
    q, k, v = _rand_chains(rng, 1, 13, 3)
    w1 = 0.5 * rng.standard_normal((6, 3))
    w2 = 0.5 * rng.standard_normal((3, 6))
    z, a1, a2 = O.ttt_mlp(q[0], k[0], v[0], w1, w2, 0.15, chunk, causal=causal)
    zr, (r1, r2) = _autograd_chunked(q[0], k[0], v[0], [w1, w2], _torch_mlp, 0.15, chunk,
                                     causal)
    np.testing.assert_allclose(z, zr, atol=1e-12)
    np.testing.assert_allclose(a1, r1, atol=1e-12)
    np.testing.assert_allclose(a2, r2, atol=1e-12)


@pytest.mark.parametrize("chunk,causal", [(1, True), (4, True), (6, False)])
def test_linear_matches_autograd(chunk, causal):
    rng = _rng(17)
    q, k, v = _rand_chains(rng, 1, 14, 4)
    w0 = 0.3 * rng.standard_normal((4, 4))
    z, w = O.ttt_linear(q[0], k[0], v[0], w0, 0.1, chunk, causal=causal)
    zr, (wr,) = _autograd_chunked(q[0], k[0], v[0], [w0], _torch_linear, 0.1, chunk, causal)
    np.testing.assert_allclose(z, zr, atol=1e-12)
    np.testing.assert_allclose(w, wr, atol=1e-12)


# ---------------------------------------------------------------- epochs (non-causal)
# ViT3 news page, observation 2 and its figure on inner batch size and epochs: the N pairs
# are split into consecutive mini-batches and the inner model is trained for several
# epochs before every query reads the final weights.

@pytest.mark.parametrize("epochs,rates", [(1, False), (2, False), (5, False), (3, True)])
def test_noncausal_full_batch_epochs_closed_form(epochs, rates):
    # Full-batch GD on sum_t r_t/2 ||W k_t - v_t||^2 is the affine map
    # W -> W (I - eta K^T D K) + eta V^T D K (D = diag(r)), whose fixed point is
    # W* = V^T D K (K^T D K)^{-1}; after E steps W_E = W* + (W0 - W*) (I - eta K^T D K)^E.
    rng = _rng(40)
    T, d = 11, 4
    q, k, v = (x[0] for x in _rand_chains(rng, 1, T, d))
    w0 = 0.3 * rng.standard_normal((d, d))
    eta = 0.05
    r = rng.uniform(0.2, 1.0, T) if rates else np.ones(T)
    z, w = O.ttt_linear(q, k, v, w0, eta, T, causal=False, epochs=epochs,
                        eta_tok=r if rates else None)
    KDK = k.T @ (r[:, None] * k)
    Wstar = v.T @ (r[:, None] * k) @ np.linalg.inv(KDK)
    WE = Wstar + (w0 - Wstar) @ np.linalg.matrix_power(np.eye(d) - eta * KDK, epochs)
    np.testing.assert_allclose(w, WE, atol=1e-10)
    np.testing.assert_allclose(z, q @ WE.T, atol=1e-10)


@pytest.mark.parametrize("chunk,epochs", [(3, 2), (7, 4), (20, 3)])
def test_noncausal_dot_loss_epochs_add_up(chunk, epochs):
    # The dot loss's gradient -v k^T does not depend on W, so every chunking and epoch
    # count give W0 + E eta V^T K.
    rng = _rng(41)
    T, d = 20, 5
    q, k, v = (x[0] for x in _rand_chains(rng, 1, T, d))
    w0 = rng.standard_normal((d, d))
    z, w = O.ttt_linear(q, k, v, w0, 0.07, chunk, causal=False, loss="dot", epochs=epochs)
    WE = w0 + epochs * 0.07 * v.T @ k
    np.testing.assert_allclose(w, WE, atol=1e-12)
    np.testing.assert_allclose(z, q @ WE.T, atol=1e-12)


@pytest.mark.parametrize("model,chunk,epochs", [("linear", 6, 2), ("linear", 14, 3),
                                                ("mlp", 5, 3), ("mlp", 13, 2)])
def test_epochs_match_autograd(model, chunk, epochs):
    rng = _rng(42)
    q, k, v = (x[0] for x in _rand_chains(rng, 1, 13, 3))
    if model == "linear":
        params, f = [0.3 * rng.standard_normal((3, 3))], _torch_linear
        z, *w = O.ttt_linear(q, k, v, params[0], 0.1, chunk, causal=False, epochs=epochs)
    else:
        params = [0.5 * rng.standard_normal((6, 3)), 0.5 * rng.standard_normal((3, 6))]
        f = _torch_mlp
        z, *w = O.ttt_mlp(q, k, v, params[0], params[1], 0.1, chunk, causal=False,
                          epochs=epochs)
    zr, wr = _autograd_chunked(q, k, v, params, f, 0.1, chunk, False, epochs=epochs)
    np.testing.assert_allclose(z, zr, atol=1e-12)
    for a, b in zip(w, wr):
        np.testing.assert_allclose(a, b, atol=1e-12)


def test_causal_layer_rejects_epochs():
    q = k = v = np.zeros((4, 2))
    with pytest.raises(ValueError):
        O.ttt_linear(q, k, v, np.zeros((2, 2)), 0.1, 2, causal=True, epochs=2)
    with pytest.raises(ValueError):
        O.ttt_mlp(q, k, v, np.zeros((3, 2)), np.zeros((2, 3)), 0.1, 2, causal=True, epochs=2)


# ---------------------------------------------------------------- per-token rates
# The "Fast weights" page writes the step with a rate per step, eta_t; the wmrh.cn summary,
# section 2.2.3, makes the rate a function of the token.  In a mini-batch each token's
# gradient is scaled by its own rate: W_t = W_{t'} - sum_{s<=t} eta_s grad l_s(W_{t'}).

@pytest.mark.parametrize("chunk,causal", [(1, True), (4, True), (5, False)])
def test_linear_token_rates_match_autograd(chunk, causal):
    rng = _rng(30)
    q, k, v = _rand_chains(rng, 1, 13, 4)
    w0 = 0.3 * rng.standard_normal((4, 4))
    r = rng.uniform(0.2, 1.0, 13)
    z, w = O.ttt_linear(q[0], k[0], v[0], w0, 0.4, chunk, causal=causal, eta_tok=r)
    zr, (wr,) = _autograd_chunked(q[0], k[0], v[0], [w0], _torch_linear, 0.4 * r, chunk, causal)
    np.testing.assert_allclose(z, zr, atol=1e-12)
    np.testing.assert_allclose(w, wr, atol=1e-12)


@pytest.mark.parametrize("chunk,causal", [(1, True), (4, True), (13, False)])
def test_mlp_token_rates_match_autograd(chunk, causal):
    rng = _rng(31)
    q, k, v = _rand_chains(rng, 1, 13, 3)
    w1 = 0.5 * rng.standard_normal((6, 3))
    w2 = 0.5 * rng.standard_normal((3, 6))
    r = rng.uniform(0.2, 1.0, 13)
    z, a1, a2 = O.ttt_mlp(q[0], k[0], v[0], w1, w2, 0.15, chunk, causal=causal, eta_tok=r)
    zr, (r1, r2) = _autograd_chunked(q[0], k[0], v[0], [w1, w2], _torch_mlp, 0.15 * r, chunk,
                                     causal)
    np.testing.assert_allclose(z, zr, atol=1e-12)
    np.testing.assert_allclose(a1, r1, atol=1e-12)
    np.testing.assert_allclose(a2, r2, atol=1e-12)


@pytest.mark.parametrize("model,chunk", [("linear", 1), ("linear", 4), ("mlp", 4), ("delta", 1)])
def test_zero_rate_token_equals_zero_key(model, chunk):
    """A token whose rate is 0 writes nothing; so does a token whose key is 0 (the gradient
    of W k and of W2 SiLU(W1 k) vanishes at k = 0).  Both runs must agree, which pins
    that token t's own gradient carries rate t."""
    rng = _rng(32)
    q, k, v = _rand_chains(rng, 2, 12, 4)
    r = rng.uniform(0.3, 1.0, (2, 12))
    mask = np.zeros((2, 12), dtype=bool)
    mask[0, [1, 4, 5, 11]] = True
    mask[1, [0, 7]] = True
    r0 = np.where(mask, 0.0, r)
    k0 = np.where(mask[..., None], 0.0, k)
    if model == "linear":
        w0 = 0.3 * rng.standard_normal((2, 4, 4))
        a = O.ttt_linear(q, k, v, w0, 0.5, chunk, eta_tok=r0)
        b = O.ttt_linear(q, k0, v, w0, 0.5, chunk, eta_tok=r)
    elif model == "delta":
        w0 = 0.3 * rng.standard_normal((2, 4, 4))
        a = O.delta_rule(q, k, v, w0, 0.5, eta_tok=r0)
        b = O.delta_rule(q, k0, v, w0, 0.5, eta_tok=r)
    else:
        w1 = 0.4 * rng.standard_normal((2, 6, 4))
        w2 = 0.4 * rng.standard_normal((2, 4, 6))
        a = O.ttt_mlp(q, k, v, w1, w2, 0.5, chunk, eta_tok=r0)
        b = O.ttt_mlp(q, k0, v, w1, w2, 0.5, chunk, eta_tok=r)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, atol=1e-12)


def test_linear_token_rates_dual_form():
    """Matrix form of one chunk with rates e (derived separately, not a loop over tokens):
    R = K W^T - V, Z = Q W^T - tril(Q K^T) diag(e) R, W <- W - (diag(e) R)^T K."""
    rng = _rng(33)
    T, d, b, eta = 21, 4, 8, 0.7
    q, k, v = _rand_chains(rng, 1, T, d)
    w0 = 0.3 * rng.standard_normal((d, d))
    r = rng.uniform(0.1, 1.0, T)
    z, w = O.ttt_linear(q, k, v, w0[None], eta, b, eta_tok=r[None])
    W = w0.copy()
    Z = np.zeros((T, d))
    for c0 in range(0, T, b):
        Q, K, V = q[0, c0:c0 + b], k[0, c0:c0 + b], v[0, c0:c0 + b]
        e = eta * r[c0:c0 + b]
        R = K @ W.T - V
        Z[c0:c0 + b] = Q @ W.T - np.tril(Q @ K.T) @ (e[:, None] * R)
        W = W - (e[:, None] * R).T @ K
    np.testing.assert_allclose(z[0], Z, atol=1e-12)
    np.testing.assert_allclose(w[0], W, atol=1e-12)


def test_linear_chunk1_equals_delta_rule_with_token_rates():
    rng = _rng(34)
    q, k, v = _rand_chains(rng, 3, 17, 5, unit=True)
    w0 = 0.2 * rng.standard_normal((3, 5, 5))
    r = rng.uniform(0.0, 1.0, (3, 17))
    za, wa = O.ttt_linear(q, k, v, w0, 0.9, 1, eta_tok=r)
    zb, wb = O.delta_rule(q, k, v, w0, 0.9, eta_tok=r)
    np.testing.assert_allclose(za, zb, atol=1e-12)
    np.testing.assert_allclose(wa, wb, atol=1e-12)


def test_constant_token_rates_equal_scalar_rate():
    rng = _rng(35)
    q, k, v = _rand_chains(rng, 2, 11, 4)
    w1 = 0.4 * rng.standard_normal((2, 6, 4))
    w2 = 0.4 * rng.standard_normal((2, 4, 6))
    a = O.ttt_mlp(q, k, v, w1, w2, 0.3, 4, eta_tok=np.full((2, 11), 0.5))
    b = O.ttt_mlp(q, k, v, w1, w2, 0.15, 4)
    for x, y in zip(a, b):
        np.testing.assert_allclose(x, y, atol=1e-12)


# ---------------------------------------------------------------- layer gradients
# The vjp is pinned to central finite differences of the numpy forward (which shares no code
# with the torch recurrence the vjp differentiates).

def _fd_vjp(q, k, v, w0, eta, chunk, dz, dw, which, direction, h=1e-6):
    args = dict(q=q, k=k, v=v, w0=w0)

    def L(x):
        a = dict(args)
        a[which] = x
        z, w = O.ttt_linear(a["q"], a["k"], a["v"], a["w0"], eta, chunk)
        return float(np.sum(z * dz) + (np.sum(w * dw) if dw is not None else 0.0))
    x = args[which]
    return (L(x + h * direction) - L(x - h * direction)) / (2 * h)


@pytest.mark.parametrize("chunk,with_dw", [(1, False), (4, True), (3, True), (10, False)])
def test_linear_vjp_matches_finite_differences(chunk, with_dw):
    rng = _rng(40 + chunk)
    N, T, d = 2, 10, 4
    q, k, v = _rand_chains(rng, N, T, d)
    w0 = 0.3 * rng.standard_normal((N, d, d))
    dz = rng.standard_normal((N, T, d))
    dw = rng.standard_normal((N, d, d)) if with_dw else None
    grads = dict(zip(("q", "k", "v", "w0"), O.ttt_linear_vjp(q, k, v, w0, 0.2, chunk, dz, dw)))
    for which, x in (("q", q), ("k", k), ("v", v), ("w0", w0)):
        for _ in range(2):
            direction = rng.standard_normal(x.shape)
            fd = _fd_vjp(q, k, v, w0, 0.2, chunk, dz, dw, which, direction)
            an = float(np.sum(grads[which] * direction))
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (which, fd, an)


@pytest.mark.parametrize("chunk,with_dw", [(1, True), (4, False), (3, True)])
def test_linear_vjp_token_rates_match_finite_differences(chunk, with_dw):
    """Per-token rate factors: every gradient, the factors' own included, against central
    differences of the numpy forward with the same factors."""
    rng = _rng(50 + chunk)
    N, T, d = 2, 9, 4
    q, k, v = _rand_chains(rng, N, T, d)
    w0 = 0.3 * rng.standard_normal((N, d, d))
    et = rng.uniform(0.2, 1.5, (N, T))
    dz = rng.standard_normal((N, T, d))
    dw = rng.standard_normal((N, d, d)) if with_dw else None
    args = dict(q=q, k=k, v=v, w0=w0, et=et)

    def L(a):
        z, w = O.ttt_linear(a["q"], a["k"], a["v"], a["w0"], 0.2, chunk, eta_tok=a["et"])
        return float(np.sum(z * dz) + (np.sum(w * dw) if dw is not None else 0.0))
    grads = dict(zip(("q", "k", "v", "w0", "et"), O.ttt_linear_vjp(q, k, v, w0, 0.2, chunk, dz, dw, eta_tok=et)))
    h = 1e-6
    for which in ("q", "k", "v", "w0", "et"):
        direction = rng.standard_normal(args[which].shape)
        ap, am = dict(args), dict(args)
        ap[which] = args[which] + h * direction
        am[which] = args[which] - h * direction
        fd = (L(ap) - L(am)) / (2 * h)
        an = float(np.sum(grads[which] * direction))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (which, fd, an)


@pytest.mark.parametrize("chunk,with_dw", [(1, True), (4, False), (5, True)])
def test_linear_vjp_dot_loss_matches_finite_differences(chunk, with_dw):
    """The negative dot-product loss: every gradient against central differences of the numpy
    forward with loss="dot"."""
    rng = _rng(70 + chunk)
    N, T, d = 2, 9, 4
    q, k, v = _rand_chains(rng, N, T, d)
    w0 = 0.3 * rng.standard_normal((N, d, d))
    dz = rng.standard_normal((N, T, d))
    dw = rng.standard_normal((N, d, d)) if with_dw else None
    args = dict(q=q, k=k, v=v, w0=w0)

    def L(a):
        z, w = O.ttt_linear(a["q"], a["k"], a["v"], a["w0"], 0.2, chunk, loss="dot")
        return float(np.sum(z * dz) + (np.sum(w * dw) if dw is not None else 0.0))
    grads = dict(zip(("q", "k", "v", "w0"), O.ttt_linear_vjp(q, k, v, w0, 0.2, chunk, dz, dw, loss="dot")))
    h = 1e-6
    for which in ("q", "k", "v", "w0"):
        direction = rng.standard_normal(args[which].shape)
        ap, am = dict(args), dict(args)
        ap[which] = args[which] + h * direction
        am[which] = args[which] - h * direction
        fd = (L(ap) - L(am)) / (2 * h)
        an = float(np.sum(grads[which] * direction))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (which, fd, an)


def test_linear_vjp_dot_loss_closed_form():
    """Dot loss, one chunk: W_t = W0 + eta sum_{s<=t} v_s k_s^T doesn't depend on W0 beyond the
    additive term, so dw0 = sum_t dz_t q_t^T (+ dw_out) and dq_t = W_t^T dz_t."""
    rng = _rng(75)
    q, k, v = _rand_chains(rng, 1, 6, 3)
    w0 = rng.standard_normal((1, 3, 3))
    dz = rng.standard_normal((1, 6, 3))
    dw = rng.standard_normal((1, 3, 3))
    dq, dk, dv, dw0 = O.ttt_linear_vjp(q, k, v, w0, 0.3, 6, dz, dw, loss="dot")
    np.testing.assert_allclose(dw0[0], dz[0].T @ q[0] + dw[0], atol=1e-12)
    for t in range(6):
        wt = w0[0] + 0.3 * sum(np.outer(v[0, s], k[0, s]) for s in range(t + 1))
        np.testing.assert_allclose(dq[0, t], wt.T @ dz[0, t], atol=1e-12)


def test_linear_vjp_unit_token_rates_match_no_rates():
    rng = _rng(55)
    q, k, v = _rand_chains(rng, 1, 11, 3)
    w0 = rng.standard_normal((1, 3, 3))
    dz = rng.standard_normal((1, 11, 3))
    base = O.ttt_linear_vjp(q, k, v, w0, 0.3, 4, dz)
    with_rates = O.ttt_linear_vjp(q, k, v, w0, 0.3, 4, dz, eta_tok=np.ones((1, 11)))
    for a, b in zip(base, with_rates[:4]):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def test_linear_vjp_zero_rate_is_the_fixed_map():
    """eta = 0: z = W0 q, so dq = dz W0, dw0 = sum_t dz_t q_t^T (+ dw_out), dk = dv = 0."""
    rng = _rng(45)
    q, k, v = _rand_chains(rng, 1, 7, 3)
    w0 = rng.standard_normal((1, 3, 3))
    dz = rng.standard_normal((1, 7, 3))
    dw = rng.standard_normal((1, 3, 3))
    dq, dk, dv, dw0 = O.ttt_linear_vjp(q, k, v, w0, 0.0, 4, dz, dw)
    np.testing.assert_allclose(dq[0], dz[0] @ w0[0], atol=1e-13)
    np.testing.assert_allclose(dw0[0], dz[0].T @ q[0] + dw[0], atol=1e-13)
    np.testing.assert_array_equal(dk, 0.0)
    np.testing.assert_array_equal(dv, 0.0)


def _fd_mlp_vjp(args, eta, chunk, dz, dw1, dw2, which, direction, h=1e-6, loss="mse"):
    def L(x):
        a = dict(args)
        a[which] = x
        z, w1, w2 = O.ttt_mlp(a["q"], a["k"], a["v"], a["w1"], a["w2"], eta, chunk, loss=loss)
        out = float(np.sum(z * dz))
        if dw1 is not None:
            out += float(np.sum(w1 * dw1) + np.sum(w2 * dw2))
        return out
    x = args[which]
    return (L(x + h * direction) - L(x - h * direction)) / (2 * h)


@pytest.mark.parametrize("chunk,with_dw", [(1, False), (4, True), (3, True), (9, False)])
def test_mlp_vjp_matches_finite_differences(chunk, with_dw):
    rng = _rng(60 + chunk)
    N, T, d, hdim = 2, 9, 3, 5
    q, k, v = _rand_chains(rng, N, T, d)
    args = dict(q=q, k=k, v=v, w1=0.5 * rng.standard_normal((N, hdim, d)),
                w2=0.5 * rng.standard_normal((N, d, hdim)))
    dz = rng.standard_normal((N, T, d))
    dw1 = rng.standard_normal((N, hdim, d)) if with_dw else None
    dw2 = rng.standard_normal((N, d, hdim)) if with_dw else None
    grads = dict(zip(("q", "k", "v", "w1", "w2"),
                     O.ttt_mlp_vjp(q, k, v, args["w1"], args["w2"], 0.2, chunk, dz, dw1, dw2)))
    for which in ("q", "k", "v", "w1", "w2"):
        for _ in range(2):
            direction = rng.standard_normal(args[which].shape)
            fd = _fd_mlp_vjp(args, 0.2, chunk, dz, dw1, dw2, which, direction)
            an = float(np.sum(grads[which] * direction))
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (which, fd, an)


@pytest.mark.parametrize("chunk,with_dw", [(1, False), (4, True), (9, True)])
def test_mlp_vjp_dot_loss_matches_finite_differences(chunk, with_dw):
    """Negative dot-product loss (ViT3 news page, section 2): the VJP against central
    differences of the forward recurrence with loss="dot", for every input."""
    rng = _rng(70 + chunk)
    N, T, d, hdim = 2, 9, 3, 5
    q, k, v = _rand_chains(rng, N, T, d)
    args = dict(q=q, k=k, v=v, w1=0.5 * rng.standard_normal((N, hdim, d)),
                w2=0.5 * rng.standard_normal((N, d, hdim)))
    dz = rng.standard_normal((N, T, d))
    dw1 = rng.standard_normal((N, hdim, d)) if with_dw else None
    dw2 = rng.standard_normal((N, d, hdim)) if with_dw else None
    grads = dict(zip(("q", "k", "v", "w1", "w2"),
                     O.ttt_mlp_vjp(q, k, v, args["w1"], args["w2"], 0.2, chunk, dz, dw1, dw2, loss="dot")))
    for which in ("q", "k", "v", "w1", "w2"):
        for _ in range(2):
            direction = rng.standard_normal(args[which].shape)
            fd = _fd_mlp_vjp(args, 0.2, chunk, dz, dw1, dw2, which, direction, loss="dot")
            an = float(np.sum(grads[which] * direction))
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (which, fd, an)


def test_mlp_vjp_dot_loss_differs_from_reconstruction():
    """The two losses give different gradients (the dot loss is not silently ignored)."""
    rng = _rng(75)
    q, k, v = _rand_chains(rng, 1, 6, 3)
    w1, w2 = rng.standard_normal((1, 4, 3)), rng.standard_normal((1, 3, 4))
    dz = rng.standard_normal((1, 6, 3))
    a = O.ttt_mlp_vjp(q, k, v, w1, w2, 0.3, 3, dz)
    b = O.ttt_mlp_vjp(q, k, v, w1, w2, 0.3, 3, dz, loss="dot")
    assert np.abs(a[1] - b[1]).max() > 1e-3


def test_mlp_vjp_zero_rate_is_the_fixed_map():
    """eta = 0: z_t = W2 SiLU(W1 q_t) with u = W1 q_t, so dw2 = sum dz_t SiLU(u_t)^T,
    dq_t = W1^T ((W2^T dz_t) * SiLU'(u_t)), dw1 = sum ((W2^T dz_t) * SiLU'(u_t)) q_t^T, and
    dk = dv = 0."""
    rng = _rng(65)
    q, k, v = _rand_chains(rng, 1, 6, 3)
    w1, w2 = rng.standard_normal((1, 4, 3)), rng.standard_normal((1, 3, 4))
    dz = rng.standard_normal((1, 6, 3))
    dq, dk, dv, dw1, dw2 = O.ttt_mlp_vjp(q, k, v, w1, w2, 0.0, 4, dz)
    u = q[0] @ w1[0].T
    gu = (dz[0] @ w2[0]) * (1 / (1 + np.exp(-u))) * (1 + u * (1 - 1 / (1 + np.exp(-u))))
    np.testing.assert_allclose(dw2[0], dz[0].T @ (u / (1 + np.exp(-u))), atol=1e-12)
    np.testing.assert_allclose(dq[0], gu @ w1[0], atol=1e-12)
    np.testing.assert_allclose(dw1[0], gu.T @ q[0], atol=1e-12)
    np.testing.assert_array_equal(dk, 0.0)
    np.testing.assert_array_equal(dv, 0.0)


# ---------------------------------------------------------------- edge cases

def test_empty_sequence():
    q = np.zeros((2, 0, 4))
    w0 = np.ones((2, 4, 4))
    z, w = O.ttt_linear(q, q, q, w0, 0.1, 16)
    assert z.shape == (2, 0, 4)
    np.testing.assert_array_equal(w, w0)


def test_chunk_longer_than_sequence_is_one_chunk():
    rng = _rng(18)
    q, k, v = _rand_chains(rng, 1, 5, 3)
    w0 = rng.standard_normal((1, 3, 3))
    a = O.ttt_linear(q, k, v, w0, 0.1, 5)
    b = O.ttt_linear(q, k, v, w0, 0.1, 64)
    np.testing.assert_allclose(a[0], b[0], atol=1e-14)


def test_ragged_last_chunk():
    """T = 10 with chunk 4: the chunks are 4, 4, 2 tokens, i.e. the same as running the
    first 8 tokens and then 2 tokens with chunk 2 from the carried state."""
    rng = _rng(19)
    q, k, v = _rand_chains(rng, 1, 10, 3)
    w0 = rng.standard_normal((1, 3, 3))
    z, w = O.ttt_linear(q, k, v, w0, 0.1, 4)
    za, wa = O.ttt_linear(q[:, :8], k[:, :8], v[:, :8], w0, 0.1, 4)
    zb, wb = O.ttt_linear(q[:, 8:], k[:, 8:], v[:, 8:], wa, 0.1, 2)
    np.testing.assert_allclose(z, np.concatenate([za, zb], 1), atol=1e-13)
    np.testing.assert_allclose(w, wb, atol=1e-13)


# ---------------------------------------------------------------- gradients of every variant
# ttt_layer_vjp (each token's inner gradient by autograd, the trajectory by autograd) against
# central finite differences of the numpy forward, for the variants the written-out VJPs do
# not cover: the non-causal layer with mini-batches and epochs, the MLP with per-token rates,
# the paper's layer norm + residual models (GELU MLP), and the gradients of the rates and of
# the layer-norm gain and bias.  On the options both cover it must equal the written-out VJPs.

_LAYER_CASES = [
    # kind, causal, chunk, epochs, rates, loss, act, ln
    ("linear", False, 3, 2, False, "mse", "silu", False),
    ("linear", False, 10, 1, True, "dot", "silu", False),
    ("linear", True, 4, 1, False, "mse", "silu", True),
    ("linear", False, 4, 2, True, "mse", "silu", True),
    ("mlp", True, 3, 1, True, "mse", "silu", False),
    ("mlp", False, 4, 2, True, "mse", "silu", False),
    ("mlp", False, 10, 1, False, "mse", "silu", False),
    ("mlp", True, 3, 1, False, "mse", "gelu", True),
    ("mlp", False, 5, 2, True, "dot", "gelu", True),
]


def _layer_forward(kind, a, eta, chunk, causal, epochs, loss, act, ln_eps):
    ln = (a["gamma"], a["beta"], ln_eps) if "gamma" in a else None
    et = a.get("et")
    if kind == "linear":
        return O.ttt_linear(a["q"], a["k"], a["v"], a["w0"], eta, chunk, causal, loss=loss,
                            eta_tok=et, epochs=epochs, ln=ln)
    return O.ttt_mlp(a["q"], a["k"], a["v"], a["w1"], a["w2"], eta, chunk, causal, loss=loss,
                     eta_tok=et, epochs=epochs, act=act, ln=ln)


@pytest.mark.parametrize("kind,causal,chunk,epochs,rates,loss,act,ln", _LAYER_CASES)
def test_layer_vjp_matches_finite_differences(kind, causal, chunk, epochs, rates, loss, act, ln):
    rng = _rng(hash((kind, causal, chunk, epochs, rates, loss, act, ln)) % 1000)
    N, T, d, h = 2, 10, 4, 5
    q, k, v = _rand_chains(rng, N, T, d)
    a = dict(q=q, k=k, v=v)
    if kind == "linear":
        a["w0"] = 0.3 * rng.standard_normal((N, d, d))
        names = ("w0",)
    else:
        a["w1"] = 0.3 * rng.standard_normal((N, h, d))
        a["w2"] = 0.3 * rng.standard_normal((N, d, h))
        names = ("w1", "w2")
    if rates:
        a["et"] = rng.uniform(0.2, 1.5, (N, T))
    eps = 0.05  # large enough that the layer norm's own curvature matters
    if ln:
        a["gamma"] = 1.0 + 0.3 * rng.standard_normal((N, d))
        a["beta"] = 0.3 * rng.standard_normal((N, d))
    eta = 0.15
    dz = rng.standard_normal((N, T, d))
    dst = tuple(rng.standard_normal(a[n].shape) for n in names)
    out = O.ttt_layer_vjp(kind, q, k, v, tuple(a[n] for n in names), eta, chunk, dz, dst,
                          causal=causal, epochs=epochs, eta_tok=a.get("et"), loss=loss, act=act,
                          ln=(a["gamma"], a["beta"], eps) if ln else None)
    grads = dict(zip(("q", "k", "v") + names + ("et", "gamma", "beta"), out))

    def L(x):
        z, *ws = _layer_forward(kind, x, eta, chunk, causal, epochs, loss, act, eps)
        return float(np.sum(z * dz) + sum(np.sum(w * g) for w, g in zip(ws, dst)))
    for which in [w for w in ("q", "k", "v") + names + ("et", "gamma", "beta") if w in a]:
        assert grads[which] is not None, which
        direction = rng.standard_normal(a[which].shape)
        hh = 1e-6
        ap, am = dict(a), dict(a)
        ap[which] = a[which] + hh * direction
        am[which] = a[which] - hh * direction
        fd = (L(ap) - L(am)) / (2 * hh)
        an = float(np.sum(grads[which] * direction))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (which, fd, an)
    if not rates:
        assert grads["et"] is None
    if not ln:
        assert grads["gamma"] is None and grads["beta"] is None


def test_layer_vjp_equals_the_written_out_vjps():
    rng = _rng(91)
    N, T, d, h = 2, 9, 4, 5
    q, k, v = _rand_chains(rng, N, T, d)
    w0 = 0.3 * rng.standard_normal((N, d, d))
    w1 = 0.3 * rng.standard_normal((N, h, d))
    w2 = 0.3 * rng.standard_normal((N, d, h))
    dz = rng.standard_normal((N, T, d))
    dw0 = rng.standard_normal((N, d, d))
    dw1 = rng.standard_normal((N, h, d))
    dw2 = rng.standard_normal((N, d, h))
    et = rng.uniform(0.2, 1.5, (N, T))
    a = O.ttt_linear_vjp(q, k, v, w0, 0.2, 4, dz, dw0, eta_tok=et)
    b = O.ttt_layer_vjp("linear", q, k, v, (w0,), 0.2, 4, dz, (dw0,), eta_tok=et)
    for x, y in zip(a, b[:5]):
        np.testing.assert_allclose(x, y, rtol=0, atol=1e-12)
    for loss in ("mse", "dot"):
        a = O.ttt_mlp_vjp(q, k, v, w1, w2, 0.2, 3, dz, dw1, dw2, loss=loss)
        b = O.ttt_layer_vjp("mlp", q, k, v, (w1, w2), 0.2, 3, dz, (dw1, dw2), loss=loss)
        for x, y in zip(a, b[:5]):
            np.testing.assert_allclose(x, y, rtol=0, atol=1e-12)


def test_noncausal_full_batch_linear_vjp_closed_form():
    """One full-batch step (chunk = T, causal = 0): W' = W0 - eta (W0 K^T - V^T) K and
    Z = Q W'^T, so dQ = dZ W', dW' = dZ^T Q, dV = eta K dW'^T, and
    dW0 = dW' (I - eta K^T K) and, per key, dk_t = -eta (W0^T dW' k_t + dW'^T r_t) with
    r_t = W0 k_t - v_t."""
    rng = _rng(92)
    N, T, d = 2, 7, 3
    q, k, v = _rand_chains(rng, N, T, d)
    w0 = 0.3 * rng.standard_normal((N, d, d))
    dz = rng.standard_normal((N, T, d))
    eta = 0.1
    dq, dk, dv, dw0, *_ = O.ttt_layer_vjp("linear", q, k, v, (w0,), eta, T, dz, None, causal=False)
    R = np.einsum("ntj,nij->nti", k, w0) - v
    W1 = w0 - eta * np.einsum("nti,ntj->nij", R, k)
    D = np.einsum("nti,ntj->nij", dz, q)       # dW'
    np.testing.assert_allclose(dq, np.einsum("nti,nij->ntj", dz, W1), atol=1e-12)
    np.testing.assert_allclose(dv, eta * np.einsum("ntj,nij->nti", k, D), atol=1e-12)
    I = np.eye(d)[None]
    np.testing.assert_allclose(dw0, np.einsum("nij,njk->nik", D, I - eta * np.einsum("ntj,ntk->njk", k, k)),
                               atol=1e-12)
    dk_ref = -eta * (np.einsum("nij,nim,ntm->ntj", w0, D, k) + np.einsum("nti,nij->ntj", R, D))
    np.testing.assert_allclose(dk, dk_ref, atol=1e-12)
