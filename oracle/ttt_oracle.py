"""CPU oracle for the TTT-layer forward pass: the primal per-token recurrence, in float64.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or execute this
module: only the test-suite, the smoke check and the CPU-baseline leg of the benchmark use
it.  It shares no code, tables or helpers with the HIP library and imports nothing from it.

What it computes (all citations are to the four web pages on test-time training that
define the method; no line numbers are given on purpose):

* Inner model f(k; W).  Linear: f(k; W) = W k with W stored [d_out][d_in]
  (page "5.1 - Fast weights and TTT layers", section 1, which uses the column-vector
  form; the blog page "TTT: Test-Time Training" uses row vectors, k W, which is the same
  model transposed).  MLP: f(k; W1, W2) = W2 SiLU(W1 k), no bias, no layer norm, no
  residual (ViT3 news page, section "2. inner model design", observation 4: a 2-layer
  SiLU MLP whose hidden width is r times the input width).
* Self-supervised loss: reconstruction, l(W; k, v) = 1/2 ||f(k; W) - v||^2 ("Fast weights"
  page, opening formula).  The negative dot-product loss l = -v^T f(k; W) of the blog page
  (section "TTT / 如何理解") is also provided; it is only used by the checks.
* Update rule: online gradient descent W_t = W_{t-1} - eta * grad l_t(W_{t-1})
  (blog page, section "TTT / 通用表示"), generalised to mini-batch GD as in the summary of
  Sun et al. 2024 on the wmrh.cn page, section 1.2.2 ("mini-batch TTT"): inside a
  mini-batch of b consecutive tokens every gradient is taken at the weights W_{t'} left by
  the previous mini-batch (W_0 for the first one), and
      W_t = W_{t'} - eta * sum_{s = t'+1..t} grad l_s(W_{t'})          (cumulative sum).
  b = 1 is plain online GD, b = T is batch GD.
* Per-token learning rates (optional eta_tok): the "Fast weights" page writes the step
  as W_t = W_{t-1} - eta_t grad l_t(W_{t-1}) with a rate per step (opening formula and
  section 1), and the wmrh.cn summary, section 2.2.3 ("learnable eta"), makes it a function
  of the token, eta(x) = eta_base * sigmoid(theta_lr . x).  The rate of token t is
  eta * eta_tok[..., t]; in a mini-batch each token's gradient is scaled by its own rate,
      W_t = W_{t'} - sum_{s = t'+1..t} eta_s grad l_s(W_{t'}).
* Paper instantiation with layer norm and residual (optional `ln`): the wmrh.cn summary of
  Sun et al. 2024, section 2.2.1, always wraps the inner model as
      f(x) = x + LN(f_res(x)),
  f_res the linear map W x or a 2-layer MLP with hidden width 4 d and a GELU activation;
  LN(y) = gamma * (y - mean(y)) / sqrt(var(y) + eps) + beta over the d features (biased
  variance), gamma and beta fixed during the inner loop (outer-loop parameters, one pair per
  head).  GELU is u * Phi(u), Phi the standard normal CDF (the exact form).  The loss is
  unchanged: 1/2 ||f(k) - v||^2 or -v^T f(k).
* Output rule: z_t = f(q_t; W_t), i.e. the output is read after the token's own update
  (blog page "TTT / 通用表示"; "Fast weights" page opening formula).
* Non-causal variant (ViT3 news page, "1. inner training setup", observation 2): the keys
  and values are used as a small data set to train the inner model (here: one pass of
  mini-batch GD over all chunks), and every query then reads the final weights.  The same
  page (observation 2, the figure on inner batch size and epochs) splits the N pairs into
  consecutive mini-batches (several updates per epoch) and trains for several epochs; an
  epoch here is one such pass over every chunk in order, starting from the weights the
  previous epoch left (optional `epochs`, non-causal only).

The recurrence is written out literally: the gradient of each token is materialised, the
per-token weights W_t are materialised, and there is no blocking, fusion or dual form.
It is vectorised only over independent (batch, head) chains.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf

__all__ = [
    "silu",
    "dsilu",
    "gelu",
    "dgelu",
    "layer_norm",
    "layer_norm_vjp",
    "linear_f",
    "mlp_f",
    "linear_loss",
    "mlp_loss",
    "linear_grad",
    "mlp_grad",
    "ttt_linear",
    "ttt_mlp",
    "delta_rule",
    "ttt_linear_vjp",
    "ttt_mlp_vjp",
    "ttt_layer_vjp",
]

LOSSES = ("mse", "dot")


# ----------------------------------------------------------------------------------------
# Inner models, losses and their gradients (per chain, batched over a leading axis N)
# ----------------------------------------------------------------------------------------

def silu(u):
    """SiLU(u) = u * sigma(u), the inner activation of the ViT3 inner MLP."""
    return u / (1.0 + np.exp(-u))


def dsilu(u):
    """d/du SiLU(u) = sigma(u) * (1 + u * (1 - sigma(u)))."""
    s = 1.0 / (1.0 + np.exp(-u))
    return s * (1.0 + u * (1.0 - s))


def gelu(u):
    """GELU(u) = u * Phi(u), Phi(u) = (1 + erf(u / sqrt 2)) / 2 (the paper MLP's activation)."""
    return 0.5 * u * (1.0 + erf(u / np.sqrt(2.0)))


def dgelu(u):
    """d/du GELU(u) = Phi(u) + u * phi(u), phi the standard normal density."""
    return 0.5 * (1.0 + erf(u / np.sqrt(2.0))) + u * np.exp(-0.5 * u * u) / np.sqrt(2.0 * np.pi)


ACTIVATIONS = {"silu": (silu, dsilu), "gelu": (gelu, dgelu)}


def layer_norm(y, gamma, beta, eps):
    """LN over the last axis: gamma * (y - mean) / sqrt(var + eps) + beta, biased variance.
    y [N, d]; gamma, beta [N, d]."""
    mu = y.mean(axis=-1, keepdims=True)
    var = ((y - mu) ** 2).mean(axis=-1, keepdims=True)
    return gamma * (y - mu) / np.sqrt(var + eps) + beta


def layer_norm_vjp(y, gamma, eps, g):
    """dl/dy given dl/dLN(y) = g (chain rule through the mean and the variance):
    with s = sqrt(var + eps), xh = (y - mean) / s and gg = gamma * g,
        dl/dy = (gg - mean(gg) - xh * mean(gg * xh)) / s."""
    mu = y.mean(axis=-1, keepdims=True)
    s = np.sqrt(((y - mu) ** 2).mean(axis=-1, keepdims=True) + eps)
    xh = (y - mu) / s
    gg = gamma * g
    return (gg - gg.mean(axis=-1, keepdims=True) - xh * (gg * xh).mean(axis=-1, keepdims=True)) / s


def _wrap(res, x, ln):
    """The inner model's output from f_res(x): res itself, or x + LN(res) with ln given."""
    return res if ln is None else x + layer_norm(res, ln[0], ln[1], ln[2])


def _unwrap_vjp(res, err, ln):
    """dl/df_res from dl/df = err (identity without ln; through LN otherwise)."""
    return err if ln is None else layer_norm_vjp(res, ln[0], ln[2], err)


def _error(out, v, loss):
    """dl/df: f - v for 1/2 ||f - v||^2, -v for -v^T f."""
    if loss == "mse":
        return out - v
    if loss == "dot":
        return -v
    raise ValueError(loss)


def linear_f(W, x, ln=None):
    """f(x; W) = W x, or x + LN(W x) with ln = (gamma [N, d], beta [N, d], eps).
    W [N, d_out, d_in], x [N, d_in] -> [N, d_out]."""
    return _wrap(np.einsum("nij,nj->ni", W, x), x, ln)


def mlp_f(W1, W2, x, act="silu", ln=None):
    """f(x; W1, W2) = W2 act(W1 x), or x + LN(W2 act(W1 x)) with ln given.
    W1 [N, h, d], W2 [N, d, h], x [N, d] -> [N, d]."""
    fa = ACTIVATIONS[act][0]
    return _wrap(np.einsum("nih,nh->ni", W2, fa(np.einsum("nhj,nj->nh", W1, x))), x, ln)


def linear_loss(W, k, v, loss="mse", ln=None):
    """Per-chain loss value: 1/2||f(k) - v||^2 (mse) or -v^T f(k) (dot).  -> [N]."""
    y = linear_f(W, k, ln)
    if loss == "mse":
        return 0.5 * np.sum((y - v) ** 2, axis=-1)
    return -np.sum(v * y, axis=-1)


def mlp_loss(W1, W2, k, v, loss="mse", act="silu", ln=None):
    """Per-chain loss value of the 2-layer inner MLP.  -> [N]."""
    y = mlp_f(W1, W2, k, act, ln)
    if loss == "mse":
        return 0.5 * np.sum((y - v) ** 2, axis=-1)
    return -np.sum(v * y, axis=-1)


def linear_grad(W, k, v, loss="mse", ln=None):
    """Gradient of the loss with respect to W for f(k; W) = W k (or k + LN(W k)).

    mse: (W k - v) k^T  ("Fast weights" page, section 1, gradient of the linear model).
    dot: -v k^T         (blog page, "TTT / 如何理解", gradient of the negative dot product,
                          written here in the column-vector form).
    With ln the error term f(k) - v (or -v) first passes back through the layer norm.
    W [N, d, d], k, v [N, d] -> [N, d, d].
    """
    y = np.einsum("nij,nj->ni", W, k)
    r = _unwrap_vjp(y, _error(_wrap(y, k, ln), v, loss), ln)
    return np.einsum("ni,nj->nij", r, k)


def mlp_grad(W1, W2, k, v, loss="mse", act="silu", ln=None):
    """Gradients (dW1, dW2) of the loss for f(k) = W2 act(W1 k) (or k + LN of it), by the
    chain rule.

    u = W1 k, a = act(u), y = W2 a, dl/dy = f - v (mse) or -v (dot), passed back through
    the layer norm when ln is given; dW2 = (dl/dy) a^T, dW1 = ((W2^T dl/dy) * act'(u)) k^T.
    """
    fa, dfa = ACTIVATIONS[act]
    u = np.einsum("nhj,nj->nh", W1, k)
    a = fa(u)
    y = np.einsum("nih,nh->ni", W2, a)
    r = _unwrap_vjp(y, _error(_wrap(y, k, ln), v, loss), ln)
    g2 = np.einsum("ni,nh->nih", r, a)
    du = np.einsum("nih,ni->nh", W2, r) * dfa(u)
    g1 = np.einsum("nh,nj->nhj", du, k)
    return g1, g2


# ----------------------------------------------------------------------------------------
# Shape helpers
# ----------------------------------------------------------------------------------------

def _flatten_tokens(x, dtype):
    x = np.asarray(x)
    if x.ndim < 2:
        raise ValueError("token tensors need shape [..., T, d]")
    lead = x.shape[:-2]
    n = int(np.prod(lead)) if lead else 1
    return np.ascontiguousarray(x.reshape((n,) + x.shape[-2:]).astype(dtype)), lead


def _broadcast_state(w, lead, dtype):
    """Broadcast an initial state [..., r, c] against the chains' leading dims."""
    w = np.asarray(w).astype(dtype)
    full = np.broadcast_to(w, tuple(lead) + w.shape[-2:])
    n = int(np.prod(lead)) if lead else 1
    return np.array(full.reshape((n,) + w.shape[-2:]), dtype=dtype, copy=True)


def _token_rates(eta, eta_tok, lead, T, dtype):
    """Per-token rates eta * eta_tok broadcast to the chains, [N, T]; None without eta_tok."""
    if eta_tok is None:
        return None
    r = np.broadcast_to(np.asarray(eta_tok).astype(dtype), tuple(lead) + (T,))
    n = int(np.prod(lead)) if lead else 1
    return dtype(eta) * np.array(r.reshape(n, T), dtype=dtype, copy=True)


def _ln_params(ln, lead, d, dtype):
    """(gamma [N, d], beta [N, d], eps) broadcast against the chains, or None.  gamma and
    beta broadcast like the states (e.g. [H, d], one pair per head)."""
    if ln is None:
        return None
    gamma, beta, eps = ln
    n = int(np.prod(lead)) if lead else 1
    g = np.broadcast_to(np.asarray(gamma).astype(dtype), tuple(lead) + (d,)).reshape(n, d)
    b = np.broadcast_to(np.asarray(beta).astype(dtype), tuple(lead) + (d,)).reshape(n, d)
    if not eps > 0:
        raise ValueError("the layer norm's eps must be positive")
    return np.array(g, copy=True), np.array(b, copy=True), dtype(eps)


def _check_epochs(epochs, causal):
    if not (isinstance(epochs, (int, np.integer)) and epochs >= 1):
        raise ValueError("epochs must be a positive integer")
    # A second pass would let a causal output see tokens after its own position.
    if causal and epochs != 1:
        raise ValueError("several epochs are defined for the non-causal layer only")
    return int(epochs)


def _check_chunk(T, chunk):
    if not (isinstance(chunk, (int, np.integer)) and chunk >= 1):
        raise ValueError("chunk must be a positive integer")
    # A chunk longer than the sequence is one chunk of length T.
    return int(min(chunk, T)) if T > 0 else int(chunk)


# ----------------------------------------------------------------------------------------
# The recurrences
# ----------------------------------------------------------------------------------------

def ttt_linear(q, k, v, w0, eta, chunk, causal=True, loss="mse", dtype=np.float64, eta_tok=None,
               epochs=1, ln=None):
    """TTT layer with the linear inner model, mini-batch GD of size `chunk`.

    q, k, v: [..., T, d]; w0: [..., d, d] (broadcast over the leading dims, e.g. [H, d, d]
    shared by every batch element); eta_tok: optional per-token rate factors [..., T];
    ln: optional (gamma, beta, eps), gamma and beta [..., d] (e.g. [H, d]), for the inner
    model f(x) = x + LN(W x).  Returns (z [..., T, d], w_final [..., d, d]).

    The last chunk is shorter when T is not a multiple of `chunk`.  causal=False trains
    over every chunk first (`epochs` passes) and then applies the final weights to every
    query.
    """
    if loss not in LOSSES:
        raise ValueError(loss)
    q2, lead = _flatten_tokens(q, dtype)
    k2, _ = _flatten_tokens(k, dtype)
    v2, _ = _flatten_tokens(v, dtype)
    N, T, d = q2.shape
    W = _broadcast_state(w0, lead, dtype)
    lnp = _ln_params(ln, lead, d, dtype)
    b = _check_chunk(T, chunk)
    epochs = _check_epochs(epochs, causal)
    et = _token_rates(eta, eta_tok, lead, T, dtype)
    eta = dtype(eta)
    z = np.zeros((N, T, d), dtype=dtype)
    chunk_starts = [c0 for _ in range(epochs) for c0 in range(0, T, b)]
    for c0 in chunk_starts:
        Wc = W.copy()                      # weights left by the previous mini-batch
        G = np.zeros_like(Wc)              # running sum of this mini-batch's gradients
        Wt = Wc
        for t in range(c0, min(c0 + b, T)):
            if et is None:
                G = G + linear_grad(Wc, k2[:, t], v2[:, t], loss, lnp)
                Wt = Wc - eta * G              # W_t, materialised
            else:                              # rate-weighted sum, each token its own rate
                G = G + et[:, t, None, None] * linear_grad(Wc, k2[:, t], v2[:, t], loss, lnp)
                Wt = Wc - G
            if causal:
                z[:, t] = linear_f(Wt, q2[:, t], lnp)
        W = Wt
    if not causal:
        for t in range(T):
            z[:, t] = linear_f(W, q2[:, t], lnp)
    return z.reshape(tuple(lead) + (T, d)), W.reshape(tuple(lead) + (d, d))


def ttt_mlp(q, k, v, w1, w2, eta, chunk, causal=True, loss="mse", dtype=np.float64, eta_tok=None,
            epochs=1, act="silu", ln=None):
    """TTT layer with the 2-layer MLP inner model, mini-batch GD of size `chunk`.

    q, k, v: [..., T, d]; w1: [..., h, d]; w2: [..., d, h] (broadcast over the leading
    dims); eta_tok: optional per-token rate factors [..., T]; epochs: passes over the
    chunks before the queries are read (non-causal only); act: "silu" (ViT3 inner MLP) or
    "gelu" (the paper's TTT-MLP); ln: optional (gamma, beta, eps) for f(x) = x + LN(MLP(x)).
    Returns (z [..., T, d], w1_final [..., h, d], w2_final [..., d, h]).
    """
    if loss not in LOSSES:
        raise ValueError(loss)
    q2, lead = _flatten_tokens(q, dtype)
    k2, _ = _flatten_tokens(k, dtype)
    v2, _ = _flatten_tokens(v, dtype)
    N, T, d = q2.shape
    W1 = _broadcast_state(w1, lead, dtype)
    W2 = _broadcast_state(w2, lead, dtype)
    h = W1.shape[-2]
    if W1.shape[-1] != d or W2.shape[-2:] != (d, h):
        raise ValueError("w1 must be [..., h, d] and w2 [..., d, h]")
    if act not in ACTIVATIONS:
        raise ValueError(act)
    lnp = _ln_params(ln, lead, d, dtype)
    b = _check_chunk(T, chunk)
    epochs = _check_epochs(epochs, causal)
    et = _token_rates(eta, eta_tok, lead, T, dtype)
    eta = dtype(eta)
    z = np.zeros((N, T, d), dtype=dtype)
    chunk_starts = [c0 for _ in range(epochs) for c0 in range(0, T, b)]
    for c0 in chunk_starts:
        W1c, W2c = W1.copy(), W2.copy()
        G1 = np.zeros_like(W1c)
        G2 = np.zeros_like(W2c)
        W1t, W2t = W1c, W2c
        for t in range(c0, min(c0 + b, T)):
            g1, g2 = mlp_grad(W1c, W2c, k2[:, t], v2[:, t], loss, act, lnp)
            if et is None:
                G1 = G1 + g1
                G2 = G2 + g2
                W1t = W1c - eta * G1
                W2t = W2c - eta * G2
            else:                              # rate-weighted sums, each token its own rate
                G1 = G1 + et[:, t, None, None] * g1
                G2 = G2 + et[:, t, None, None] * g2
                W1t = W1c - G1
                W2t = W2c - G2
            if causal:
                z[:, t] = mlp_f(W1t, W2t, q2[:, t], act, lnp)
        W1, W2 = W1t, W2t
    if not causal:
        for t in range(T):
            z[:, t] = mlp_f(W1, W2, q2[:, t], act, lnp)
    return (z.reshape(tuple(lead) + (T, d)), W1.reshape(tuple(lead) + (h, d)),
            W2.reshape(tuple(lead) + (d, h)))


def delta_rule(q, k, v, w0, eta, dtype=np.float64, eta_tok=None):
    """The delta rule, written out as its closed-form update.

    "Fast weights" page, section 1: W_t = W_{t-1} + eta_t (v_t - W_{t-1} k_t) k_t^T, and the
    output z_t = W_t q_t; eta_t = eta, or eta * eta_tok[..., t] with per-token factors.
    Returns (z [..., T, d], w_final [..., d, d]).
    """
    q2, lead = _flatten_tokens(q, dtype)
    k2, _ = _flatten_tokens(k, dtype)
    v2, _ = _flatten_tokens(v, dtype)
    N, T, d = q2.shape
    W = _broadcast_state(w0, lead, dtype)
    et = _token_rates(eta, eta_tok, lead, T, dtype)
    eta = dtype(eta)
    z = np.zeros((N, T, d), dtype=dtype)
    for t in range(T):
        kt = k2[:, t]
        err = v2[:, t] - np.einsum("nij,nj->ni", W, kt)      # prediction error
        if et is None:
            W = W + eta * np.einsum("ni,nj->nij", err, kt)
        else:
            W = W + et[:, t, None, None] * np.einsum("ni,nj->nij", err, kt)
        z[:, t] = np.einsum("nij,nj->ni", W, q2[:, t])
    return z.reshape(tuple(lead) + (T, d)), W.reshape(tuple(lead) + (d, d))


# ----------------------------------------------------------------------------------------
# Gradients of the layer (outer-loop backward pass)
# ----------------------------------------------------------------------------------------

def ttt_linear_vjp(q, k, v, w0, eta, chunk, dz, dw_out=None, eta_tok=None, loss="mse"):
    """Vector-Jacobian product of the causal TTT-Linear layer (reconstruction loss).

    The outer loop trains K, V, Q projections and the initial state by backpropagating
    through the inner updates (wmrh.cn summary, section 2.2: the outer loop; "Fast weights"
    page, opening paragraph: the slow parameters, initialisation and rate are trained on
    the outer objective).  For upstream gradients dz [..., T, d] of z and dw_out [..., d, d]
    of the final state (or None), returns (dq, dk, dv [..., T, d], dw0 [..., d, d]) with
    dw0 per chain (not summed over a shared leading dimension).  With per-token rate factors
    eta_tok [..., T] (token t's gradient taken with rate eta * eta_tok[t], as in ttt_linear;
    wmrh.cn summary, section 2.2.3, the learnable rate) it also returns their gradient
    deta_tok [..., T] (per chain).  loss="dot" takes the negative dot-product loss -v^T W k of
    ttt_linear (ViT3 news page, section 2), whose gradient row is r = -v.

    The definition, written out: the primal recurrence of ttt_linear, in float64 torch
    tensors, differentiated by torch.autograd (reverse mode) -- no hand-derived backward.
    """
    import torch
    q2, lead = _flatten_tokens(q, np.float64)
    k2, _ = _flatten_tokens(k, np.float64)
    v2, _ = _flatten_tokens(v, np.float64)
    N, T, d = q2.shape
    W0 = _broadcast_state(w0, lead, np.float64)
    dz2, _ = _flatten_tokens(dz, np.float64)
    b = _check_chunk(T, chunk)
    Q = torch.tensor(q2, requires_grad=True)
    K = torch.tensor(k2, requires_grad=True)
    V = torch.tensor(v2, requires_grad=True)
    Wi = torch.tensor(W0, requires_grad=True)
    E = None
    if eta_tok is not None:
        E = torch.tensor(np.asarray(eta_tok, dtype=np.float64).reshape(N, T), requires_grad=True)
    W = Wi
    zs = []
    for c0 in range(0, T, b):
        Wc = W
        G = torch.zeros_like(Wc)
        Wt = Wc
        for t in range(c0, min(c0 + b, T)):
            if loss == "dot":
                r = -V[:, t]
            else:
                r = torch.einsum("nij,nj->ni", Wc, K[:, t]) - V[:, t]
            if E is not None:
                r = r * E[:, t, None]  # token t's gradient with its own rate factor
            G = G + torch.einsum("ni,nj->nij", r, K[:, t])
            Wt = Wc - eta * G
            zs.append(torch.einsum("nij,nj->ni", Wt, Q[:, t]))
        W = Wt
    Z = torch.stack(zs, dim=1) if zs else torch.zeros((N, 0, d), dtype=torch.float64)
    outs, grads = [Z], [torch.tensor(dz2)]
    if dw_out is not None:
        outs.append(W)
        grads.append(torch.tensor(_broadcast_state(dw_out, lead, np.float64)))
    wrt = (Q, K, V, Wi) + ((E,) if E is not None else ())
    got = torch.autograd.grad(outs, wrt, grads, allow_unused=True)
    dq, dk, dv, dw0 = got[:4]
    shape = tuple(lead) + (T, d)
    zero = lambda t: np.zeros((N, T, d)) if t is None else t.numpy()
    res = (zero(dq).reshape(shape), zero(dk).reshape(shape), zero(dv).reshape(shape),
           (np.zeros_like(W0) if dw0 is None else dw0.numpy()).reshape(tuple(lead) + (d, d)))
    if E is not None:
        de = got[4]
        res = res + ((np.zeros((N, T)) if de is None else de.numpy()).reshape(tuple(lead) + (T,)),)
    return res


def ttt_mlp_vjp(q, k, v, w1, w2, eta, chunk, dz, dw1_out=None, dw2_out=None, loss="mse"):
    """Vector-Jacobian product of the causal TTT-MLP layer (2-layer SiLU inner MLP,
    reconstruction loss), the MLP counterpart of ttt_linear_vjp.  loss="dot" takes the
    negative dot-product loss -v^T f(k) of ttt_mlp (ViT3 news page, section 2), whose error
    term is r = -v whatever the weights are.

    For upstream gradients dz [..., T, d] of z and dw1_out [..., h, d], dw2_out [..., d, h]
    of the final states (or None), returns (dq, dk, dv [..., T, d], dw1 [..., h, d],
    dw2 [..., d, h]) per chain.

    The definition, written out: the primal recurrence of ttt_mlp (each token's gradient by
    the chain rule, summed at the chunk-start weights, the output read after the update), in
    float64 torch tensors, differentiated by torch.autograd -- so the second-order terms (the
    gradient of the inner gradient) come from autograd, not from a hand derivation.
    """
    import torch
    q2, lead = _flatten_tokens(q, np.float64)
    k2, _ = _flatten_tokens(k, np.float64)
    v2, _ = _flatten_tokens(v, np.float64)
    N, T, d = q2.shape
    W1i = torch.tensor(_broadcast_state(w1, lead, np.float64), requires_grad=True)
    W2i = torch.tensor(_broadcast_state(w2, lead, np.float64), requires_grad=True)
    h = W1i.shape[-2]
    dz2, _ = _flatten_tokens(dz, np.float64)
    b = _check_chunk(T, chunk)
    Q = torch.tensor(q2, requires_grad=True)
    K = torch.tensor(k2, requires_grad=True)
    V = torch.tensor(v2, requires_grad=True)
    silu_t = lambda u: u * torch.sigmoid(u)

    def dsilu_t(u):
        s = torch.sigmoid(u)
        return s * (1.0 + u * (1.0 - s))

    W1, W2 = W1i, W2i
    zs = []
    for c0 in range(0, T, b):
        W1c, W2c = W1, W2
        G1 = torch.zeros_like(W1c)
        G2 = torch.zeros_like(W2c)
        W1t, W2t = W1c, W2c
        for t in range(c0, min(c0 + b, T)):
            u = torch.einsum("nhj,nj->nh", W1c, K[:, t])
            a = silu_t(u)
            if loss == "mse":
                r = torch.einsum("nih,nh->ni", W2c, a) - V[:, t]
            elif loss == "dot":
                r = -V[:, t]
            else:
                raise ValueError(loss)
            du = torch.einsum("nih,ni->nh", W2c, r) * dsilu_t(u)
            G1 = G1 + torch.einsum("nh,nj->nhj", du, K[:, t])
            G2 = G2 + torch.einsum("ni,nh->nih", r, a)
            W1t = W1c - eta * G1
            W2t = W2c - eta * G2
            zs.append(torch.einsum("nih,nh->ni", W2t, silu_t(torch.einsum("nhj,nj->nh", W1t, Q[:, t]))))
        W1, W2 = W1t, W2t
    Z = torch.stack(zs, dim=1) if zs else torch.zeros((N, 0, d), dtype=torch.float64)
    outs, grads = [Z], [torch.tensor(dz2)]
    if dw1_out is not None:
        outs.append(W1)
        grads.append(torch.tensor(_broadcast_state(dw1_out, lead, np.float64)))
    if dw2_out is not None:
        outs.append(W2)
        grads.append(torch.tensor(_broadcast_state(dw2_out, lead, np.float64)))
    res = torch.autograd.grad(outs, (Q, K, V, W1i, W2i), grads, allow_unused=True)
    shape = tuple(lead) + (T, d)
    tok = lambda t: (np.zeros((N, T, d)) if t is None else t.numpy()).reshape(shape)
    st = lambda t, like, sh: (np.zeros(like.shape) if t is None else t.numpy()).reshape(tuple(lead) + sh)
    return (tok(res[0]), tok(res[1]), tok(res[2]), st(res[3], W1i, (h, d)), st(res[4], W2i, (d, h)))


def ttt_layer_vjp(kind, q, k, v, state, eta, chunk, dz, dstate=None, *, causal=True, epochs=1,
                  eta_tok=None, loss="mse", act="silu", ln=None):
    """Vector-Jacobian product of every TTT layer variant of ttt_linear / ttt_mlp: causal or
    not, mini-batches and epochs, per-token rate factors, either loss, SiLU or GELU, with or
    without the paper's layer norm and residual.

    The outer loop trains the projections that make q, k, v, the initial state, the rates
    and the layer-norm parameters through the inner updates (wmrh.cn summary, section 2.2,
    the outer loop and its "gradient of the gradient"; section 2.2.3, the learnable rate;
    "Fast weights" page, opening paragraph and section 2: the outer gradient runs through
    the whole update trajectory; ViT3 news page, section 1: K and V are learned end to end).

    kind: "linear" (state = (w0,)) or "mlp" (state = (w1, w2)); every other argument as in
    ttt_linear / ttt_mlp, ln = (gamma, beta, eps).  dz [..., T, d]: upstream gradient of z;
    dstate: upstream gradients of the final states (a tuple like state) or None.
    Returns (dq, dk, dv, dstate..., deta_tok, dgamma, dbeta), per chain; deta_tok is None
    without rates, dgamma and dbeta are None without ln.

    The definition, written out: the recurrence of ttt_linear / ttt_mlp in float64 torch
    tensors, where each token's inner gradient is itself taken by torch.autograd (with
    create_graph, at the chunk-start weights) rather than written out, and the whole
    trajectory is differentiated by torch.autograd in reverse mode.
    """
    import torch
    if kind not in ("linear", "mlp"):
        raise ValueError(kind)
    if loss not in LOSSES:
        raise ValueError(loss)
    q2, lead = _flatten_tokens(q, np.float64)
    k2, _ = _flatten_tokens(k, np.float64)
    v2, _ = _flatten_tokens(v, np.float64)
    N, T, d = q2.shape
    b = _check_chunk(T, chunk)
    epochs = _check_epochs(epochs, causal)
    Q = torch.tensor(q2, requires_grad=True)
    K = torch.tensor(k2, requires_grad=True)
    V = torch.tensor(v2, requires_grad=True)
    W0 = [torch.tensor(_broadcast_state(s, lead, np.float64), requires_grad=True) for s in state]
    E = None
    if eta_tok is not None:
        E = torch.tensor(np.broadcast_to(np.asarray(eta_tok, np.float64), tuple(lead) + (T,))
                         .reshape(N, T).copy(), requires_grad=True)
    G_, B_, eps = None, None, None
    if ln is not None:
        G_ = torch.tensor(np.broadcast_to(np.asarray(ln[0], np.float64), tuple(lead) + (d,))
                          .reshape(N, d).copy(), requires_grad=True)
        B_ = torch.tensor(np.broadcast_to(np.asarray(ln[1], np.float64), tuple(lead) + (d,))
                          .reshape(N, d).copy(), requires_grad=True)
        eps = float(ln[2])

    def activation(u):
        if act == "silu":
            return u * torch.sigmoid(u)
        if act == "gelu":
            return 0.5 * u * (1.0 + torch.erf(u / np.sqrt(2.0)))
        raise ValueError(act)

    def f(x, W):
        if kind == "linear":
            y = torch.einsum("nij,nj->ni", W[0], x)
        else:
            y = torch.einsum("nih,nh->ni", W[1], activation(torch.einsum("nhj,nj->nh", W[0], x)))
        if G_ is None:
            return y
        mu = y.mean(dim=-1, keepdim=True)
        var = ((y - mu) ** 2).mean(dim=-1, keepdim=True)
        return x + G_ * (y - mu) / torch.sqrt(var + eps) + B_

    def inner_loss(fx, vt):
        if loss == "mse":
            return 0.5 * ((fx - vt) ** 2).sum()
        return -(vt * fx).sum()

    W = W0
    zs = [None] * T
    for c0 in [c for _ in range(epochs) for c in range(0, T, b)]:
        Wc = W
        G = [torch.zeros_like(w) for w in Wc]
        Wt = Wc
        for t in range(c0, min(c0 + b, T)):
            g = torch.autograd.grad(inner_loss(f(K[:, t], Wc), V[:, t]), Wc, create_graph=True,
                                    allow_unused=True)
            g = [torch.zeros_like(w) if gi is None else gi for gi, w in zip(g, Wc)]
            G = [Gi + (gi if E is None else E[:, t].reshape((N,) + (1,) * (gi.dim() - 1)) * gi)
                 for Gi, gi in zip(G, g)]
            Wt = [w - eta * Gi for w, Gi in zip(Wc, G)]
            if causal:
                zs[t] = f(Q[:, t], Wt)
        W = Wt
    if not causal:
        for t in range(T):
            zs[t] = f(Q[:, t], W)
    Z = torch.stack(zs, dim=1) if T else torch.zeros((N, 0, d), dtype=torch.float64)
    outs, grads = [Z], [torch.tensor(_flatten_tokens(dz, np.float64)[0])]
    if dstate is not None:
        for w, ds in zip(W, dstate):
            if ds is not None:
                outs.append(w)
                grads.append(torch.tensor(_broadcast_state(ds, lead, np.float64)))
    wrt = [Q, K, V] + W0 + [x for x in (E, G_, B_) if x is not None]
    got = list(torch.autograd.grad(outs, wrt, grads, allow_unused=True))
    zero_like = lambda t, ref: np.zeros(ref.shape) if t is None else t.numpy()
    res = [zero_like(got[i], x).reshape(tuple(lead) + (T, d)) for i, x in enumerate((Q, K, V))]
    for j, w in enumerate(W0):
        res.append(zero_like(got[3 + j], w).reshape(tuple(lead) + tuple(w.shape[1:])))
    i = 3 + len(W0)
    if E is not None:
        res.append(zero_like(got[i], E).reshape(tuple(lead) + (T,)))
        i += 1
    else:
        res.append(None)
    if G_ is not None:
        res.append(zero_like(got[i], G_).reshape(tuple(lead) + (d,)))
        res.append(zero_like(got[i + 1], B_).reshape(tuple(lead) + (d,)))
    else:
        res += [None, None]
    return tuple(res)
