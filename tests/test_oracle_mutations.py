"""Plant plausible mistakes in a copy of the oracle (CPU only) and check the pins catch them.

Each mutation edits the oracle's source text (a dropped term, a wrong sign, a transposed
operand, the wrong weights for a gradient or an output) and loads the edited text as a
throw-away module.  The pins of test_oracle_pins are then run against that module; at
least one of them must fail for every mutation.  The real oracle is never modified.
"""
import inspect
import types

import pytest

import oracle.ttt_oracle as real_oracle
import tests.test_oracle_pins as pins

MUTATIONS = {
    "output_reads_chunk_start_weights": (
        "z[:, t] = linear_f(Wt, q2[:, t], lnp)", "z[:, t] = linear_f(Wc, q2[:, t], lnp)"),
    "gradient_at_current_not_chunk_start": (
        "G = G + linear_grad(Wc, k2[:, t]", "G = G + linear_grad(Wt, k2[:, t]"),
    "dropped_learning_rate": ("Wt = Wc - eta * G", "Wt = Wc - G"),
    "wrong_update_sign": ("Wt = Wc - eta * G", "Wt = Wc + eta * G"),
    "transposed_linear_gradient": (
        'return np.einsum("ni,nj->nij", r, k)', 'return np.einsum("ni,nj->nij", k, r)'),
    "transposed_linear_model": (
        'return _wrap(np.einsum("nij,nj->ni", W, x)', 'return _wrap(np.einsum("nji,nj->ni", W, x)'),
    "dot_loss_sign": ('    if loss == "dot":\n        return -v', '    if loss == "dot":\n        return v'),
    "delta_rule_transposed_write": (
        'W = W + eta * np.einsum("ni,nj->nij", err, kt)',
        'W = W + eta * np.einsum("ni,nj->nij", kt, err)'),
    "delta_rule_output_before_write": (
        '            W = W + et[:, t, None, None] * np.einsum("ni,nj->nij", err, kt)\n'
        '        z[:, t] = np.einsum("nij,nj->ni", W, q2[:, t])',
        '            W = W + et[:, t, None, None] * np.einsum("ni,nj->nij", err, kt)\n'
        '        z[:, t] = np.einsum("nij,nj->ni", W - np.einsum("ni,nj->nij", err, kt) * '
        '(eta if et is None else et[:, t, None, None]), q2[:, t])'),
    "silu_derivative_missing_term": ("return s * (1.0 + u * (1.0 - s))", "return s"),
    "silu_is_sigmoid": ("return u / (1.0 + np.exp(-u))", "return 1.0 / (1.0 + np.exp(-u))"),
    "mlp_backward_skips_activation": (
        'du = np.einsum("nih,ni->nh", W2, r) * dfa(u)',
        'du = np.einsum("nih,ni->nh", W2, r)'),
    "mlp_second_layer_not_updated": ("W2t = W2c - eta * G2", "W2t = W2c"),
    "mlp_gradient_at_current_weights": (
        "g1, g2 = mlp_grad(W1c, W2c, k2[:, t]", "g1, g2 = mlp_grad(W1t, W2t, k2[:, t]"),
    "last_token_of_chunk_dropped": (
        "for t in range(c0, min(c0 + b, T)):\n            if et is None:\n                G = G + linear_grad",
        "for t in range(c0, min(c0 + b, T) - 1):\n            if et is None:\n                G = G + linear_grad"),
    "token_rate_of_previous_token": (
        "G = G + et[:, t, None, None] * linear_grad", "G = G + et[:, max(t - 1, 0), None, None] * linear_grad"),
    "token_rate_applied_twice": (
        "                G = G + et[:, t, None, None] * linear_grad(Wc, k2[:, t], v2[:, t], loss, lnp)\n"
        "                Wt = Wc - G",
        "                G = G + et[:, t, None, None] * linear_grad(Wc, k2[:, t], v2[:, t], loss, lnp)\n"
        "                Wt = Wc - eta * G"),
    "mlp_second_layer_ignores_token_rate": (
        "G2 = G2 + et[:, t, None, None] * g2", "G2 = G2 + eta * g2"),
    "delta_rule_ignores_token_rate": (
        'W = W + et[:, t, None, None] * np.einsum("ni,nj->nij", err, kt)',
        'W = W + eta * np.einsum("ni,nj->nij", err, kt)'),
    "vjp_residual_at_current_weights": (
        'r = torch.einsum("nij,nj->ni", Wc, K[:, t]) - V[:, t]',
        'r = torch.einsum("nij,nj->ni", Wt, K[:, t]) - V[:, t]'),
    "vjp_output_before_update": (
        'zs.append(torch.einsum("nij,nj->ni", Wt, Q[:, t]))',
        'zs.append(torch.einsum("nij,nj->ni", Wc, Q[:, t]))'),
    "mlp_vjp_gradient_at_current_weights": (
        'u = torch.einsum("nhj,nj->nh", W1c, K[:, t])', 'u = torch.einsum("nhj,nj->nh", W1t, K[:, t])'),
    "mlp_vjp_output_before_update": (
        'zs.append(torch.einsum("nih,nh->ni", W2t, silu_t(torch.einsum("nhj,nj->nh", W1t, Q[:, t]))))',
        'zs.append(torch.einsum("nih,nh->ni", W2c, silu_t(torch.einsum("nhj,nj->nh", W1c, Q[:, t]))))'),
    "epochs_ignored": (
        "chunk_starts = [c0 for _ in range(epochs) for c0", "chunk_starts = [c0 for _ in range(1) for c0"),
    "mlp_epochs_ignored": (
        "    chunk_starts = [c0 for _ in range(epochs) for c0 in range(0, T, b)]\n    for c0 in chunk_starts:\n        W1c",
        "    chunk_starts = [c0 for _ in range(1) for c0 in range(0, T, b)]\n    for c0 in chunk_starts:\n        W1c"),
    "epoch_restarts_from_initial_weights": (
        "    for c0 in chunk_starts:\n        Wc = W.copy()",
        "    for i, c0 in enumerate(chunk_starts):\n"
        "        W = _broadcast_state(w0, lead, dtype) if (i and c0 == 0) else W\n"
        "        Wc = W.copy()"),
    "ln_vjp_drops_variance_term": (
        "gg - gg.mean(axis=-1, keepdims=True) - xh * (gg * xh).mean(axis=-1, keepdims=True)",
        "gg - gg.mean(axis=-1, keepdims=True)"),
    "ln_vjp_drops_mean_term": (
        "gg - gg.mean(axis=-1, keepdims=True) - xh", "gg - xh"),
    "ln_unbiased_variance": (
        "var = ((y - mu) ** 2).mean(axis=-1, keepdims=True)",
        "var = ((y - mu) ** 2).sum(axis=-1, keepdims=True) / (y.shape[-1] - 1)"),
    "ln_eps_outside_sqrt": (
        "return gamma * (y - mu) / np.sqrt(var + eps) + beta",
        "return gamma * (y - mu) / (np.sqrt(var) + eps) + beta"),
    "ln_residual_dropped": (
        "return res if ln is None else x + layer_norm(", "return res if ln is None else layer_norm("),
    "ln_gradient_skips_layer_norm": (
        "return err if ln is None else layer_norm_vjp(res, ln[0], ln[2], err)", "return err"),
    "gelu_derivative_missing_density_term": (
        "return 0.5 * (1.0 + erf(u / np.sqrt(2.0))) + u * np.exp(-0.5 * u * u) / np.sqrt(2.0 * np.pi)",
        "return 0.5 * (1.0 + erf(u / np.sqrt(2.0)))"),
    "gelu_is_silu": ('"gelu": (gelu, dgelu)', '"gelu": (silu, dsilu)'),
    "layer_vjp_inner_gradient_at_current_weights": (
        "g = torch.autograd.grad(inner_loss(f(K[:, t], Wc), V[:, t]), Wc,",
        "g = torch.autograd.grad(inner_loss(f(K[:, t], Wt), V[:, t]), Wt,"),
    "layer_vjp_rate_dropped": (
        "G = [Gi + (gi if E is None else", "G = [Gi + (gi if True else"),
    "layer_vjp_noncausal_reads_initial_weights": (
        "            zs[t] = f(Q[:, t], W)\n", "            zs[t] = f(Q[:, t], W0)\n"),
    "layer_vjp_ln_residual_dropped": (
        "return x + G_ * (y - mu) / torch.sqrt(var + eps) + B_",
        "return G_ * (y - mu) / torch.sqrt(var + eps) + B_"),
    "layer_vjp_epochs_ignored": (
        "for c0 in [c for _ in range(epochs) for c in range(0, T, b)]:",
        "for c0 in [c for _ in range(1) for c in range(0, T, b)]:"),
    "layer_vjp_gelu_is_silu": (
        "            return 0.5 * u * (1.0 + torch.erf(u / np.sqrt(2.0)))",
        "            return u * torch.sigmoid(u)"),
    "noncausal_reads_initial_weights": (
        "    if not causal:\n        for t in range(T):\n            z[:, t] = linear_f(W, q2[:, t], lnp)",
        "    if not causal:\n        W = _broadcast_state(w0, lead, dtype)\n"
        "        for t in range(T):\n            z[:, t] = linear_f(W, q2[:, t], lnp)"),
}


def _pin_calls():
    calls = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if not params:
            calls.append((name, fn, {}))
            continue
        m = params[0]
        argnames = [a.strip() for a in m.args[0].split(",")]
        for vals in m.args[1]:
            if len(argnames) == 1:
                vals = (vals,)
            calls.append((f"{name}{vals}", fn, dict(zip(argnames, vals))))
    return calls


def _mutant(old, new):
    src = inspect.getsource(real_oracle)
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new, 1), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, monkeypatch):
    old, new = MUTATIONS[name]
    monkeypatch.setattr(pins, "O", _mutant(old, new))
    caught = []
    for pin_name, fn, kw in _pin_calls():
        try:
            fn(**kw)
        except Exception:  # assertion or a shape error both count as caught
            caught.append(pin_name)
    assert caught, f"no pin caught mutation {name}"


def test_unmutated_copy_passes_every_pin(monkeypatch):
    """Control: the exec'd copy of the untouched source passes all pins."""
    monkeypatch.setattr(pins, "O", _mutant("import numpy as np", "import numpy as np"))
    for pin_name, fn, kw in _pin_calls():
        fn(**kw)
