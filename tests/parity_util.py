"""Shared helpers of the GPU parity tests: run the HIP path and the oracle on the same
seeded inputs and compare slab by slab (one slab = one (batch, head) sequence)."""
import numpy as np

from oracle import ttt_oracle as O
from test_sequence_layers_amd.workloads import (make_inputs, make_ln_params, make_token_rates,
                                                workload)

FP32_TOL = 1e-4   # relative Frobenius error per slab, float32 I/O
LN_EPS = 1e-6     # layer-norm epsilon of the paper's inner models in the parity cases
BF16_TOL = 2e-2   # relative Frobenius error per slab, bfloat16 I/O, float32 state


def tol_for(io):
    return FP32_TOL if io == "f32" else BF16_TOL


def slab_rel(z, ref):
    """max over (b, h) of ||z - ref||_F / ||ref||_F (ref all-zero slabs use the abs error)."""
    z = np.asarray(z, np.float64)
    ref = np.asarray(ref, np.float64)
    lead = ref.shape[:-2]
    zz = z.reshape((-1,) + ref.shape[-2:])
    rr = ref.reshape((-1,) + ref.shape[-2:])
    num = np.sqrt(((zz - rr) ** 2).sum(axis=(-2, -1)))
    den = np.sqrt((rr ** 2).sum(axis=(-2, -1)))
    rel = np.where(den > 0, num / np.maximum(den, 1e-300), num)
    return float(rel.max()) if rel.size else 0.0, rel.reshape(lead)


def to_device(inp, io):
    import torch
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    out = {}
    for key in ("q", "k", "v"):
        out[key] = torch.from_numpy(np.ascontiguousarray(inp[key])).to("cuda").to(dt).contiguous()
    for key in ("w0", "w1", "w2", "eta_tok", "ln_w", "ln_b"):
        if key in inp:
            out[key] = torch.from_numpy(np.ascontiguousarray(inp[key])).to("cuda").contiguous()
    return out


def run_gpu(kind, dev, eta, chunk, causal, return_state=True, loss="mse", epochs=1):
    """HIP path; with "ln_w" / "ln_b" in dev the paper's inner model (x + LN(f_res(x)), GELU
    in the MLP)."""
    import test_sequence_layers_amd as ttt
    et = dev.get("eta_tok")
    if "ln_w" in dev:
        ln = (dev["ln_w"], dev["ln_b"])
        if kind == "linear":
            return ttt.ttt_linear_ln_fwd(dev["q"], dev["k"], dev["v"], dev["w0"], *ln, eta, chunk,
                                         causal, ln_eps=LN_EPS, eta_tok=et, loss=loss,
                                         epochs=epochs, return_state=return_state)
        return ttt.ttt_mlp_ln_fwd(dev["q"], dev["k"], dev["v"], dev["w1"], dev["w2"], *ln, eta,
                                  chunk, causal, ln_eps=LN_EPS, eta_tok=et, loss=loss,
                                  epochs=epochs, return_state=return_state)
    if kind == "linear":
        return ttt.ttt_linear_fwd(dev["q"], dev["k"], dev["v"], dev["w0"], eta, chunk, causal,
                                  eta_tok=et, loss=loss, epochs=epochs, return_state=return_state)
    if kind == "delta":
        return ttt.delta_rule_fwd(dev["q"], dev["k"], dev["v"], dev["w0"], eta, eta_tok=et,
                                  return_state=return_state)
    return ttt.ttt_mlp_fwd(dev["q"], dev["k"], dev["v"], dev["w1"], dev["w2"], eta, chunk,
                           causal, eta_tok=et, loss=loss, epochs=epochs, return_state=return_state)


def run_oracle(kind, inp, eta, chunk, causal, sel=None, loss="mse", epochs=1):
    """Oracle on (optionally) a subset of (b, h) pairs: sel = list of (b, h)."""
    q, k, v = inp["q"], inp["k"], inp["v"]
    et = inp.get("eta_tok")
    lw, lb = inp.get("ln_w"), inp.get("ln_b")
    if sel is not None:
        bs = [b for b, _ in sel]
        hs = [h for _, h in sel]
        q, k, v = q[bs, hs][None], k[bs, hs][None], v[bs, hs][None]
        et = et[bs, hs][None] if et is not None else None
        lw = lw[hs][None] if lw is not None else None
        lb = lb[hs][None] if lb is not None else None
        pick = lambda w: w[hs][None] if w.ndim == 3 else w[bs, hs][None]
    else:
        pick = lambda w: w
    ln = (lw, lb, LN_EPS) if lw is not None else None
    if kind == "linear":
        return O.ttt_linear(q, k, v, pick(inp["w0"]), eta, chunk, causal, loss=loss, eta_tok=et,
                            epochs=epochs, ln=ln)
    if kind == "delta":
        return O.delta_rule(q, k, v, pick(inp["w0"]), eta, eta_tok=et)
    return O.ttt_mlp(q, k, v, pick(inp["w1"]), pick(inp["w2"]), eta, chunk, causal, loss=loss,
                     eta_tok=et, epochs=epochs, ln=ln, act="gelu" if ln is not None else "silu")


def to_np(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy()
