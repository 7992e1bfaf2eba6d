"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on seeded inputs.

Small cases span several chunks/tiles and a ragged tail.  The five measured workloads run at
full size, in the launch configuration the benchmark times, and every (batch, head)
sequence is compared (the oracle runs them in parallel CPU worker processes).  Each
comparison asserts two measures per sequence, the relative Frobenius error and the largest
element-wise error relative to the sequence's largest reference value (tests/parity_util.py
states the bounds and their derivation).
"""
import numpy as np
import pytest
import sys

from tests.parity_util import (BF16_LN_ELEM_TOL, BF16_TOL, FP32_TOL, check_close, make_inputs, make_ln_params,
                               make_token_rates, run_gpu, run_oracle, run_oracle_all, to_device,
                               to_np, tol_for, workload)

pytestmark = pytest.mark.gpu


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _check(kind, w, inp, sel=None, state_tol=None, loss="mse", epochs=1, full=False):
    """sel: compare only these (b, h) sequences; full: every sequence, the oracle in parallel
    worker processes (the full-size workloads)."""
    _note(f"[parity] {kind} {w.name} B={w.B} H={w.H} T={w.T} d={w.d} h={w.h} chunk={w.chunk} "
          f"causal={w.causal} io={w.io} seed={w.seed} loss={loss} rates={'eta_tok' in inp} "
          f"epochs={epochs} paper_ln={'ln_w' in inp}")
    dev = to_device(inp, w.io)
    out = run_gpu(kind, dev, w.eta, w.chunk, w.causal, loss=loss, epochs=epochs)
    import torch
    torch.cuda.synchronize()
    z = to_np(out[0])
    states = [to_np(s) for s in out[1:]]
    del out, dev
    if full:
        _note("[parity]   oracle over every sequence (worker processes)")
        ref = run_oracle_all(kind, inp, w.eta, w.chunk, w.causal, loss=loss, epochs=epochs)
    else:
        ref = run_oracle(kind, inp, w.eta, w.chunk, w.causal, sel, loss=loss, epochs=epochs)
    if sel is not None:
        bs = [b for b, _ in sel]
        hs = [h for _, h in sel]
        z = z[bs, hs][None]
        states = [s[bs, hs][None] for s in states]
    tol = tol_for(w.io)
    etol = BF16_LN_ELEM_TOL if ("ln_w" in inp and w.io == "bf16") else None
    rel, _ = check_close("z", z, ref[0], tol, _note, elem_tol=etol)
    for i, (s, r) in enumerate(zip(states, ref[1:])):
        check_close(f"state{i}", s, r, state_tol or tol, _note, elem_tol=etol)
    return rel


# ------------------------------------------------------------------ TTT-Linear

def test_linear_config_tiny_fp32():
    w = workload(0)
    _check("linear", w, make_inputs(w))


@pytest.mark.parametrize("d", [16, 32, 64])
@pytest.mark.parametrize("chunk", [1, 5, 16, 77])
@pytest.mark.parametrize("causal", [True, False])
def test_linear_fp32_shapes(d, chunk, causal):
    w = workload(0).replace(B=2, H=3, T=77, d=d, chunk=chunk, causal=causal, init="normal",
                            eta=0.2, seed=7 + d + chunk)
    _check("linear", w, make_inputs(w))


def test_linear_fp32_per_batch_state():
    w = workload(0).replace(B=3, H=2, T=40, d=32, chunk=8, init="normal", seed=3)
    inp = make_inputs(w)
    rng = np.random.default_rng(0)
    inp["w0"] = (0.05 * rng.standard_normal((3, 2, 32, 32))).astype(np.float32)
    _check("linear", w, inp)


@pytest.mark.parametrize("T", [16, 200, 333])
def test_linear_bf16_d64_chunk16(T):
    w = workload(1).replace(B=2, H=3, T=T, seed=11 + T)
    _check("linear", w, make_inputs(w))


@pytest.mark.parametrize("chunk,causal", [(16, False), (8, True), (32, True), (1, True)])
def test_linear_bf16_other_modes(chunk, causal):
    w = workload(1).replace(B=1, H=4, T=130, chunk=chunk, causal=causal, seed=5 + chunk)
    _check("linear", w, make_inputs(w))


@pytest.mark.parametrize("B,H", [(13, 1), (3, 5)])
def test_linear_bf16_chain_count_not_multiple_of_8(B, H):
    # the matrix-core kernel maps chains to block indices in groups of 8 (both workgroups of
    # a chain on one XCD); 13 and 15 chains leave the last group partly empty
    w = workload(1).replace(B=B, H=H, T=70, init="normal", seed=60 + B)
    _check("linear", w, make_inputs(w))


def test_linear_config_full_size():
    w = workload(1)
    _check("linear", w, make_inputs(w), full=True)


# ------------------------------------------------------------------ delta rule

@pytest.mark.parametrize("d,io", [(16, "f32"), (64, "f32"), (64, "bf16"), (32, "bf16")])
def test_delta_small(d, io):
    w = workload(2).replace(B=2, H=2, T=150, d=d, io=io, init="normal", seed=21 + d)
    _check("delta", w, make_inputs(w))


def test_delta_bf16_chain_count_not_multiple_of_8():
    w = workload(2).replace(B=5, H=3, T=45, init="normal", seed=70)
    _check("delta", w, make_inputs(w))


def test_delta_config_full_size():
    w = workload(2)
    _check("delta", w, make_inputs(w), full=True)


# ------------------------------------------------------------------ TTT-MLP

@pytest.mark.parametrize("chunk,causal", [(1, True), (4, True), (16, True), (37, True),
                                          (37, False), (10, False)])
def test_mlp_fp32_shapes(chunk, causal):
    w = workload(3).replace(B=2, H=2, T=37, d=16, h=32, chunk=chunk, causal=causal, io="f32",
                            seed=31 + chunk)
    _check("mlp", w, make_inputs(w))


def test_mlp_bf16_h256_small():
    w = workload(3).replace(B=1, H=3, T=100, seed=41)
    _check("mlp", w, make_inputs(w))


def test_mlp_vision_small():
    w = workload(4).replace(B=2, H=3, seed=42)
    _check("mlp", w, make_inputs(w))


# One full-batch step at the vision shape runs the kernel that splits the hidden units over two
# waves and the tiles over two token groups: one token, a partial tile, one and two whole tiles,
# odd and even tile counts (the second token group's last round is then empty), both losses,
# rates, and an odd chain count.
@pytest.mark.parametrize("T,B,H,loss,rates", [
    (1, 1, 3, "mse", False), (5, 2, 1, "mse", True), (16, 1, 2, "mse", False),
    (17, 1, 3, "dot", False), (33, 3, 1, "mse", True), (48, 1, 1, "dot", True),
    (100, 1, 3, "mse", False)])
def test_mlp_vision_single_step_shapes(T, B, H, loss, rates):
    w = workload(4).replace(B=B, H=H, T=T, chunk=T, eta=0.5, seed=60 + T)
    inp = _with_rates(w, 13) if rates else make_inputs(w)
    _check("mlp", w, inp, loss=loss)


def test_mlp_config_full_size():
    w = workload(3)
    _check("mlp", w, make_inputs(w), full=True)


def test_mlp_vision_config_full_size():
    w = workload(4)
    _check("mlp", w, make_inputs(w), full=True)


# ------------------------------------------------------------------ two workgroups per chain
# ttt_mlp_fwd_ws / ttt_mlp_ln_fwd_ws: the recursion on one compute unit, the outputs on a
# second that replays the same updates.  Same operands and products in the same order as the
# one-workgroup kernel, so z and the final states must match it bit for bit; and the oracle.

def _ws_same_as_one_workgroup(w, inp, loss="mse"):
    import torch
    import test_sequence_layers_amd as ttt
    dev = to_device(inp, w.io)
    one = run_gpu("mlp", dev, w.eta, w.chunk, w.causal, loss=loss)
    ws_bytes = ttt.ttt_mlp_fwd_workspace_size(w.B, w.H, w.T, w.d, w.h, w.chunk, w.causal, w.io)
    assert ws_bytes > 0
    # a workspace that holds garbage (and, on the second call, the first call's flags)
    ws = torch.full((ws_bytes,), 0xA5, dtype=torch.uint8, device=dev["q"].device)
    et = dev.get("eta_tok")
    for rep in range(2):
        if "ln_w" in dev:
            two = ttt.ttt_mlp_ln_fwd_ws(dev["q"], dev["k"], dev["v"], dev["w1"], dev["w2"],
                                        dev["ln_w"], dev["ln_b"], w.eta, w.chunk, w.causal,
                                        workspace=ws, ln_eps=1e-6, eta_tok=et, loss=loss,
                                        return_state=True)
        else:
            two = ttt.ttt_mlp_fwd_ws(dev["q"], dev["k"], dev["v"], dev["w1"], dev["w2"], w.eta,
                                     w.chunk, w.causal, workspace=ws, eta_tok=et, loss=loss,
                                     return_state=True)
        torch.cuda.synchronize()
        for name, a, b in zip(("z", "w1_out", "w2_out"), one, two):
            same = torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))
            _note(f"[parity]   call {rep}: {name} bit-identical to the one-workgroup kernel: {same}")
            assert same, name


@pytest.mark.parametrize("T,B,H", [(16, 1, 1), (17, 1, 3), (100, 2, 3), (333, 3, 3), (2048, 1, 2)])
def test_mlp_ws_matches_one_workgroup_kernel(T, B, H):
    w = workload(3).replace(B=B, H=H, T=T, seed=70 + T)
    _note(f"[parity] mlp_ws bit-identity B={B} H={H} T={T}")
    _ws_same_as_one_workgroup(w, make_inputs(w))


@pytest.mark.parametrize("loss,rates,paper", [("dot", False, False), ("mse", True, False),
                                              ("mse", False, True), ("dot", True, True)])
def test_mlp_ws_variants_match_one_workgroup_kernel(loss, rates, paper):
    w = workload(3).replace(B=2, H=3, T=150, seed=80)
    inp = _with_rates(w, 15) if rates else make_inputs(w)
    if paper:
        inp["ln_w"], inp["ln_b"] = make_ln_params(w, 10)
    _note(f"[parity] mlp_ws variant loss={loss} rates={rates} paper={paper}")
    _ws_same_as_one_workgroup(w, inp, loss=loss)


@pytest.mark.parametrize("T", [16, 77, 200])
def test_mlp_ws_small(T):
    w = workload(3).replace(B=2, H=3, T=T, seed=90 + T)
    _check("mlp_ws", w, make_inputs(w))


def test_mlp_ws_config_full_size():
    w = workload(3)
    _check("mlp_ws", w, make_inputs(w), full=True)


def test_mlp_ws_config_full_size_same_as_one_workgroup():
    w = workload(3)
    _ws_same_as_one_workgroup(w, make_inputs(w))


def test_mlp_ws_paper_config_full_size():
    w = workload(3)
    inp = make_inputs(w)
    inp["ln_w"], inp["ln_b"] = make_ln_params(w, 8)
    _check("mlp_ws", w, inp, full=True)


def test_mlp_ws_formal_protocol_is_bit_identical():
    # the agent-scope hand-off (the path for workgroups on different XCCs), forced
    import test_sequence_layers_amd as ttt
    w = workload(3).replace(B=2, H=3, T=333, seed=95)
    prev = ttt.set_split_debug(1)
    try:
        _note("[parity] mlp_ws with the agent-scope hand-off forced")
        _ws_same_as_one_workgroup(w, make_inputs(w))
    finally:
        ttt.set_split_debug(prev)


def test_mlp_ws_forced_failure_fills_nan_and_returns():
    # the output workgroups' bounded wait, made to fail from the host: z is all NaN, the
    # recursion's final states are still right, and the next call is normal again
    import torch
    import test_sequence_layers_amd as ttt
    w = workload(3).replace(B=2, H=3, T=100, seed=96)
    dev = to_device(make_inputs(w), w.io)
    one = run_gpu("mlp", dev, w.eta, w.chunk, w.causal)
    prev = ttt.set_split_debug(2)
    try:
        _note("[parity] mlp_ws with a forced failure of the output workgroups' wait")
        two = run_gpu("mlp_ws", dev, w.eta, w.chunk, w.causal)
        torch.cuda.synchronize()
    finally:
        ttt.set_split_debug(prev)
    assert torch.isnan(two[0].float()).all()
    assert torch.equal(one[1], two[1]) and torch.equal(one[2], two[2])
    _ws_same_as_one_workgroup(w, make_inputs(w))


def test_mlp_ws_per_batch_initial_states():
    # W1, W2 per (batch, head) ([B, H, ...], w_batch_stride = H h d) and a ragged last chunk
    w = workload(3).replace(B=3, H=2, T=77, seed=94)
    inp = make_inputs(w)
    rng = np.random.default_rng(194)
    inp["w1"] = (0.02 * rng.standard_normal((w.B, w.H, w.h, w.d))).astype(np.float32)
    inp["w2"] = (0.02 * rng.standard_normal((w.B, w.H, w.d, w.h))).astype(np.float32)
    _note("[parity] mlp_ws with per-batch initial states")
    _ws_same_as_one_workgroup(w, inp)
    _check("mlp_ws", w, inp)


def test_mlp_ws_more_sequences_than_resident_workgroups():
    # 300 sequences: 600 workgroups of one compute unit each, more than the chip holds at
    # once; the recursion workgroups (lower block indices) are dispatched first and never
    # wait, so every output workgroup's wait ends
    w = workload(3).replace(B=25, H=12, T=128, seed=97)
    _note("[parity] mlp_ws with 600 workgroups")
    _ws_same_as_one_workgroup(w, make_inputs(w))


def test_mlp_ws_two_calls_on_two_streams():
    # two calls in flight at once on two streams, each with its own workspace
    import torch
    import test_sequence_layers_amd as ttt
    ws_list, outs, refs = [], [], []
    cases = [workload(3).replace(B=4, H=12, T=512, seed=98), workload(3).replace(B=3, H=12, T=333, seed=99)]
    devs = [to_device(make_inputs(w), w.io) for w in cases]
    for w, dev in zip(cases, devs):
        refs.append(run_gpu("mlp", dev, w.eta, w.chunk, w.causal)[0])
        n = ttt.ttt_mlp_fwd_workspace_size(w.B, w.H, w.T, w.d, w.h, w.chunk, w.causal, w.io)
        ws_list.append(torch.empty(n, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    _note("[parity] mlp_ws on two streams at once")
    for w, dev, ws, st in zip(cases, devs, ws_list, streams):
        with torch.cuda.stream(st):
            outs.append(ttt.ttt_mlp_fwd_ws(dev["q"], dev["k"], dev["v"], dev["w1"], dev["w2"], w.eta,
                                           w.chunk, w.causal, workspace=ws, stream=st))
    torch.cuda.synchronize()
    for a, b in zip(refs, outs):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_mlp_ws_other_shapes_run_the_plain_call():
    # no workspace is needed (size 0) for any other shape; the _ws call is then ttt_mlp_fwd
    import test_sequence_layers_amd as ttt
    w = workload(3).replace(B=1, H=2, T=37, d=16, h=32, io="f32", seed=99)
    assert ttt.ttt_mlp_fwd_workspace_size(w.B, w.H, w.T, w.d, w.h, w.chunk, w.causal, w.io) == 0
    _check("mlp_ws", w, make_inputs(w))


# ------------------------------------------------------------------ edge cases

def test_zero_length_sequence_returns_initial_state():
    import torch
    import test_sequence_layers_amd as ttt
    q = torch.zeros((2, 3, 0, 16), device="cuda")
    w0 = torch.randn((3, 16, 16), device="cuda")
    z, w = ttt.ttt_linear_fwd(q, q, q, w0, 0.1, 16, return_state=True)
    torch.cuda.synchronize()
    assert z.shape == (2, 3, 0, 16)
    assert torch.equal(w, w0.expand(2, 3, 16, 16))


def test_zero_learning_rate_is_a_fixed_linear_map():
    import torch
    import test_sequence_layers_amd as ttt
    w = workload(1).replace(B=1, H=2, T=48)
    inp = make_inputs(w)
    dev = to_device(inp, "f32")
    z = ttt.ttt_linear_fwd(dev["q"], dev["k"], dev["v"], dev["w0"], 0.0, 16)
    ref = torch.einsum("hij,bhtj->bhti", dev["w0"], dev["q"])
    torch.cuda.synchronize()
    assert torch.allclose(z, ref, atol=1e-5, rtol=1e-5)


def test_unsupported_shape_raises():
    import torch
    import test_sequence_layers_amd as ttt
    q = torch.zeros((1, 1, 4, 48), device="cuda")
    with pytest.raises(ttt.TTTError, match="not supported"):
        ttt.ttt_linear_fwd(q, q, q, torch.zeros((1, 48, 48), device="cuda"), 0.1, 4)


# ------------------------------------------------------------------ per-token rates
# token t learns at eta * eta_tok[t]; every kernel path (generic, matrix-core linear and
# delta rule, causal and non-causal MLP) against the oracle with the same factors

def _with_rates(w, seed, lo=0.0, hi=1.0):
    inp = make_inputs(w)
    inp["eta_tok"] = make_token_rates(w, seed, lo, hi)
    return inp


@pytest.mark.parametrize("chunk,causal", [(5, True), (16, False), (1, True)])
def test_token_rates_linear_fp32(chunk, causal):
    w = workload(0).replace(B=2, H=3, T=77, d=32, chunk=chunk, causal=causal, init="normal",
                            eta=0.4, seed=80 + chunk)
    _check("linear", w, _with_rates(w, 1))


@pytest.mark.parametrize("T", [16, 200, 333])
def test_token_rates_linear_bf16_d64_chunk16(T):
    w = workload(1).replace(B=2, H=3, T=T, init="normal", eta=0.5, seed=90 + T)
    _check("linear", w, _with_rates(w, 2))


def test_token_rates_linear_config_full_size():
    w = workload(1)
    _check("linear", w, _with_rates(w, 3), full=True)


@pytest.mark.parametrize("d,io", [(16, "f32"), (64, "bf16")])
def test_token_rates_delta(d, io):
    w = workload(2).replace(B=2, H=2, T=150, d=d, io=io, init="normal", seed=100 + d)
    _check("delta", w, _with_rates(w, 4))


def test_token_rates_delta_config_full_size():
    w = workload(2)
    _check("delta", w, _with_rates(w, 5), full=True)


@pytest.mark.parametrize("chunk,causal", [(4, True), (37, False)])
def test_token_rates_mlp_fp32(chunk, causal):
    w = workload(3).replace(B=1, H=2, T=37, d=16, h=24, io="f32", chunk=chunk, causal=causal,
                            seed=110 + chunk)
    _check("mlp", w, _with_rates(w, 6))


def test_token_rates_mlp_bf16_h256():
    w = workload(3).replace(B=2, H=2, T=70, seed=120)
    _check("mlp", w, _with_rates(w, 7))


def test_token_rates_mlp_vision():
    w = workload(4).replace(B=2, H=3, seed=130)
    _check("mlp", w, _with_rates(w, 8))


# ------------------------------------------------------------------ dot-product loss
# loss -v^T f(k): the error term of every gradient is -v (blog page, TTT / 如何理解; ViT3
# news page, section 2); every kernel path against the oracle with loss="dot"

@pytest.mark.parametrize("chunk,causal", [(5, True), (16, False)])
def test_dot_loss_linear_fp32(chunk, causal):
    w = workload(0).replace(B=2, H=2, T=61, d=32, chunk=chunk, causal=causal, init="normal",
                            eta=0.1, seed=140 + chunk)
    _check("linear", w, make_inputs(w), loss="dot")


@pytest.mark.parametrize("T,rates", [(200, False), (333, True)])
def test_dot_loss_linear_bf16_d64_chunk16(T, rates):
    w = workload(1).replace(B=2, H=3, T=T, init="normal", eta=0.05, seed=150 + T)
    inp = _with_rates(w, 9) if rates else make_inputs(w)
    _check("linear", w, inp, loss="dot")


@pytest.mark.parametrize("chunk,causal", [(4, True), (37, False)])
def test_dot_loss_mlp_fp32(chunk, causal):
    w = workload(3).replace(B=1, H=2, T=37, d=16, h=24, io="f32", chunk=chunk, causal=causal,
                            seed=160 + chunk)
    _check("mlp", w, make_inputs(w), loss="dot")


@pytest.mark.parametrize("rates", [False, True])
def test_dot_loss_mlp_bf16_h256(rates):
    w = workload(3).replace(B=2, H=2, T=70, eta=0.05, seed=170)
    _check("mlp", w, _with_rates(w, 10) if rates else make_inputs(w), loss="dot")


@pytest.mark.parametrize("rates", [False, True])
def test_dot_loss_mlp_vision(rates):
    w = workload(4).replace(B=2, H=3, eta=0.1, seed=180)
    _check("mlp", w, _with_rates(w, 11) if rates else make_inputs(w), loss="dot")


def test_dot_loss_mlp_vision_config_full_size():
    w = workload(4).replace(eta=0.1)
    _check("mlp", w, make_inputs(w), loss="dot", full=True)


# ------------------------------------------------------------------ mini-batches and epochs
# Non-causal layer trained over consecutive mini-batches (N/2, N/3, N/4 of the N pairs) for
# several epochs before the queries read it (ViT3 news page, observation 2).  The rates keep
# the recurrence bounded: at the vision workload's eta = 1 several steps diverge in float64.

@pytest.mark.parametrize("chunk,epochs", [(196, 2), (98, 1), (66, 1), (49, 2), (49, 4), (16, 1),
                                          (5, 2), (300, 3)])
def test_epochs_mlp_vision(chunk, epochs):
    w = workload(4).replace(B=2, H=3, chunk=chunk, unit_keys=True, eta=0.1, seed=200 + chunk)
    _check("mlp", w, make_inputs(w), epochs=epochs)


@pytest.mark.parametrize("loss,rates", [("mse", True), ("dot", False), ("dot", True)])
def test_epochs_mlp_vision_loss_and_rates(loss, rates):
    w = workload(4).replace(B=2, H=3, chunk=66, unit_keys=True, eta=0.1, seed=210)
    _check("mlp", w, _with_rates(w, 12) if rates else make_inputs(w), loss=loss, epochs=2)


def test_epochs_mlp_vision_config_full_size():
    w = workload(4).replace(chunk=49, eta=0.01)
    _check("mlp", w, make_inputs(w), epochs=2, full=True)


@pytest.mark.parametrize("chunk,epochs", [(10, 3), (37, 2)])
def test_epochs_mlp_fp32(chunk, epochs):
    w = workload(3).replace(B=2, H=2, T=37, d=16, h=32, chunk=chunk, causal=False, io="f32",
                            eta=0.05, seed=220 + chunk)
    _check("mlp", w, make_inputs(w), epochs=epochs)


@pytest.mark.parametrize("d,chunk,epochs,io", [(16, 16, 2, "f32"), (32, 77, 3, "f32"),
                                               (64, 49, 2, "bf16")])
def test_epochs_linear(d, chunk, epochs, io):
    w = workload(0).replace(B=2, H=3, T=196, d=d, chunk=chunk, causal=False, init="normal",
                            eta=0.1, io=io, seed=230 + d)
    _check("linear", w, make_inputs(w), epochs=epochs)


# ------------------------------------------------------------------ non-causal TTT-Linear
# The linear layer trained first on all pairs, then read by every query (ViT3 news page,
# section 1; wmrh.cn summary, section 2.1.1), at the vision shape on the matrix cores
# (d = 64, bf16): one full-batch step, or mini-batches and epochs.

def _linear_nc(**kw):
    base = dict(kind="linear", h=0, chunk=196, causal=False, name="linear_nc_N196")
    base.update(kw)
    return workload(4).replace(**base)


@pytest.mark.parametrize("T", [1, 15, 16, 17, 100, 196, 333])
def test_linear_nc_full_batch(T):
    w = _linear_nc(B=2, H=3, T=T, chunk=T, seed=300 + T)
    _check("linear", w, make_inputs(w))


@pytest.mark.parametrize("chunk,epochs", [(98, 1), (66, 2), (49, 3), (16, 1), (5, 2), (300, 2)])
def test_linear_nc_minibatches_and_epochs(chunk, epochs):
    w = _linear_nc(B=2, H=3, chunk=chunk, unit_keys=True, eta=0.1, seed=310 + chunk)
    _check("linear", w, make_inputs(w), epochs=epochs)


@pytest.mark.parametrize("loss,rates,chunk,epochs", [("mse", True, 196, 1), ("dot", False, 196, 1),
                                                     ("dot", True, 49, 2), ("mse", True, 66, 2)])
def test_linear_nc_loss_and_rates(loss, rates, chunk, epochs):
    w = _linear_nc(B=2, H=3, chunk=chunk, unit_keys=True, eta=0.1, seed=320 + chunk)
    _check("linear", w, _with_rates(w, 13) if rates else make_inputs(w), loss=loss, epochs=epochs)


def test_linear_nc_per_batch_state_and_chain_count():
    w = _linear_nc(B=13, H=1, T=150, chunk=150, seed=330)
    inp = make_inputs(w)
    rng = np.random.default_rng(1)
    inp["w0"] = (0.05 * rng.standard_normal((13, 1, 64, 64))).astype(np.float32)
    _check("linear", w, inp)


def test_linear_nc_vision_shape_full_size():
    w = _linear_nc()
    _check("linear", w, make_inputs(w), full=True)


def test_linear_nc_vision_shape_dot_loss_full_size():
    # with the dot-product loss one full-batch step from W0 is W0 + eta V^T K: non-causal
    # linear attention (the blog page, section TTT / 如何理解)
    w = _linear_nc()
    _check("linear", w, make_inputs(w), loss="dot", full=True)


# ------------------------------------------------------------------ the paper's inner models
# f(x) = x + LN(f_res(x)), f_res = W x or W2 GELU(W1 x) (wmrh.cn summary, section 2.2.1):
# ttt_linear_ln_fwd / ttt_mlp_ln_fwd against the oracle's ln / act="gelu"

def _with_ln(w, seed, rates_seed=None):
    inp = make_inputs(w)
    inp["ln_w"], inp["ln_b"] = make_ln_params(w, seed)
    if rates_seed is not None:
        inp["eta_tok"] = make_token_rates(w, rates_seed)
    return inp


@pytest.mark.parametrize("d", [16, 32, 64])
@pytest.mark.parametrize("chunk,causal", [(1, True), (5, True), (16, True), (77, False)])
def test_paper_linear_fp32(d, chunk, causal):
    w = workload(0).replace(B=2, H=3, T=77, d=d, chunk=chunk, causal=causal, init="normal",
                            eta=0.2, seed=300 + d + chunk)
    _check("linear", w, _with_ln(w, 1))


@pytest.mark.parametrize("T,rates,loss", [(16, False, "mse"), (200, False, "mse"),
                                          (333, True, "mse"), (200, False, "dot")])
def test_paper_linear_bf16_d64_chunk16(T, rates, loss):
    w = workload(1).replace(B=2, H=3, T=T, seed=310 + T)
    _check("linear", w, _with_ln(w, 2, 13 if rates else None), loss=loss)


def test_paper_linear_bf16_per_batch_state():
    # a [B, H, d, d] initial state (w0_batch_stride = H d^2) and a ragged last chunk
    w = workload(1).replace(B=3, H=2, T=77, seed=315)
    inp = _with_ln(w, 9)
    rng = np.random.default_rng(316)
    inp["w0"] = (0.05 * rng.standard_normal((w.B, w.H, w.d, w.d))).astype(np.float32)
    _check("linear", w, inp)


def test_paper_linear_noncausal_epochs():
    w = workload(1).replace(B=2, H=3, T=196, chunk=49, causal=False, seed=320)
    _check("linear", w, _with_ln(w, 3), epochs=2)


def test_paper_linear_config_full_size():
    w = workload(1)
    _check("linear", w, _with_ln(w, 4), full=True)


@pytest.mark.parametrize("chunk,causal", [(1, True), (4, True), (16, True), (37, False),
                                          (10, False)])
def test_paper_mlp_fp32(chunk, causal):
    w = workload(3).replace(B=2, H=2, T=37, d=16, h=64, chunk=chunk, causal=causal, io="f32",
                            seed=330 + chunk)
    inp = _with_ln(w, 5)
    if chunk == 1:
        # With N(0, 0.02^2) initial weights the spread of the LN input (about 1.5e-3) is of
        # the order of sqrt(eps), and one-token steps then amplify a 1e-7 perturbation of the
        # inputs about 300x in the float64 oracle itself; ten times larger initial weights
        # keep the same path well conditioned (chunks 4 and 16 agree to ~2e-7 either way).
        inp["w1"], inp["w2"] = inp["w1"] * 10, inp["w2"] * 10
    _check("mlp", w, inp)


@pytest.mark.parametrize("T,rates,loss", [(100, False, "mse"), (70, True, "mse"),
                                          (70, False, "dot")])
def test_paper_mlp_bf16_h256(T, rates, loss):
    # the paper's TTT-MLP: hidden 4 d = 256, GELU, LN + residual, mini-batch 16
    w = workload(3).replace(B=2, H=2, T=T, seed=340 + T)
    _check("mlp", w, _with_ln(w, 6, 14 if rates else None), loss=loss)


def test_paper_mlp_vision_noncausal_epochs():
    w = workload(4).replace(B=2, H=3, chunk=98, unit_keys=True, eta=0.1, seed=350)
    _check("mlp", w, _with_ln(w, 7), epochs=2)


def test_paper_mlp_config_full_size():
    w = workload(3)
    _check("mlp", w, _with_ln(w, 8), full=True)


# ------------------------------------------------------------------ backward pass
# ttt_linear_bwd against the oracle's vector-Jacobian product (autograd of the primal
# recurrence in float64, pinned to finite differences)

def _check_bwd(w, inp, with_dw, sel=None, seed=0, rates=False, loss="mse", full=False):
    import torch
    import test_sequence_layers_amd as ttt
    from oracle import ttt_oracle as O
    from tests.oracle_pool import run_chains
    _note(f"[parity] linear_bwd B={w.B} H={w.H} T={w.T} d={w.d} chunk={w.chunk} io={w.io} "
          f"dw_out={with_dw} rates={rates} loss={loss} seed={w.seed} full={full}")
    rng = np.random.default_rng(20_000 + seed)
    dz = rng.standard_normal((w.B, w.H, w.T, w.d)).astype(np.float32)
    if w.io == "bf16":
        dz = to_np(torch.from_numpy(dz).to(torch.bfloat16))
    dw = rng.standard_normal((w.B, w.H, w.d, w.d)).astype(np.float32) if with_dw else None
    dev = to_device(inp, w.io)
    dt = dev["q"].dtype
    dzd = torch.from_numpy(dz).to("cuda").to(dt).contiguous()
    dwd = torch.from_numpy(dw).to("cuda").contiguous() if with_dw else None
    et = make_token_rates(w, seed) if rates else None
    etd = torch.from_numpy(et).to("cuda").contiguous() if rates else None
    out = ttt.ttt_linear_bwd(dev["q"], dev["k"], dev["v"], dev["w0"], w.eta, w.chunk, dzd, dwd,
                             eta_tok=etd, loss=loss)
    torch.cuda.synchronize()
    got = [to_np(t) for t in out]
    del out, dev
    q, k, v, dzz = inp["q"], inp["k"], inp["v"], dz
    w0 = np.broadcast_to(inp["w0"], (w.B, w.H, w.d, w.d)) if inp["w0"].ndim == 3 else inp["w0"]
    dww = dw
    if full:
        _note("[parity]   oracle over every sequence (worker processes)")
        ref = run_chains("ttt_linear_vjp", w.B, w.H, (q, k, v, w0, w.eta, w.chunk, dzz, dww),
                         {"eta_tok": et, "loss": loss}, {})
    else:
        if sel is not None:
            bs = [b for b, _ in sel]
            hs = [h for _, h in sel]
            q, k, v, dzz, w0 = (q[bs, hs][None], k[bs, hs][None], v[bs, hs][None],
                                dzz[bs, hs][None], w0[bs, hs][None])
            dww = dw[bs, hs][None] if dw is not None else None
            et = et[bs, hs][None] if rates else None
            got = [g[bs, hs][None] for g in got]
        ref = O.ttt_linear_vjp(q, k, v, w0, w.eta, w.chunk, dzz, dww, eta_tok=et, loss=loss)
    tol = tol_for(w.io)
    for name, g, r in zip(("dq", "dk", "dv", "dw0", "deta_tok"), got, ref):
        if name == "deta_tok":  # [.., T]: one row per sequence
            g, r = g[..., None, :], r[..., None, :]
        check_close(name, g, r, tol, _note)


@pytest.mark.parametrize("d,chunk,with_dw", [(16, 4, True), (16, 1, False), (32, 16, True)])
def test_linear_bwd_token_rates_fp32(d, chunk, with_dw):
    # per-token rate factors in [0, 1) and their gradient (the learnable rate)
    w = workload(0).replace(B=2, H=2, T=37, d=d, chunk=chunk, init="normal", eta=0.3,
                            seed=230 + d + chunk)
    _check_bwd(w, make_inputs(w), with_dw, seed=d + chunk, rates=True)


@pytest.mark.parametrize("T,with_dw", [(77, True), (200, False)])
def test_linear_bwd_token_rates_bf16_d64(T, with_dw):
    w = workload(1).replace(B=2, H=3, T=T, seed=240 + T)
    _check_bwd(w, make_inputs(w), with_dw, seed=T, rates=True)


@pytest.mark.parametrize("d,chunk,rates", [(16, 4, False), (32, 16, True)])
def test_linear_bwd_dot_loss_fp32(d, chunk, rates):
    # the negative dot-product loss (R = -V): linear attention with a trained update
    w = workload(0).replace(B=2, H=2, T=37, d=d, chunk=chunk, init="normal", eta=0.3,
                            seed=260 + d + chunk)
    _check_bwd(w, make_inputs(w), True, seed=d + chunk, rates=rates, loss="dot")


@pytest.mark.parametrize("T,with_dw,rates", [(77, True, False), (200, False, True)])
def test_linear_bwd_dot_loss_bf16_d64(T, with_dw, rates):
    w = workload(1).replace(B=2, H=3, T=T, seed=270 + T)
    _check_bwd(w, make_inputs(w), with_dw, seed=T, rates=rates, loss="dot")


def test_linear_bwd_token_rates_full_size():
    w = workload(1)
    _check_bwd(w, make_inputs(w), True, seed=5, rates=True, full=True)


@pytest.mark.parametrize("d,chunk,with_dw", [(16, 4, True), (16, 1, False), (32, 16, True),
                                             (16, 37, False)])
def test_linear_bwd_fp32(d, chunk, with_dw):
    w = workload(0).replace(B=2, H=2, T=37 if chunk != 37 else 13, d=d, chunk=chunk,
                            init="normal", eta=0.3, seed=190 + d + chunk)
    _check_bwd(w, make_inputs(w), with_dw, seed=d + chunk)


@pytest.mark.parametrize("T", [16, 200])
def test_linear_bwd_bf16_d64_chunk16(T):
    w = workload(1).replace(B=2, H=3, T=T, seed=200 + T)
    _check_bwd(w, make_inputs(w), True, seed=T)


@pytest.mark.parametrize("T,with_dw,per_batch,eta", [(77, False, False, 0.125), (33, True, True, 0.125),
                                                     (1000, False, False, 0.5)])
def test_linear_bwd_bf16_matrix_core_cases(T, with_dw, per_batch, eta):
    # the matrix-core backward without an upstream state gradient, with a [B, H, d, d] initial
    # state, ragged last chunks and a larger rate
    w = workload(1).replace(B=2, H=3, T=T, eta=eta, seed=210 + T)
    inp = make_inputs(w)
    if per_batch:
        rng = np.random.default_rng(211)
        inp["w0"] = (0.05 * rng.standard_normal((w.B, w.H, w.d, w.d))).astype(np.float32)
    _check_bwd(w, inp, with_dw, seed=T + 1)


def test_linear_bwd_bf16_w0_offset_by_one_float():
    # w0 starting 4 bytes past a 16-byte boundary: the matrix-core backward reads w0 rows with
    # 16-byte loads, so this call must take the vector-ALU path (and still match the oracle)
    import torch
    import test_sequence_layers_amd as ttt
    from oracle import ttt_oracle as O
    w = workload(1).replace(B=2, H=3, T=45, seed=290)
    inp = make_inputs(w)
    dev = to_device(inp, w.io)
    buf = torch.zeros(1 + w.H * w.d * w.d, dtype=torch.float32, device="cuda")
    w0 = buf[1:].view(w.H, w.d, w.d)
    w0.copy_(dev["w0"])
    assert w0.data_ptr() % 16 == 4
    rng = np.random.default_rng(291)
    dz = to_np(torch.from_numpy(rng.standard_normal((w.B, w.H, w.T, w.d)).astype(np.float32))
               .to(torch.bfloat16))
    dzd = torch.from_numpy(dz).to("cuda").to(torch.bfloat16).contiguous()
    out = ttt.ttt_linear_bwd(dev["q"], dev["k"], dev["v"], w0, w.eta, w.chunk, dzd)
    torch.cuda.synchronize()
    got = [to_np(t) for t in out]
    ref = O.ttt_linear_vjp(inp["q"], inp["k"], inp["v"], inp["w0"], w.eta, w.chunk, dz)
    for name, g, r in zip(("dq", "dk", "dv", "dw0"), got, ref):
        check_close(name, g, r, BF16_TOL, _note)


def test_linear_bwd_config_full_size():
    w = workload(1)
    _check_bwd(w, make_inputs(w), True, seed=1, full=True)


def _check_mlp_bwd(w, inp, with_dw, sel=None, seed=0, loss="mse", full=False, rates=False):
    import torch
    import test_sequence_layers_amd as ttt
    from oracle import ttt_oracle as O
    from tests.oracle_pool import run_chains
    _note(f"[parity] mlp_bwd B={w.B} H={w.H} T={w.T} d={w.d} h={w.h} chunk={w.chunk} io={w.io} "
          f"dw_out={with_dw} loss={loss} rates={rates} seed={w.seed} full={full}")
    rng = np.random.default_rng(30_000 + seed)
    dz = rng.standard_normal((w.B, w.H, w.T, w.d)).astype(np.float32)
    if w.io == "bf16":
        dz = to_np(torch.from_numpy(dz).to(torch.bfloat16))
    dw1 = rng.standard_normal((w.B, w.H, w.h, w.d)).astype(np.float32) if with_dw else None
    dw2 = rng.standard_normal((w.B, w.H, w.d, w.h)).astype(np.float32) if with_dw else None
    dev = to_device(inp, w.io)
    dzd = torch.from_numpy(dz).to("cuda").to(dev["q"].dtype).contiguous()
    dd1 = torch.from_numpy(dw1).to("cuda").contiguous() if with_dw else None
    dd2 = torch.from_numpy(dw2).to("cuda").contiguous() if with_dw else None
    et = make_token_rates(w, seed) if rates else None
    etd = torch.from_numpy(et).to("cuda").contiguous() if rates else None
    out = ttt.ttt_mlp_bwd(dev["q"], dev["k"], dev["v"], dev["w1"], dev["w2"], w.eta, w.chunk, dzd,
                          dd1, dd2, eta_tok=etd, loss=loss)
    torch.cuda.synchronize()
    got = [to_np(t) for t in out]
    del out, dev
    bc = lambda x, sh: np.broadcast_to(x, (w.B, w.H) + sh) if x.ndim == 3 else x
    q, k, v, dzz = inp["q"], inp["k"], inp["v"], dz
    w1, w2 = bc(inp["w1"], (w.h, w.d)), bc(inp["w2"], (w.d, w.h))
    if rates:  # the general VJP (per-token rates), returning (..., deta_tok, None, None)
        dst = (dw1, dw2) if with_dw else None
        args = ("mlp", q, k, v, (w1, w2), w.eta, w.chunk, dzz, dst)
        kw = dict(eta_tok=et, loss=loss)
        if full:
            _note("[parity]   oracle over every sequence (worker processes)")
            ref = run_chains("ttt_layer_vjp", w.B, w.H, args, kw, {})
        else:
            ref = O.ttt_layer_vjp(*args, **kw)
        for name, g, r in zip(("dq", "dk", "dv", "dw1", "dw2", "deta_tok"), got, ref):
            if name == "deta_tok":
                g, r = g[..., None, :], r[..., None, :]
            check_close(name, g, r, tol_for(w.io), _note)
        return
    if full:
        _note("[parity]   oracle over every sequence (worker processes)")
        ref = run_chains("ttt_mlp_vjp", w.B, w.H, (q, k, v, w1, w2, w.eta, w.chunk, dzz, dw1, dw2),
                         {"loss": loss}, {})
    else:
        if sel is not None:
            bs = [b for b, _ in sel]
            hs = [h for _, h in sel]
            pick = lambda x: x[bs, hs][None] if x is not None else None
            q, k, v, dzz, w1, w2, dw1, dw2 = map(pick, (q, k, v, dzz, w1, w2, dw1, dw2))
            got = [g[bs, hs][None] for g in got]
        ref = O.ttt_mlp_vjp(q, k, v, w1, w2, w.eta, w.chunk, dzz, dw1, dw2, loss=loss)
    tol = tol_for(w.io)
    for name, g, r in zip(("dq", "dk", "dv", "dw1", "dw2"), got, ref):
        check_close(name, g, r, tol, _note)


@pytest.mark.parametrize("d,h,chunk,with_dw", [(16, 32, 4, True), (16, 32, 1, False),
                                               (32, 64, 16, True), (16, 24, 5, False),
                                               (64, 64, 16, False)])
def test_mlp_bwd_fp32(d, h, chunk, with_dw):
    w = workload(3).replace(B=2, H=2, T=37, d=d, h=h, chunk=chunk, io="f32", eta=0.2,
                            seed=500 + d + h + chunk)
    _check_mlp_bwd(w, make_inputs(w), with_dw, seed=d + chunk)


@pytest.mark.parametrize("T,with_dw", [(16, True), (70, False)])
def test_mlp_bwd_bf16_h256(T, with_dw):
    w = workload(3).replace(B=2, H=2, T=T, seed=520 + T)
    _check_mlp_bwd(w, make_inputs(w), with_dw, seed=T)


@pytest.mark.parametrize("T,with_dw,per_batch,eta", [(77, True, True, 0.1), (33, False, False, 0.3),
                                                     (200, True, False, 0.1)])
def test_mlp_bwd_bf16_matrix_core_cases(T, with_dw, per_batch, eta):
    # the matrix-core backward (and its history-mode forward) with [B, H, h, d] / [B, H, d, h]
    # initial states, no upstream state gradient, ragged last chunks and a larger rate
    w = workload(3).replace(B=2, H=2, T=T, eta=eta, seed=540 + T)
    inp = make_inputs(w)
    if per_batch:
        rng = np.random.default_rng(541)
        inp["w1"] = (0.02 * rng.standard_normal((w.B, w.H, w.h, w.d))).astype(np.float32)
        inp["w2"] = (0.02 * rng.standard_normal((w.B, w.H, w.d, w.h))).astype(np.float32)
    _check_mlp_bwd(w, inp, with_dw, seed=T + 3)


@pytest.mark.parametrize("d,h,chunk,with_dw", [(16, 32, 4, True), (32, 64, 16, False),
                                               (16, 24, 5, True)])
def test_mlp_bwd_dot_loss_fp32(d, h, chunk, with_dw):
    # negative dot-product loss: error term -v (vector-ALU backward)
    w = workload(3).replace(B=2, H=2, T=37, d=d, h=h, chunk=chunk, io="f32", eta=0.2,
                            seed=560 + d + h + chunk)
    _check_mlp_bwd(w, make_inputs(w), with_dw, seed=d + chunk + 7, loss="dot")


@pytest.mark.parametrize("T,with_dw", [(16, True), (45, False)])
def test_mlp_bwd_dot_loss_bf16_h256(T, with_dw):
    # the causal MLP workload's shape (d 64, hidden 256, chunk 16) in bf16 with the dot loss
    w = workload(3).replace(B=2, H=2, T=T, seed=580 + T)
    _check_mlp_bwd(w, make_inputs(w), with_dw, seed=T + 9, loss="dot")


def test_mlp_bwd_config_full_size():
    w = workload(3)
    _check_mlp_bwd(w, make_inputs(w), True, seed=2, full=True)


def test_mlp_bwd_empty_sequence_copies_state_gradients():
    import torch
    import test_sequence_layers_amd as ttt
    q = torch.zeros((2, 3, 0, 16), device="cuda")
    w1, w2 = torch.randn((3, 8, 16), device="cuda"), torch.randn((3, 16, 8), device="cuda")
    d1, d2 = torch.randn((2, 3, 8, 16), device="cuda"), torch.randn((2, 3, 16, 8), device="cuda")
    *_, g1, g2 = ttt.ttt_mlp_bwd(q, q, q, w1, w2, 0.1, 16, q, d1, d2)
    torch.cuda.synchronize()
    assert torch.equal(g1, d1) and torch.equal(g2, d2)


def test_linear_bwd_empty_sequence_copies_dw_out():
    import torch
    import test_sequence_layers_amd as ttt
    q = torch.zeros((2, 3, 0, 16), device="cuda")
    w0 = torch.randn((3, 16, 16), device="cuda")
    dw = torch.randn((2, 3, 16, 16), device="cuda")
    dq, dk, dv, dw0 = ttt.ttt_linear_bwd(q, q, q, w0, 0.1, 16, q, dw)
    torch.cuda.synchronize()
    assert torch.equal(dw0, dw)
    _, _, _, dw0 = ttt.ttt_linear_bwd(q, q, q, w0, 0.1, 16, q)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dw0).item() == 0


# ------------------------------------------------------------------ backward of the non-causal layers
# ttt_linear_nc_bwd / ttt_mlp_nc_bwd against the oracle's ttt_layer_vjp (torch.autograd
# through the recurrence, pinned by central differences of the numpy forward): one
# full-batch step at the vision shape, and mini-batches, epochs, rates and both losses.

def _check_nc_bwd(kind, w, inp, with_dw, seed=0, rates=False, loss="mse", epochs=1, full=False):
    import torch
    import test_sequence_layers_amd as ttt
    from oracle import ttt_oracle as O
    from tests.oracle_pool import run_chains
    _note(f"[parity] {kind}_nc_bwd B={w.B} H={w.H} T={w.T} d={w.d} h={w.h} chunk={w.chunk} "
          f"epochs={epochs} io={w.io} dw_out={with_dw} rates={rates} loss={loss} seed={w.seed} "
          f"full={full}")
    rng = np.random.default_rng(40_000 + seed)
    dz = rng.standard_normal((w.B, w.H, w.T, w.d)).astype(np.float32)
    if w.io == "bf16":
        dz = to_np(torch.from_numpy(dz).to(torch.bfloat16))
    names = ("w0",) if kind == "linear" else ("w1", "w2")
    shapes = {"w0": (w.d, w.d), "w1": (w.h, w.d), "w2": (w.d, w.h)}
    dst = tuple(rng.standard_normal((w.B, w.H) + shapes[n]).astype(np.float32) for n in names) \
        if with_dw else None
    dev = to_device(inp, w.io)
    dzd = torch.from_numpy(dz).to("cuda").to(dev["q"].dtype).contiguous()
    dsd = tuple(torch.from_numpy(x).to("cuda").contiguous() for x in dst) if with_dw else None
    et = make_token_rates(w, seed) if rates else None
    etd = torch.from_numpy(et).to("cuda").contiguous() if rates else None
    if kind == "linear":
        out = ttt.ttt_linear_nc_bwd(dev["q"], dev["k"], dev["v"], dev["w0"], w.eta, w.chunk, dzd,
                                    dsd[0] if with_dw else None, epochs=epochs, eta_tok=etd,
                                    loss=loss)
    else:
        out = ttt.ttt_mlp_nc_bwd(dev["q"], dev["k"], dev["v"], dev["w1"], dev["w2"], w.eta, w.chunk,
                                 dzd, *(dsd if with_dw else (None, None)), epochs=epochs,
                                 eta_tok=etd, loss=loss)
    torch.cuda.synchronize()
    got = [to_np(t) for t in out]
    del out, dev
    state = tuple(inp[n] for n in names)
    kw = dict(causal=False, epochs=epochs, eta_tok=et, loss=loss)
    args = (kind, inp["q"], inp["k"], inp["v"], state, w.eta, w.chunk, dz, dst)
    if full:
        _note("[parity]   oracle over every sequence (worker processes)")
        ref = run_chains("ttt_layer_vjp", w.B, w.H, args, kw, {4: 3})
    else:
        ref = O.ttt_layer_vjp(*args, **kw)
    ref = [r for r in ref if r is not None]
    tol = tol_for(w.io)
    labels = ("dq", "dk", "dv") + tuple("d" + n for n in names) + (("deta_tok",) if rates else ())
    assert len(got) == len(ref) == len(labels)
    for name, g, r in zip(labels, got, ref):
        if name == "deta_tok":  # [.., T]: one row per sequence
            g, r = g[..., None, :], r[..., None, :]
        check_close(name, g, r, tol, _note)


@pytest.mark.parametrize("d,T,chunk,epochs,with_dw,rates,loss", [
    (16, 30, 4, 2, True, False, "mse"), (16, 40, 40, 1, False, True, "mse"),
    (32, 33, 7, 3, True, True, "dot"), (64, 50, 16, 1, False, False, "mse")])
def test_linear_nc_bwd_fp32(d, T, chunk, epochs, with_dw, rates, loss):
    w = workload(0).replace(B=2, H=3, T=T, d=d, chunk=chunk, causal=False, init="normal",
                            eta=0.1, seed=400 + d + chunk)
    _check_nc_bwd("linear", w, make_inputs(w), with_dw, seed=d, rates=rates, loss=loss,
                  epochs=epochs)


@pytest.mark.parametrize("d,h,T,chunk,epochs,with_dw,rates,loss", [
    (16, 32, 30, 5, 2, True, True, "mse"), (16, 24, 37, 37, 1, False, False, "dot"),
    (32, 64, 41, 9, 2, True, False, "mse"), (16, 256, 20, 8, 1, True, True, "mse"),
    (64, 128, 20, 20, 1, False, False, "mse")])
def test_mlp_nc_bwd_fp32(d, h, T, chunk, epochs, with_dw, rates, loss):
    w = workload(3).replace(B=2, H=2, T=T, d=d, h=h, chunk=chunk, causal=False, io="f32",
                            eta=0.05, seed=410 + h + chunk)
    _check_nc_bwd("mlp", w, make_inputs(w), with_dw, seed=h, rates=rates, loss=loss,
                  epochs=epochs)


@pytest.mark.parametrize("kind,rates,loss,epochs,chunk", [
    ("linear", False, "mse", 1, 196), ("linear", True, "dot", 2, 66),
    ("mlp", False, "mse", 1, 196), ("mlp", True, "mse", 2, 49), ("mlp", False, "dot", 1, 196)])
def test_nc_bwd_bf16_vision_shape(kind, rates, loss, epochs, chunk):
    w = workload(4).replace(B=2, H=3, chunk=chunk, seed=420 + chunk)
    if kind == "linear":
        w = w.replace(kind="linear", h=0)
    if epochs > 1:
        w = w.replace(unit_keys=True, eta=0.1)
    _check_nc_bwd(kind, w, make_inputs(w), with_dw=True, seed=7, rates=rates, loss=loss,
                  epochs=epochs)


@pytest.mark.parametrize("T,rates,loss,with_dw", [
    (1, False, "mse", True), (16, True, "mse", False), (37, False, "dot", True),
    (100, True, "dot", True), (196, True, "mse", True), (256, False, "mse", False)])
def test_mlp_nc_bwd_matrix_core_cases(T, rates, loss, with_dw):
    # one full-batch step at d = hidden = 64, bf16: the matrix-core backward for 16 <= T <= 256
    # (T = 1 checks that shorter sequences go to the fp32 kernel)
    w = workload(4).replace(B=2, H=3, T=T, chunk=T, seed=440 + T)
    _check_nc_bwd("mlp", w, make_inputs(w), with_dw, seed=T, rates=rates, loss=loss)


@pytest.mark.parametrize("T,rates,loss,with_dw", [
    (1, True, "mse", True), (16, False, "dot", True), (45, True, "mse", False),
    (128, True, "dot", False), (256, False, "mse", True)])
def test_linear_nc_bwd_matrix_core_cases(T, rates, loss, with_dw):
    # one full-batch step at d = 64, bf16: the matrix-core backward for 16 <= T <= 256
    # (T = 1 checks that shorter sequences go to the fp32 kernel)
    w = workload(4).replace(kind="linear", h=0, B=2, H=3, T=T, chunk=T, seed=460 + T)
    _check_nc_bwd("linear", w, make_inputs(w), with_dw, seed=T, rates=rates, loss=loss)


def test_linear_nc_bwd_matrix_core_per_batch_state():
    w = workload(4).replace(kind="linear", h=0, B=3, H=2, T=70, chunk=70, seed=470)
    inp = make_inputs(w)
    inp["w0"] = (0.05 * np.random.default_rng(8).standard_normal((3, 2, 64, 64))).astype(np.float32)
    _check_nc_bwd("linear", w, inp, with_dw=True, rates=True)


def test_mlp_nc_bwd_matrix_core_per_batch_states():
    w = workload(4).replace(B=3, H=2, T=70, chunk=70, seed=450)
    inp = make_inputs(w)
    rng = np.random.default_rng(6)
    inp["w1"] = (0.05 * rng.standard_normal((3, 2, 64, 64))).astype(np.float32)
    inp["w2"] = (0.05 * rng.standard_normal((3, 2, 64, 64))).astype(np.float32)
    _check_nc_bwd("mlp", w, inp, with_dw=True, rates=True)


def test_nc_bwd_per_batch_states():
    w = workload(4).replace(B=3, H=2, T=50, chunk=20, unit_keys=True, eta=0.1, seed=430)
    inp = make_inputs(w)
    rng = np.random.default_rng(5)
    inp["w1"] = (0.05 * rng.standard_normal((3, 2, 64, 64))).astype(np.float32)
    inp["w2"] = (0.05 * rng.standard_normal((3, 2, 64, 64))).astype(np.float32)
    _check_nc_bwd("mlp", w, inp, with_dw=False, epochs=2)


def test_mlp_nc_bwd_vision_config_full_size():
    w = workload(4)
    _check_nc_bwd("mlp", w, make_inputs(w), with_dw=False, full=True)


def test_linear_nc_bwd_vision_shape_full_size():
    w = workload(4).replace(kind="linear", h=0)
    _check_nc_bwd("linear", w, make_inputs(w), with_dw=False, full=True)


def test_nc_bwd_empty_sequence_copies_state_gradients():
    import torch
    import test_sequence_layers_amd as ttt
    z = torch.zeros((2, 3, 0, 16), dtype=torch.float32, device="cuda")
    w1 = torch.zeros((3, 24, 16), device="cuda")
    w2 = torch.zeros((3, 16, 24), device="cuda")
    d1 = torch.randn((2, 3, 24, 16), device="cuda")
    d2 = torch.randn((2, 3, 16, 24), device="cuda")
    out = ttt.ttt_mlp_nc_bwd(z, z, z, w1, w2, 0.1, 4, z, d1, d2, epochs=2)
    torch.cuda.synchronize()
    assert torch.equal(out[3], d1) and torch.equal(out[4], d2)


# ------------------------------------------------------------------ MLP backward with per-token rates
# ttt_mlp_bwd with eta_tok (the learnable rate of the wmrh.cn summary, section 2.2.3) and its
# gradient deta_tok, against the oracle's ttt_layer_vjp (pinned by central differences).

@pytest.mark.parametrize("d,h,chunk,with_dw,loss", [(16, 32, 4, True, "mse"), (32, 64, 16, False, "mse"),
                                                    (16, 24, 5, True, "dot"), (16, 32, 1, False, "mse")])
def test_mlp_bwd_token_rates_fp32(d, h, chunk, with_dw, loss):
    w = workload(3).replace(B=2, H=2, T=37, d=d, h=h, chunk=chunk, io="f32", eta=0.1,
                            seed=500 + h + chunk)
    _check_mlp_bwd(w, make_inputs(w), with_dw, seed=chunk, loss=loss, rates=True)


@pytest.mark.parametrize("T,with_dw", [(16, True), (70, False)])
def test_mlp_bwd_token_rates_bf16_h256(T, with_dw):
    w = workload(3).replace(B=1, H=2, T=T, seed=510 + T)
    _check_mlp_bwd(w, make_inputs(w), with_dw, seed=T, rates=True)


def test_mlp_bwd_token_rates_config_full_size():
    w = workload(3)
    _check_mlp_bwd(w, make_inputs(w), False, seed=3, rates=True, full=True)


# ------------------------------------------------------------------ backward of the paper's TTT-Linear
# ttt_linear_ln_bwd (f(x) = x + LN(W x); wmrh.cn summary, section 2.2.1) against the oracle's
# ttt_layer_vjp with ln, including the layer norm's gain and bias gradients.

def _check_ln_bwd(w, inp, with_dw, seed=0, rates=False, loss="mse", full=False, w_scale=None):
    import torch
    import test_sequence_layers_amd as ttt
    from oracle import ttt_oracle as O
    from tests.oracle_pool import run_chains
    from tests.parity_util import LN_EPS
    _note(f"[parity] linear_ln_bwd B={w.B} H={w.H} T={w.T} d={w.d} chunk={w.chunk} io={w.io} "
          f"dw_out={with_dw} rates={rates} loss={loss} seed={w.seed} full={full}")
    if w_scale is not None:
        inp["w0"] = (inp["w0"] * w_scale).astype(np.float32)
    rng = np.random.default_rng(50_000 + seed)
    dz = rng.standard_normal((w.B, w.H, w.T, w.d)).astype(np.float32)
    if w.io == "bf16":
        dz = to_np(torch.from_numpy(dz).to(torch.bfloat16))
    dw = rng.standard_normal((w.B, w.H, w.d, w.d)).astype(np.float32) if with_dw else None
    lw, lb = make_ln_params(w, seed)
    et = make_token_rates(w, seed) if rates else None
    dev = to_device(inp, w.io)
    out = ttt.ttt_linear_ln_bwd(
        dev["q"], dev["k"], dev["v"], dev["w0"], torch.from_numpy(lw).cuda(),
        torch.from_numpy(lb).cuda(), w.eta, w.chunk,
        torch.from_numpy(dz).to("cuda").to(dev["q"].dtype).contiguous(),
        torch.from_numpy(dw).cuda() if with_dw else None, ln_eps=LN_EPS,
        eta_tok=torch.from_numpy(et).cuda() if rates else None, loss=loss)
    torch.cuda.synchronize()
    got = [to_np(t) for t in out]
    del out, dev
    args = ("linear", inp["q"], inp["k"], inp["v"], (inp["w0"],), w.eta, w.chunk, dz,
            (dw,) if with_dw else None)
    kw = dict(eta_tok=et, loss=loss, ln=(lw, lb, LN_EPS))
    if full:
        _note("[parity]   oracle over every sequence (worker processes)")
        ref = run_chains("ttt_layer_vjp", w.B, w.H, args, kw, {4: 3, "ln": 2})
    else:
        ref = O.ttt_layer_vjp(*args, **kw)
    dq, dk, dv, dw0, de, dg, db = ref
    refs = [dq, dk, dv, dw0, dg, db] + ([de] if rates else [])
    tol = tol_for(w.io)
    for name, g, r in zip(("dq", "dk", "dv", "dw0", "dln_weight", "dln_bias", "deta_tok"), got, refs):
        if name in ("deta_tok", "dln_weight", "dln_bias"):  # one row per sequence
            g, r = g[..., None, :], r[..., None, :]
        check_close(name, g, r, tol, _note)


@pytest.mark.parametrize("d,chunk,with_dw,rates,loss", [
    (16, 4, True, True, "mse"), (32, 16, False, False, "dot"), (64, 5, True, False, "mse"),
    (16, 1, False, True, "mse")])
def test_linear_ln_bwd_fp32(d, chunk, with_dw, rates, loss):
    w = workload(0).replace(B=2, H=3, T=37, d=d, chunk=chunk, init="normal", eta=0.2,
                            seed=600 + d + chunk)
    # chunk 1: larger initial weights, so that the first tokens' layer-norm inputs are not of
    # the order of sqrt(eps) (where the recurrence itself is ill-conditioned)
    _check_ln_bwd(w, make_inputs(w), with_dw, seed=d, rates=rates, loss=loss,
                  w_scale=10.0 if chunk == 1 else None)


@pytest.mark.parametrize("T,with_dw,rates,loss", [(16, True, False, "mse"), (77, False, True, "mse"),
                                                  (200, True, False, "dot")])
def test_linear_ln_bwd_bf16_d64_chunk16(T, with_dw, rates, loss):
    w = workload(1).replace(B=2, H=3, T=T, seed=610 + T)
    _check_ln_bwd(w, make_inputs(w), with_dw, seed=T, rates=rates, loss=loss)


def test_linear_ln_bwd_config_full_size():
    w = workload(1)
    _check_ln_bwd(w, make_inputs(w), False, seed=1, full=True)


def test_linear_ln_bwd_empty_sequence():
    import torch
    import test_sequence_layers_amd as ttt
    z = torch.zeros((2, 3, 0, 16), device="cuda")
    w0 = torch.zeros((3, 16, 16), device="cuda")
    lw, lb = torch.ones((3, 16), device="cuda"), torch.zeros((3, 16), device="cuda")
    d0 = torch.randn((2, 3, 16, 16), device="cuda")
    out = ttt.ttt_linear_ln_bwd(z, z, z, w0, lw, lb, 0.1, 4, z, d0)
    torch.cuda.synchronize()
    assert torch.equal(out[3], d0) and not out[4].any() and not out[5].any()


# ------------------------------------------------------------------ backward of the paper's TTT-MLP
# ttt_mlp_ln_bwd (f(x) = x + LN(W2 GELU(W1 x)); wmrh.cn summary, section 2.2.1) against the
# oracle's ttt_layer_vjp with act="gelu" and ln.

def _check_mlp_ln_bwd(w, inp, with_dw, seed=0, rates=False, loss="mse", full=False, w_scale=None):
    import torch
    import test_sequence_layers_amd as ttt
    from oracle import ttt_oracle as O
    from tests.oracle_pool import run_chains
    from tests.parity_util import LN_EPS
    _note(f"[parity] mlp_ln_bwd B={w.B} H={w.H} T={w.T} d={w.d} h={w.h} chunk={w.chunk} "
          f"io={w.io} dw_out={with_dw} rates={rates} loss={loss} seed={w.seed} full={full}")
    if w_scale is not None:
        inp["w1"] = (inp["w1"] * w_scale).astype(np.float32)
        inp["w2"] = (inp["w2"] * w_scale).astype(np.float32)
    rng = np.random.default_rng(60_000 + seed)
    dz = rng.standard_normal((w.B, w.H, w.T, w.d)).astype(np.float32)
    if w.io == "bf16":
        dz = to_np(torch.from_numpy(dz).to(torch.bfloat16))
    dw1 = rng.standard_normal((w.B, w.H, w.h, w.d)).astype(np.float32) if with_dw else None
    dw2 = rng.standard_normal((w.B, w.H, w.d, w.h)).astype(np.float32) if with_dw else None
    lw, lb = make_ln_params(w, seed)
    et = make_token_rates(w, seed) if rates else None
    dev = to_device(inp, w.io)
    out = ttt.ttt_mlp_ln_bwd(
        dev["q"], dev["k"], dev["v"], dev["w1"], dev["w2"], torch.from_numpy(lw).cuda(),
        torch.from_numpy(lb).cuda(), w.eta, w.chunk,
        torch.from_numpy(dz).to("cuda").to(dev["q"].dtype).contiguous(),
        torch.from_numpy(dw1).cuda() if with_dw else None,
        torch.from_numpy(dw2).cuda() if with_dw else None, ln_eps=LN_EPS,
        eta_tok=torch.from_numpy(et).cuda() if rates else None, loss=loss)
    torch.cuda.synchronize()
    got = [to_np(t) for t in out]
    del out, dev
    args = ("mlp", inp["q"], inp["k"], inp["v"], (inp["w1"], inp["w2"]), w.eta, w.chunk, dz,
            (dw1, dw2) if with_dw else None)
    kw = dict(eta_tok=et, loss=loss, act="gelu", ln=(lw, lb, LN_EPS))
    if full:
        _note("[parity]   oracle over every sequence (worker processes)")
        ref = run_chains("ttt_layer_vjp", w.B, w.H, args, kw, {4: 3, "ln": 2})
    else:
        ref = O.ttt_layer_vjp(*args, **kw)
    dq, dk, dv, d1, d2, de, dg, db = ref
    refs = [dq, dk, dv, d1, d2, dg, db] + ([de] if rates else [])
    tol = tol_for(w.io)
    names = ("dq", "dk", "dv", "dw1", "dw2", "dln_weight", "dln_bias", "deta_tok")
    for name, g, r in zip(names, got, refs):
        if name in ("deta_tok", "dln_weight", "dln_bias"):  # one row per sequence
            g, r = g[..., None, :], r[..., None, :]
        check_close(name, g, r, tol, _note)


@pytest.mark.parametrize("d,h,chunk,with_dw,rates,loss", [
    (16, 32, 4, True, True, "mse"), (32, 64, 16, False, False, "dot"), (16, 24, 5, True, False, "mse"),
    (16, 32, 1, False, True, "mse")])
def test_mlp_ln_bwd_fp32(d, h, chunk, with_dw, rates, loss):
    w = workload(3).replace(B=2, H=2, T=37, d=d, h=h, chunk=chunk, io="f32", eta=0.1,
                            seed=700 + h + chunk)
    _check_mlp_ln_bwd(w, make_inputs(w), with_dw, seed=h, rates=rates, loss=loss,
                      w_scale=10.0 if chunk == 1 else None)


@pytest.mark.parametrize("T,with_dw,rates,loss", [(16, True, False, "mse"), (70, False, True, "mse"),
                                                  (45, True, False, "dot")])
def test_mlp_ln_bwd_bf16_h256(T, with_dw, rates, loss):
    w = workload(3).replace(B=1, H=2, T=T, seed=710 + T)
    _check_mlp_ln_bwd(w, make_inputs(w), with_dw, seed=T, rates=rates, loss=loss)


def test_mlp_ln_bwd_config_full_size():
    w = workload(3)
    _check_mlp_ln_bwd(w, make_inputs(w), False, seed=2, full=True)


# ------------------------------------------------------------------ backward of the delta rule
# ttt_linear_bwd with chunk 1 runs the exact chunked form 16 tokens at a time; the oracle's
# ttt_linear_vjp walks the tokens one by one.

@pytest.mark.parametrize("d,T,with_dw,rates,loss", [
    (16, 37, True, False, "mse"), (32, 50, False, True, "mse"), (64, 33, True, True, "mse"),
    (16, 21, True, False, "dot"), (64, 1, True, True, "mse")])
def test_delta_bwd_fp32(d, T, with_dw, rates, loss):
    w = workload(2).replace(B=2, H=3, T=T, d=d, io="f32", eta=0.3, seed=800 + d + T)
    _check_bwd(w, make_inputs(w), with_dw, seed=d, rates=rates, loss=loss)


@pytest.mark.parametrize("T,rates", [(200, False), (333, True)])
def test_delta_bwd_bf16_d64(T, rates):
    w = workload(2).replace(B=2, H=3, T=T, seed=810 + T)
    _check_bwd(w, make_inputs(w), True, seed=T, rates=rates)


def test_delta_bwd_config_full_size():
    w = workload(2)
    _check_bwd(w, make_inputs(w), False, seed=2, full=True)
