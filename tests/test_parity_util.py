"""CPU checks of the parity machinery itself: the per-slab measures and the parallel oracle."""
import numpy as np
import pytest

from oracle import ttt_oracle as O
from tests.oracle_pool import run_chains
from tests.parity_util import BF16_TOL, check_close, run_oracle_all, slab_errors
from test_sequence_layers_amd.workloads import make_inputs, make_ln_params, make_token_rates, workload


def test_element_wise_measure_catches_one_wrong_element():
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((2, 3, 2048, 64))
    got = ref.copy()
    got[1, 2, 700, 5] += 0.25 * np.abs(ref[1, 2]).max()
    (f, frel, _), (e, erel, ei) = slab_errors(got, ref)
    # one wrong element hides inside the Frobenius measure of a 2048 x 64 slab ...
    assert f < 5e-3
    # ... but not inside the element-wise one, which also names the slab
    assert e == pytest.approx(0.25) and ei == 5 and erel[1, 2] == e
    with pytest.raises(AssertionError):
        check_close("z", got, ref, BF16_TOL, note=lambda m: None)
    check_close("z", ref, ref, BF16_TOL, note=lambda m: None)


def test_zero_reference_slab_uses_absolute_error():
    ref = np.zeros((1, 2, 4, 4))
    got = ref.copy()
    got[0, 1, 0, 0] = 3e-3
    (f, _, _), (e, _, _) = slab_errors(got, ref)
    assert f == pytest.approx(3e-3) and e == pytest.approx(3e-3)


@pytest.mark.parametrize("kind,idx", [("linear", 1), ("delta", 2), ("mlp", 3), ("mlp", 4)])
def test_parallel_oracle_equals_direct_call(kind, idx):
    w = workload(idx).replace(B=3, H=2, T=37 if idx != 4 else 20)
    inp = make_inputs(w)
    inp["eta_tok"] = make_token_rates(w, 1)
    if kind != "delta":
        inp["ln_w"], inp["ln_b"] = make_ln_params(w, 2)
    got = run_oracle_all(kind, inp, w.eta, w.chunk, w.causal)
    et = inp["eta_tok"]
    if kind == "linear":
        ref = O.ttt_linear(inp["q"], inp["k"], inp["v"], inp["w0"], w.eta, w.chunk, w.causal,
                           eta_tok=et, ln=(inp["ln_w"], inp["ln_b"], 1e-6))
    elif kind == "delta":
        ref = O.delta_rule(inp["q"], inp["k"], inp["v"], inp["w0"], w.eta, eta_tok=et)
    else:
        ref = O.ttt_mlp(inp["q"], inp["k"], inp["v"], inp["w1"], inp["w2"], w.eta, w.chunk,
                        w.causal, eta_tok=et, ln=(inp["ln_w"], inp["ln_b"], 1e-6), act="gelu")
    assert len(got) == len(ref)
    for g, r in zip(got, ref):
        np.testing.assert_array_equal(g, r)


def test_parallel_vjp_per_batch_state():
    w = workload(1).replace(B=2, H=3, T=20, d=16)
    inp = make_inputs(w)
    rng = np.random.default_rng(3)
    w0 = rng.standard_normal((2, 3, 16, 16)) * 0.05
    dz = rng.standard_normal((2, 3, 20, 16))
    got = run_chains("ttt_linear_vjp", 2, 3, (inp["q"], inp["k"], inp["v"], w0, 0.1, 4, dz), {}, {})
    ref = O.ttt_linear_vjp(inp["q"], inp["k"], inp["v"], w0, 0.1, 4, dz)
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r, rtol=0, atol=1e-12)
