"""CPU checks behind the readings of the measured workloads (the oracle alone, no GPU).

The causal MLP workload (d = 64, hidden 256, chunk 16, eta = 0.1) is stated with raw keys;
the float64 recurrence itself overflows with them, which is why the workload uses unit
keys.  These checks keep that evidence in the repository: with raw N(0, 1) keys the state
norm explodes and the outputs leave the finite range within 256 tokens, while with unit keys
the states stay bounded over the whole sequence and the oracle's own float32 and float64
runs agree far below the bf16 tolerance.
"""
import numpy as np
import pytest

from oracle import ttt_oracle as O
from test_sequence_layers_amd.workloads import make_inputs, workload


def _mlp(unit_keys, T, H=2, dtype=np.float64):
    w = workload(3).replace(unit_keys=unit_keys)
    inp = make_inputs(w)
    q, k, v = (inp[x][:1, :H, :T] for x in ("q", "k", "v"))
    with np.errstate(over="ignore", invalid="ignore"):
        return O.ttt_mlp(q, k, v, inp["w1"][:H], inp["w2"][:H], w.eta, w.chunk, True, dtype=dtype)


@pytest.mark.slow
def test_raw_keys_make_the_causal_mlp_recurrence_overflow():
    z, w1, w2 = _mlp(unit_keys=False, T=256)
    norm = np.linalg.norm(w1[0, :, :, :].reshape(2, -1), axis=-1)
    # inf / NaN in the outputs, or a state that has grown by many orders of magnitude
    assert (not np.isfinite(z).all()) or (not np.isfinite(norm).all()) or norm.max() > 1e6


@pytest.mark.slow
def test_unit_keys_keep_the_causal_mlp_recurrence_bounded():
    z64, a1, a2 = _mlp(unit_keys=True, T=2048)
    assert np.isfinite(z64).all()
    n1 = np.linalg.norm(a1.reshape(2, -1), axis=-1)
    n2 = np.linalg.norm(a2.reshape(2, -1), axis=-1)
    assert n1.max() < 50 and n2.max() < 50          # from about 2.6 at the start
    z32, _, _ = _mlp(unit_keys=True, T=2048, dtype=np.float32)
    rel = np.linalg.norm(z32 - z64) / np.linalg.norm(z64)
    assert rel < 1e-5                                  # oracle noise far below the 2e-2 bound
