"""The allocation-free linear backward (ttt_linear_bwd_noalloc) against ttt_linear_bwd.

Both entry points run the same kernels; the allocation-free one keeps the chunk-start state
history in the library's fixed scratch array instead of a stream-ordered workspace.  Two
calls in a row, the second with a smaller input, on the matrix-core and on the vector-ALU
path, each compared with the allocating entry point on the same inputs.
"""
import sys

import numpy as np
import pytest

from tests.parity_util import BF16_TOL, FP32_TOL, check_close, make_inputs, make_token_rates, workload

pytestmark = pytest.mark.gpu


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _case(w, seed, rates, with_dw):
    import torch
    import test_sequence_layers_amd as ttt
    _note(f"[no_alloc] B={w.B} H={w.H} T={w.T} d={w.d} chunk={w.chunk} io={w.io} rates={rates} "
          f"dw_out={with_dw}")
    inp = make_inputs(w)
    dt = torch.bfloat16 if w.io == "bf16" else torch.float32
    dev = {x: torch.from_numpy(inp[x]).to("cuda").to(dt).contiguous() for x in ("q", "k", "v")}
    w0 = torch.from_numpy(inp["w0"]).to("cuda").contiguous()
    rng = np.random.default_rng(seed)
    dz = torch.from_numpy(rng.standard_normal((w.B, w.H, w.T, w.d)).astype(np.float32)).to("cuda").to(dt)
    dw = (torch.from_numpy(rng.standard_normal((w.B, w.H, w.d, w.d)).astype(np.float32)).to("cuda")
          if with_dw else None)
    et = torch.from_numpy(make_token_rates(w, seed)).to("cuda") if rates else None
    ref = ttt.ttt_linear_bwd(dev["q"], dev["k"], dev["v"], w0, w.eta, w.chunk, dz, dw, eta_tok=et)
    got = ttt.ttt_linear_bwd_noalloc(dev["q"], dev["k"], dev["v"], w0, w.eta, w.chunk, dz, dw,
                                     eta_tok=et)
    torch.cuda.synchronize()
    tol = BF16_TOL if w.io == "bf16" else FP32_TOL
    for name, g, r in zip(("dq", "dk", "dv", "dw0", "deta_tok"), got, ref):
        g = g.float().cpu().numpy()
        r = r.float().cpu().numpy()
        if name == "deta_tok":
            g, r = g[..., None, :], r[..., None, :]
        check_close(name, g, r, tol, _note)
        # the same kernels on the same inputs: the same bits
        assert np.array_equal(g, r), name


def test_no_alloc_matrix_core_path_two_calls():
    w = workload(1).replace(B=3, H=4, T=300, init="normal", seed=600)
    _case(w, 601, rates=True, with_dw=True)
    _case(w.replace(B=1, H=2, T=77, seed=602), 603, rates=False, with_dw=False)


def test_no_alloc_vector_alu_path_two_calls():
    w = workload(0).replace(B=2, H=3, T=90, d=32, chunk=4, init="normal", eta=0.2, seed=610)
    _case(w, 611, rates=False, with_dw=True)
    _case(w.replace(B=1, H=2, T=21, seed=612), 613, rates=True, with_dw=False)


def test_no_alloc_delta_rule_two_calls():
    # chunk 1: the chunked delta-rule backward keeps its states and 16 x 16 matrices there
    w = workload(2).replace(B=2, H=3, T=90, d=32, io="f32", eta=0.3, seed=620)
    _case(w, 621, rates=True, with_dw=True)
    _case(w.replace(B=1, H=2, T=37, io="bf16", d=64, seed=622), 623, rates=False, with_dw=False)


def test_no_alloc_rejects_a_history_beyond_the_scratch_array():
    import torch
    import test_sequence_layers_amd as ttt
    # B*H*ceil(T/16)*8 KB = 80 MiB > 64 MiB: rejected before any work is enqueued
    q = torch.zeros((5, 16, 2048, 64), dtype=torch.bfloat16, device="cuda")
    w0 = torch.zeros((16, 64, 64), device="cuda")
    with pytest.raises(ttt.TTTError, match="scratch"):
        ttt.ttt_linear_bwd_noalloc(q, q, q, w0, 0.1, 16, q)
