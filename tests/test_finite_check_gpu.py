"""The library's finite check of the outputs (a debugging switch of the C ABI) on the GPU.

With the check on, a call whose outputs are finite returns them unchanged (bit for bit the
outputs of the same call with the check off), and a call that produces a NaN or an infinity
fails with TTT_E_NONFINITE naming the output.  The non-finite values are forced from the
host through the caller's data (a NaN in v, an infinity in dz, a rate so large that the
inner updates overflow); nothing here faults the GPU.
"""
import math

import pytest

import test_sequence_layers_amd as ttt

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _tokens(B, H, T, d, dtype, seed):
    torch = _torch()
    g = torch.Generator().manual_seed(seed)
    q, k, v = (torch.randn(B, H, T, d, generator=g) for _ in range(3))
    k = k / k.norm(dim=-1, keepdim=True)
    return [x.to(dtype).cuda().contiguous() for x in (q, k, v)]


@pytest.fixture
def check_on():
    prev = ttt.set_check_finite(True)
    yield
    ttt.set_check_finite(prev)


@pytest.mark.parametrize("dtype_name,d,chunk", [("bf16", 64, 16), ("fp32", 32, 5)])
def test_finite_outputs_pass_unchanged(check_on, dtype_name, d, chunk):
    torch = _torch()
    dtype = torch.bfloat16 if dtype_name == "bf16" else torch.float32
    print(f"[finite] linear fwd {dtype_name} d={d} chunk={chunk}", flush=True)
    q, k, v = _tokens(2, 3, 45, d, dtype, 1)
    w0 = (0.02 * torch.randn(3, d, d, generator=torch.Generator().manual_seed(2))).cuda()
    z_on, w_on = ttt.ttt_linear_fwd(q, k, v, w0, 0.1, chunk, return_state=True)
    ttt.set_check_finite(False)
    z_off, w_off = ttt.ttt_linear_fwd(q, k, v, w0, 0.1, chunk, return_state=True)
    torch.cuda.synchronize()
    assert torch.equal(z_on, z_off) and torch.equal(w_on, w_off)


def test_nan_in_values_is_reported_in_z(check_on):
    torch = _torch()
    print("[finite] linear fwd bf16 d=64 with a NaN in v", flush=True)
    q, k, v = _tokens(2, 3, 64, 64, torch.bfloat16, 3)
    v[1, 2, 20, 7] = float("nan")
    w0 = (0.02 * torch.randn(3, 64, 64, generator=torch.Generator().manual_seed(4))).cuda()
    with pytest.raises(ttt.TTTError) as ei:
        ttt.ttt_linear_fwd(q, k, v, w0, 0.1, 16, return_state=True)
    assert ei.value.code == ttt.TTT_E_NONFINITE
    assert "ttt_linear_fwd" in str(ei.value) and "non-finite values in z" in str(ei.value)
    # with the check off the same call succeeds and the NaN is there
    ttt.set_check_finite(False)
    z, w_out = ttt.ttt_linear_fwd(q, k, v, w0, 0.1, 16, return_state=True)
    torch.cuda.synchronize()
    assert torch.isnan(z[1, 2, 20:].float()).any()
    assert torch.isfinite(z[0].float()).all() and torch.isfinite(z[1, :2].float()).all()
    assert not torch.isfinite(w_out[1, 2]).all()


def test_divergent_mlp_is_reported(check_on):
    torch = _torch()
    print("[finite] mlp fwd bf16 d=64 h=256 at eta=1e30", flush=True)
    q, k, v = _tokens(1, 2, 64, 64, torch.bfloat16, 5)
    gen = torch.Generator().manual_seed(6)
    w1 = (0.1 * torch.randn(2, 256, 64, generator=gen)).cuda()
    w2 = (0.1 * torch.randn(2, 64, 256, generator=gen)).cuda()
    with pytest.raises(ttt.TTTError) as ei:
        ttt.ttt_mlp_fwd(q, k, v, w1, w2, 1e30, 16)
    assert ei.value.code == ttt.TTT_E_NONFINITE and "in z" in str(ei.value)
    # a moderate rate stays finite and passes
    z = ttt.ttt_mlp_fwd(q, k, v, w1, w2, 0.1, 16)
    assert torch.isfinite(z.float()).all()


def test_infinite_upstream_gradient_is_reported_in_dq(check_on):
    torch = _torch()
    print("[finite] linear bwd bf16 d=64 with an infinity in dz", flush=True)
    q, k, v = _tokens(1, 2, 48, 64, torch.bfloat16, 7)
    w0 = (0.02 * torch.randn(2, 64, 64, generator=torch.Generator().manual_seed(8))).cuda()
    dz = torch.randn(1, 2, 48, 64, generator=torch.Generator().manual_seed(9)).to(torch.bfloat16).cuda()
    dq, dk, dv, dw0 = ttt.ttt_linear_bwd(q, k, v, w0, 0.1, 16, dz)
    assert all(bool(torch.isfinite(t.float()).all()) for t in (dq, dk, dv, dw0))
    dz[0, 1, 30, 5] = math.inf
    with pytest.raises(ttt.TTTError) as ei:
        ttt.ttt_linear_bwd(q, k, v, w0, 0.1, 16, dz)
    assert ei.value.code == ttt.TTT_E_NONFINITE and "non-finite values in dq" in str(ei.value)


def test_two_workgroup_mlp_under_the_check(check_on):
    # ttt_mlp_fwd_ws with the check on: finite outputs unchanged; a NaN in v reported in z
    torch = _torch()
    print("[finite] mlp fwd on two workgroups, bf16 d=64 h=256", flush=True)
    q, k, v = _tokens(2, 3, 70, 64, torch.bfloat16, 7)
    g = torch.Generator().manual_seed(8)
    w1 = (0.02 * torch.randn(3, 256, 64, generator=g)).cuda()
    w2 = (0.02 * torch.randn(3, 64, 256, generator=g)).cuda()
    z_on, w1_on, w2_on = ttt.ttt_mlp_fwd_ws(q, k, v, w1, w2, 0.1, 16, return_state=True)
    ttt.set_check_finite(False)
    z_off, w1_off, w2_off = ttt.ttt_mlp_fwd_ws(q, k, v, w1, w2, 0.1, 16, return_state=True)
    torch.cuda.synchronize()
    assert torch.equal(z_on, z_off) and torch.equal(w1_on, w1_off) and torch.equal(w2_on, w2_off)
    ttt.set_check_finite(True)
    v[0, 1, 33, 5] = float("nan")
    with pytest.raises(ttt.TTTError) as ei:
        ttt.ttt_mlp_fwd_ws(q, k, v, w1, w2, 0.1, 16)
    assert ei.value.code == ttt.TTT_E_NONFINITE
    assert "ttt_mlp_fwd_ws" in str(ei.value) and "z" in str(ei.value)
