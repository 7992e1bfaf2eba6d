"""Host-side checks of the C ABI (CPU only: no call here reaches a HIP runtime function).

The library must load, export every function include/ttt.h declares, and reject invalid
arguments with the documented status and message before touching the GPU.
"""
import ctypes
import os
import re

import pytest

import test_sequence_layers_amd as ttt
from test_sequence_layers_amd import _binding

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "ttt.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return ttt.load_library()


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("ttt_linear_fwd", "ttt_mlp_fwd", "delta_rule_fwd", "ttt_linear_bwd", "ttt_mlp_bwd",
              "ttt_linear_ln_fwd", "ttt_mlp_ln_fwd", "ttt_last_error", "ttt_abi_version",
              "ttt_linear_nc_bwd", "ttt_mlp_nc_bwd", "ttt_linear_bwd_noalloc",
              "ttt_set_check_finite", "ttt_get_check_finite", "ttt_mlp_fwd_workspace_size",
              "ttt_mlp_fwd_ws", "ttt_mlp_ln_fwd_ws", "ttt_set_split_debug"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert name in _binding.SIGNATURES, f"binding lacks {name}"


def test_abi_version(lib):
    assert lib.ttt_abi_version() == 14


FAKE = 0x1000  # never dereferenced: validation fails before any HIP call


def _linear(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, w0=FAKE, stride=0, z=FAKE, w_out=None, B=1, H=1, T=16,
             d=16, chunk=16, causal=1, eta=0.1, eta_tok=None, loss=0, epochs=1, io=0)
    a.update(kw)
    return lib.ttt_linear_fwd(a["q"], a["k"], a["v"], a["w0"], a["stride"], a["z"], a["w_out"],
                              a["B"], a["H"], a["T"], a["d"], a["chunk"], a["causal"],
                              a["eta"], a["eta_tok"], a["loss"], a["epochs"], a["io"], None)


def _mlp(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, w1=FAKE, w2=FAKE, stride=0, z=FAKE, B=1, H=1, T=16, d=16,
             dh=32, chunk=16, causal=1, eta=0.1, eta_tok=None, loss=0, epochs=1, io=0)
    a.update(kw)
    return lib.ttt_mlp_fwd(a["q"], a["k"], a["v"], a["w1"], a["w2"], a["stride"], a["z"], None,
                           None, a["B"], a["H"], a["T"], a["d"], a["dh"], a["chunk"],
                           a["causal"], a["eta"], a["eta_tok"], a["loss"], a["epochs"], a["io"],
                           None)


def _delta(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, w0=FAKE, stride=0, z=FAKE, B=1, H=1, T=16, d=16, eta=0.1,
             eta_tok=None, io=0)
    a.update(kw)
    return lib.delta_rule_fwd(a["q"], a["k"], a["v"], a["w0"], a["stride"], a["z"], None,
                              a["B"], a["H"], a["T"], a["d"], a["eta"], a["eta_tok"], a["io"],
                              None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(q=None), ttt.TTT_E_INVALID, "non-null"),
    (dict(z=None), ttt.TTT_E_INVALID, "non-null"),
    (dict(w0=None), ttt.TTT_E_INVALID, "w0"),
    (dict(B=0), ttt.TTT_E_INVALID, "positive"),
    (dict(H=-1), ttt.TTT_E_INVALID, "positive"),
    (dict(T=-5), ttt.TTT_E_INVALID, "positive"),
    (dict(d=0), ttt.TTT_E_INVALID, "positive"),
    (dict(chunk=0), ttt.TTT_E_INVALID, "chunk"),
    (dict(causal=2), ttt.TTT_E_INVALID, "causal"),
    (dict(eta=float("nan")), ttt.TTT_E_INVALID, "finite"),
    (dict(eta=float("inf")), ttt.TTT_E_INVALID, "finite"),
    (dict(io=7), ttt.TTT_E_INVALID, "dtype"),
    (dict(stride=-1), ttt.TTT_E_INVALID, "stride"),
    (dict(B=1 << 30, H=1 << 30, T=1 << 30, d=64), ttt.TTT_E_INVALID, "overflow"),
    (dict(d=48), ttt.TTT_E_UNSUPPORTED, "d=48"),
    (dict(d=128), ttt.TTT_E_UNSUPPORTED, "d=128"),
    (dict(eta_tok=FAKE + 2), ttt.TTT_E_INVALID, "eta_tok"),
    (dict(loss=2), ttt.TTT_E_INVALID, "loss"),
    (dict(epochs=0), ttt.TTT_E_INVALID, "epochs"),
    (dict(epochs=2), ttt.TTT_E_INVALID, "causal = 0"),
    (dict(epochs=-1, causal=0), ttt.TTT_E_INVALID, "epochs"),
])
def test_linear_rejects(lib, kw, code, msg):
    assert _linear(lib, **kw) == code
    assert msg in ttt.last_error()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(w1=None), ttt.TTT_E_INVALID, "w1"),
    (dict(w2=None), ttt.TTT_E_INVALID, "w2"),
    (dict(dh=0), ttt.TTT_E_INVALID, "dh"),
    (dict(dh=1024), ttt.TTT_E_UNSUPPORTED, "dh=1024"),
    (dict(d=100), ttt.TTT_E_UNSUPPORTED, "d=100"),
    (dict(chunk=-3), ttt.TTT_E_INVALID, "chunk"),
    (dict(io=2), ttt.TTT_E_INVALID, "dtype"),
    (dict(v=None), ttt.TTT_E_INVALID, "non-null"),
    (dict(eta_tok=FAKE + 1), ttt.TTT_E_INVALID, "eta_tok"),
    (dict(loss=-1), ttt.TTT_E_INVALID, "loss"),
    (dict(epochs=0, causal=0), ttt.TTT_E_INVALID, "epochs"),
    (dict(epochs=3), ttt.TTT_E_INVALID, "causal = 0"),
])
def test_mlp_rejects(lib, kw, code, msg):
    assert _mlp(lib, **kw) == code
    assert msg in ttt.last_error()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(k=None), ttt.TTT_E_INVALID, "non-null"),
    (dict(w0=None), ttt.TTT_E_INVALID, "w0"),
    (dict(d=8), ttt.TTT_E_UNSUPPORTED, "d=8"),
    (dict(eta=float("-inf")), ttt.TTT_E_INVALID, "finite"),
    (dict(eta_tok=FAKE + 3), ttt.TTT_E_INVALID, "eta_tok"),
])
def test_delta_rejects(lib, kw, code, msg):
    assert _delta(lib, **kw) == code
    assert msg in ttt.last_error()


def _bwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, w0=FAKE, stride=0, dz=FAKE, dw_out=None, dq=FAKE, dk=FAKE,
             dv=FAKE, dw0=FAKE, B=1, H=1, T=16, d=16, chunk=16, eta=0.1, eta_tok=None,
             deta_tok=None, loss=0, io=0)
    a.update(kw)
    return lib.ttt_linear_bwd(a["q"], a["k"], a["v"], a["w0"], a["stride"], a["dz"], a["dw_out"],
                              a["dq"], a["dk"], a["dv"], a["dw0"], a["B"], a["H"], a["T"],
                              a["d"], a["chunk"], a["eta"], a["eta_tok"], a["deta_tok"],
                              a["loss"], a["io"], None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(dz=None), ttt.TTT_E_INVALID, "non-null"),
    (dict(dq=None), ttt.TTT_E_INVALID, "dq"),
    (dict(dw0=None), ttt.TTT_E_INVALID, "dw0"),
    (dict(w0=None), ttt.TTT_E_INVALID, "w0"),
    (dict(chunk=0), ttt.TTT_E_INVALID, "chunk"),
    (dict(eta=float("nan")), ttt.TTT_E_INVALID, "finite"),
    (dict(io=3), ttt.TTT_E_INVALID, "dtype"),
    (dict(d=48), ttt.TTT_E_UNSUPPORTED, "d=48"),
    (dict(chunk=32, T=64), ttt.TTT_E_UNSUPPORTED, "16 tokens"),
    (dict(deta_tok=FAKE), ttt.TTT_E_INVALID, "needs eta_tok"),
    (dict(eta_tok=FAKE, deta_tok=FAKE + 2), ttt.TTT_E_INVALID, "deta_tok"),
    (dict(eta_tok=FAKE + 1), ttt.TTT_E_INVALID, "eta_tok"),
    (dict(loss=2), ttt.TTT_E_INVALID, "loss"),
])
def test_linear_bwd_rejects(lib, kw, code, msg):
    assert _bwd(lib, **kw) == code
    assert msg in ttt.last_error()


def _linear_ln(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, w0=FAKE, stride=0, ln_w=FAKE, ln_b=FAKE, eps=1e-6, z=FAKE,
             w_out=None, B=1, H=1, T=16, d=16, chunk=16, causal=1, eta=0.1, eta_tok=None, loss=0,
             epochs=1, io=0)
    a.update(kw)
    return lib.ttt_linear_ln_fwd(a["q"], a["k"], a["v"], a["w0"], a["stride"], a["ln_w"],
                                 a["ln_b"], a["eps"], a["z"], a["w_out"], a["B"], a["H"], a["T"],
                                 a["d"], a["chunk"], a["causal"], a["eta"], a["eta_tok"],
                                 a["loss"], a["epochs"], a["io"], None)


def _mlp_ln(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, w1=FAKE, w2=FAKE, stride=0, ln_w=FAKE, ln_b=FAKE, eps=1e-6,
             z=FAKE, B=1, H=1, T=16, d=16, dh=64, chunk=16, causal=1, eta=0.1, eta_tok=None,
             loss=0, epochs=1, io=0)
    a.update(kw)
    return lib.ttt_mlp_ln_fwd(a["q"], a["k"], a["v"], a["w1"], a["w2"], a["stride"], a["ln_w"],
                              a["ln_b"], a["eps"], a["z"], None, None, a["B"], a["H"], a["T"],
                              a["d"], a["dh"], a["chunk"], a["causal"], a["eta"], a["eta_tok"],
                              a["loss"], a["epochs"], a["io"], None)


@pytest.mark.parametrize("fn", [_linear_ln, _mlp_ln])
@pytest.mark.parametrize("kw,code,msg", [
    (dict(ln_w=None), ttt.TTT_E_INVALID, "ln_weight"),
    (dict(ln_b=None), ttt.TTT_E_INVALID, "ln_bias"),
    (dict(eps=0.0), ttt.TTT_E_INVALID, "ln_eps"),
    (dict(eps=-1e-5), ttt.TTT_E_INVALID, "ln_eps"),
    (dict(eps=float("nan")), ttt.TTT_E_INVALID, "ln_eps"),
    (dict(q=None), ttt.TTT_E_INVALID, "non-null"),
    (dict(d=48), ttt.TTT_E_UNSUPPORTED, "d=48"),
    (dict(epochs=2), ttt.TTT_E_INVALID, "causal = 0"),
    (dict(loss=5), ttt.TTT_E_INVALID, "loss"),
])
def test_paper_models_reject(lib, fn, kw, code, msg):
    assert fn(lib, **kw) == code
    assert msg in ttt.last_error()
    assert ("ttt_linear_ln_fwd" if fn is _linear_ln else "ttt_mlp_ln_fwd") in ttt.last_error()


def _mlp_bwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, w1=FAKE, w2=FAKE, stride=0, dz=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
             dw1=FAKE, dw2=FAKE, B=1, H=1, T=16, d=16, dh=32, chunk=16, eta=0.1, loss=0, io=0)
    a.update(kw)
    return lib.ttt_mlp_bwd(a["q"], a["k"], a["v"], a["w1"], a["w2"], a["stride"], a["dz"], None,
                           None, a["dq"], a["dk"], a["dv"], a["dw1"], a["dw2"], a["B"], a["H"],
                           a["T"], a["d"], a["dh"], a["chunk"], a["eta"], a.get("eta_tok"),
                           a.get("deta"), a["loss"], a["io"], None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(dz=None), ttt.TTT_E_INVALID, "non-null"),
    (dict(dw2=None), ttt.TTT_E_INVALID, "dw2"),
    (dict(w1=None), ttt.TTT_E_INVALID, "w1"),
    (dict(dk=None), ttt.TTT_E_INVALID, "dk"),
    (dict(dh=0), ttt.TTT_E_INVALID, "dh"),
    (dict(dh=300), ttt.TTT_E_UNSUPPORTED, "dh=300"),
    (dict(chunk=0), ttt.TTT_E_INVALID, "chunk"),
    (dict(chunk=32, T=64), ttt.TTT_E_UNSUPPORTED, "16 tokens"),
    (dict(eta=float("inf")), ttt.TTT_E_INVALID, "finite"),
    (dict(d=24), ttt.TTT_E_UNSUPPORTED, "d=24"),
    (dict(loss=7), ttt.TTT_E_INVALID, "unknown loss"),
    (dict(deta=FAKE), ttt.TTT_E_INVALID, "deta_tok needs eta_tok"),
    (dict(eta_tok=FAKE, deta=FAKE + 1), ttt.TTT_E_INVALID, "aligned"),
])
def test_mlp_bwd_rejects(lib, kw, code, msg):
    assert _mlp_bwd(lib, **kw) == code
    assert msg in ttt.last_error()


def test_mlp_workspace_size(lib):
    # causal d 64, hidden 256, chunk 16, bf16: 128-byte flags per sequence (rounded up to
    # 256 bytes) and 18 KB of hand-off per chunk of 16 tokens
    B, H, T = 8, 12, 2048
    flags = (B * H * 128 + 255) // 256 * 256
    assert lib.ttt_mlp_fwd_workspace_size(B, H, T, 64, 256, 16, 1, 1) == flags + B * H * (T // 16) * 18432
    assert lib.ttt_mlp_fwd_workspace_size(1, 1, 17, 64, 256, 16, 1, 1) == 256 + 2 * 18432
    # every other shape needs none (the _ws call is then the plain one)
    for args in [(8, 12, 2048, 64, 256, 16, 0, 1), (8, 12, 2048, 64, 256, 16, 1, 0),
                 (8, 12, 2048, 64, 128, 16, 1, 1), (8, 12, 2048, 32, 256, 16, 1, 1),
                 (8, 12, 2048, 64, 256, 8, 1, 1), (8, 12, 0, 64, 256, 16, 1, 1),
                 (0, 12, 2048, 64, 256, 16, 1, 1)]:
        assert lib.ttt_mlp_fwd_workspace_size(*args) == 0, args


def _mlp_ws(lib, ws, ws_bytes, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, w1=FAKE, w2=FAKE, stride=0, z=FAKE, B=2, H=3, T=40, d=64,
             dh=256, chunk=16, causal=1, eta=0.1, eta_tok=None, loss=0, epochs=1, io=1)
    a.update(kw)
    return lib.ttt_mlp_fwd_ws(a["q"], a["k"], a["v"], a["w1"], a["w2"], a["stride"], a["z"], None,
                              None, a["B"], a["H"], a["T"], a["d"], a["dh"], a["chunk"],
                              a["causal"], a["eta"], a["eta_tok"], a["loss"], a["epochs"],
                              a["io"], ws, ws_bytes, None)


def test_mlp_ws_rejects_a_small_or_misaligned_workspace(lib):
    need = lib.ttt_mlp_fwd_workspace_size(2, 3, 40, 64, 256, 16, 1, 1)
    assert _mlp_ws(lib, 0x10000, need - 1) == ttt.TTT_E_INVALID
    assert "workspace of" in ttt.last_error() and "ttt_mlp_fwd_ws" in ttt.last_error()
    assert _mlp_ws(lib, 0x10010, need) == ttt.TTT_E_INVALID
    assert "256-byte aligned" in ttt.last_error()
    # the usual argument checks come first
    assert _mlp_ws(lib, 0x10000, need, q=None) == ttt.TTT_E_INVALID
    assert "non-null" in ttt.last_error()


def test_split_debug_switch(lib):
    prev = lib.ttt_set_split_debug(3)
    try:
        assert lib.ttt_set_split_debug(1) == 3
        assert lib.ttt_set_split_debug(0xFF) == 1
        assert lib.ttt_set_split_debug(0) == 3      # unknown bits are dropped
    finally:
        lib.ttt_set_split_debug(prev)


def test_error_text_is_per_call(lib):
    assert _linear(lib, chunk=0) == ttt.TTT_E_INVALID
    assert "chunk" in ttt.last_error()
    assert _linear(lib, d=48) == ttt.TTT_E_UNSUPPORTED
    assert "chunk" not in ttt.last_error()


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        _binding.load_library.__wrapped__(str(tmp_path / "nope.so")) if hasattr(
            _binding.load_library, "__wrapped__") else _load_missing(tmp_path)


def _load_missing(tmp_path):
    saved = _binding._lib
    try:
        _binding._lib = None
        _binding.load_library(str(tmp_path / "nope.so"))
    finally:
        _binding._lib = saved


def test_linear_bwd_noalloc_rejects_a_history_beyond_its_scratch(lib):
    # 64 x 16 sequences of 8192 tokens: a 4 GiB state history against the 64 MiB scratch
    # array; the check precedes any HIP call
    rc = lib.ttt_linear_bwd_noalloc(FAKE, FAKE, FAKE, FAKE, 0, FAKE, None, FAKE, FAKE, FAKE, FAKE,
                                    64, 16, 8192, 64, 16, 0.1, None, None, 0, 1, None)
    assert rc == ttt.TTT_E_UNSUPPORTED
    assert "scratch" in ttt.last_error()


def _nc_bwd(lib, fn, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, w1=FAKE, w2=FAKE, stride=0, dz=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
             dw1=FAKE, dw2=FAKE, B=1, H=1, T=16, d=16, dh=32, chunk=4, epochs=2, eta=0.1,
             eta_tok=None, deta=None, loss=0, io=0)
    a.update(kw)
    if fn == "linear":
        return lib.ttt_linear_nc_bwd(a["q"], a["k"], a["v"], a["w1"], a["stride"], a["dz"], None,
                                     a["dq"], a["dk"], a["dv"], a["dw1"], a["B"], a["H"], a["T"],
                                     a["d"], a["chunk"], a["epochs"], a["eta"], a["eta_tok"],
                                     a["deta"], a["loss"], a["io"], None)
    return lib.ttt_mlp_nc_bwd(a["q"], a["k"], a["v"], a["w1"], a["w2"], a["stride"], a["dz"], None,
                              None, a["dq"], a["dk"], a["dv"], a["dw1"], a["dw2"], a["B"], a["H"],
                              a["T"], a["d"], a["dh"], a["chunk"], a["epochs"], a["eta"],
                              a["eta_tok"], a["deta"], a["loss"], a["io"], None)


@pytest.mark.parametrize("fn", ["linear", "mlp"])
@pytest.mark.parametrize("kw,code,msg", [
    (dict(epochs=0), ttt.TTT_E_INVALID, "epochs"),
    (dict(chunk=0), ttt.TTT_E_INVALID, "chunk"),
    (dict(dz=None), ttt.TTT_E_INVALID, "non-null"),
    (dict(dk=None), ttt.TTT_E_INVALID, "dk"),
    (dict(dw1=None), ttt.TTT_E_INVALID, "non-null"),
    (dict(deta=FAKE), ttt.TTT_E_INVALID, "deta_tok needs eta_tok"),
    (dict(eta_tok=FAKE + 2), ttt.TTT_E_INVALID, "aligned"),
    (dict(loss=7), ttt.TTT_E_INVALID, "loss"),
    (dict(d=48), ttt.TTT_E_UNSUPPORTED, "d=48"),
    (dict(stride=-1), ttt.TTT_E_INVALID, "stride"),
    (dict(io=5), ttt.TTT_E_INVALID, "io_dtype"),
])
def test_nc_bwd_rejects(lib, fn, kw, code, msg):
    rc = _nc_bwd(lib, fn, **kw)
    assert rc == code and msg in ttt.last_error(), (rc, ttt.last_error())


@pytest.mark.parametrize("kw,code,msg", [
    (dict(dh=0), ttt.TTT_E_INVALID, "dh"),
    (dict(dh=300), ttt.TTT_E_UNSUPPORTED, "dh=300"),
    (dict(w2=None), ttt.TTT_E_INVALID, "non-null"),
])
def test_mlp_nc_bwd_rejects(lib, kw, code, msg):
    rc = _nc_bwd(lib, "mlp", **kw)
    assert rc == code and msg in ttt.last_error(), (rc, ttt.last_error())


def _ln_bwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, w0=FAKE, stride=0, lw=FAKE, lb=FAKE, eps=1e-6, dz=FAKE,
             dq=FAKE, dk=FAKE, dv=FAKE, dw0=FAKE, dlw=FAKE, dlb=FAKE, B=1, H=1, T=16, d=16,
             chunk=16, eta=0.1, eta_tok=None, deta=None, loss=0, io=0)
    a.update(kw)
    return lib.ttt_linear_ln_bwd(a["q"], a["k"], a["v"], a["w0"], a["stride"], a["lw"], a["lb"],
                                 a["eps"], a["dz"], None, a["dq"], a["dk"], a["dv"], a["dw0"],
                                 a["dlw"], a["dlb"], a["B"], a["H"], a["T"], a["d"], a["chunk"],
                                 a["eta"], a["eta_tok"], a["deta"], a["loss"], a["io"], None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(eps=0.0), ttt.TTT_E_INVALID, "ln_eps"),
    (dict(lw=None), ttt.TTT_E_INVALID, "ln_bias must be non-null"),
    (dict(dlb=None), ttt.TTT_E_INVALID, "dln_bias"),
    (dict(chunk=32, T=64), ttt.TTT_E_UNSUPPORTED, "16 tokens"),
    (dict(d=48), ttt.TTT_E_UNSUPPORTED, "d=48"),
    (dict(deta=FAKE), ttt.TTT_E_INVALID, "deta_tok needs eta_tok"),
    (dict(loss=3), ttt.TTT_E_INVALID, "loss"),
])
def test_linear_ln_bwd_rejects(lib, kw, code, msg):
    rc = _ln_bwd(lib, **kw)
    assert rc == code and msg in ttt.last_error(), (rc, ttt.last_error())


def test_mlp_ln_bwd_rejects_oversized_hidden_and_bad_eps(lib):
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, 1e-6, FAKE, None, None, FAKE, FAKE, FAKE,
            FAKE, FAKE, FAKE, FAKE, 1, 1, 16, 16, 300, 16, 0.1, None, None, 0, 0, None]
    assert lib.ttt_mlp_ln_bwd(*args) == ttt.TTT_E_UNSUPPORTED and "dh=300" in ttt.last_error()
    args[8] = -1.0
    assert lib.ttt_mlp_ln_bwd(*args) == ttt.TTT_E_INVALID and "ln_eps" in ttt.last_error()


def test_finite_check_switch(lib):
    """The debug switch is process-wide, off by default and reports its previous value; it
    does not change argument validation."""
    prev = ttt.set_check_finite(False)
    try:
        assert ttt.get_check_finite() is False
        assert ttt.set_check_finite(True) is False
        assert ttt.get_check_finite() is True
        assert lib.ttt_set_check_finite(7) == 1  # any nonzero value is on
        assert lib.ttt_get_check_finite() == 1
        # an invalid call still fails validation first (no GPU call, no check)
        assert _linear(lib, q=None) == ttt.TTT_E_INVALID
        assert "non-null" in ttt.last_error()
        assert ttt.set_check_finite(False) is True
        assert ttt.get_check_finite() is False
    finally:
        ttt.set_check_finite(prev)


@pytest.mark.parametrize("value,on", [("1", True), ("yes", True), ("0", False), ("", False)])
def test_finite_check_environment(value, on):
    """TTT_CHECK_FINITE sets the switch for a fresh process."""
    import subprocess
    import sys
    code = ("import test_sequence_layers_amd as t; print(int(t.get_check_finite()))")
    env = dict(os.environ, TTT_CHECK_FINITE=value)
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=root,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == ("1" if on else "0")
