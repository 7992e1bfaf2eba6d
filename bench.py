"""Benchmark of the TTT-layer forward pass on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu] [--no-others]

A step is one forward call over one batch of the workload (default: TTT-Linear,
B=8 H=12 T=2048 d=64, chunk 16, bf16 Q/K/V, fp32 state).  Inputs are seeded synthetic
tensors already resident in HBM; R independent input/output sets are rotated so that the
working set (R x ~100 MB) exceeds the 256 MB Infinity Cache and every step streams from
HBM.  W warm-up steps, then K timed steps between two synchronisations, timed with HIP
events recorded on the stream the kernels are launched on.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
FP32_VALU_PEAK_TFLOPS = 157.3


def algorithmic_cost(w, epochs=1):
    """(bytes, flops) of one forward call: Q, K, V read + Z written + initial state read;
    flops of the method (tril-masked b x b products counted at half).  With several epochs
    (non-causal) the training flops repeat per epoch; the bytes stay those read once."""
    esz = 2 if w.io == "bf16" else 4
    tok = w.B * w.H * w.T * w.d * esz
    if w.kind in ("linear", "delta"):
        state = w.H * w.d * w.d * 4
        b = 1 if w.kind == "delta" else min(w.chunk, w.T)
        # R = K W^T - V, Q W^T, W update: 3 x 2 d^2 per head-token; tril(QK^T) and P R:
        # 2 x (b/2) x 2d ... counted as 2 b d per head-token.
        fl = w.B * w.H * w.T * ((4 * epochs + 2) * w.d * w.d + (2 * b * w.d if b > 1 and w.causal else 0))
    else:
        state = 2 * w.H * w.d * w.h * 4
        b = min(w.chunk, w.T)
        # training: U, O, R W2, both gradient sums (10 d h); queries: 4 d h
        per = (10 * epochs + 4) * w.d * w.h + (2 * b * (w.d + w.h) if w.causal else 0)
        fl = w.B * w.H * w.T * per
    return 4 * tok + state, fl


def named_workload(name):
    """A workload of the method by name: the five measured workloads, and the non-causal
    TTT-Linear layer at the vision workload's shape (B 64, H 6, N 196, d 64; one full-batch
    step at eta 1, raw keys), the linear inner model of the same setting."""
    from test_sequence_layers_amd.workloads import workload
    if name == "linear_nc_N196":
        return workload("mlp_vision_N196").replace(name=name, kind="linear", h=0)
    return workload(name)


def _profile_record(workload_name, kind, kernel=None):
    """A committed rocprofv3 counter record (profiles/<workload>_<kind>.json), or None when
    none exists, it was taken on another kernel than `kernel` (a name prefix), or the kernel
    source has changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{workload_name}_{kind}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if kernel is not None and not rec.get("kernel", "").startswith(kernel):
        return None
    src = os.path.join(ROOT, rec["source"])
    if not os.path.exists(src):
        return None
    with open(src, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != rec["source_sha256"]:
            return None
    return rec


def measured_traffic(workload_name, kernel=None):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE for the kernel of
    this workload, or None when no record exists or the kernel source has changed since."""
    rec = _profile_record(workload_name, "traffic", kernel)
    return None if rec is None else rec["fetch_bytes"] + rec["write_bytes"]


def measured_mfma_util(workload_name, kernel=None):
    """MFMA utilisation (%) of this workload's kernel from the rocprofv3 derived counter
    MfmaUtil (matrix-core busy cycles over active cycles of all SIMDs), or None."""
    rec = _profile_record(workload_name, "mfma", kernel)
    return None if rec is None else rec["mfma_util_pct"]


def make_device_inputs(w, seed, torch, rates=False, paper=False):
    import numpy as np
    from test_sequence_layers_amd.workloads import make_inputs, make_ln_params, make_token_rates
    inp = make_inputs(w, seed=seed)
    if rates:
        inp["eta_tok"] = make_token_rates(w, seed)
    if paper:
        inp["ln_w"], inp["ln_b"] = make_ln_params(w, seed)
    dt = torch.bfloat16 if w.io == "bf16" else torch.float32
    dev = {}
    for key in ("q", "k", "v"):
        dev[key] = torch.from_numpy(np.ascontiguousarray(inp[key])).to("cuda").to(dt).contiguous()
    for key in ("w0", "w1", "w2", "eta_tok", "ln_w", "ln_b"):
        if key in inp:
            dev[key] = torch.from_numpy(inp[key]).to("cuda").contiguous()
    dev["z"] = torch.empty_like(dev["q"])
    return dev


def launch(w, dev, ttt, loss="mse", epochs=1, ws=None):
    """One forward call.  ws: a workspace for the MLP entry points that take one
    (ttt_mlp_fwd_ws / ttt_mlp_ln_fwd_ws: two workgroups per sequence)."""
    et = dev.get("eta_tok")
    if "ln_w" in dev:  # the paper's inner models: x + LN(f_res(x)), GELU in the MLP
        ln = (dev["ln_w"], dev["ln_b"])
        if w.kind == "linear":
            ttt.ttt_linear_ln_fwd(dev["q"], dev["k"], dev["v"], dev["w0"], *ln, w.eta, w.chunk,
                                  w.causal, eta_tok=et, loss=loss, epochs=epochs, z=dev["z"])
        elif ws is not None:
            ttt.ttt_mlp_ln_fwd_ws(dev["q"], dev["k"], dev["v"], dev["w1"], dev["w2"], *ln, w.eta,
                                  w.chunk, w.causal, workspace=ws, eta_tok=et, loss=loss,
                                  epochs=epochs, z=dev["z"])
        else:
            ttt.ttt_mlp_ln_fwd(dev["q"], dev["k"], dev["v"], dev["w1"], dev["w2"], *ln, w.eta,
                               w.chunk, w.causal, eta_tok=et, loss=loss, epochs=epochs, z=dev["z"])
        return
    if ws is not None and w.kind == "mlp":
        ttt.ttt_mlp_fwd_ws(dev["q"], dev["k"], dev["v"], dev["w1"], dev["w2"], w.eta, w.chunk,
                           w.causal, workspace=ws, eta_tok=et, loss=loss, epochs=epochs, z=dev["z"])
        return
    if w.kind == "linear":
        ttt.ttt_linear_fwd(dev["q"], dev["k"], dev["v"], dev["w0"], w.eta, w.chunk, w.causal,
                           eta_tok=et, loss=loss, epochs=epochs, z=dev["z"])
    elif w.kind == "delta":
        ttt.delta_rule_fwd(dev["q"], dev["k"], dev["v"], dev["w0"], w.eta, eta_tok=et, z=dev["z"])
    else:
        ttt.ttt_mlp_fwd(dev["q"], dev["k"], dev["v"], dev["w1"], dev["w2"], w.eta, w.chunk,
                        w.causal, eta_tok=et, loss=loss, epochs=epochs, z=dev["z"])


def split_workspace(w, torch, ttt):
    """A workspace for the two-workgroup MLP kernel when the workload has its shape (allocated
    once, outside the timed region), else None."""
    if w.kind != "mlp":
        return None
    n = ttt.ttt_mlp_fwd_workspace_size(w.B, w.H, w.T, w.d, w.h, w.chunk, w.causal, w.io)
    return torch.empty(n, dtype=torch.uint8, device="cuda") if n > 0 else None


def time_workload(w, steps, warmup, torch, ttt, rotate=None, rates=False, loss="mse", epochs=1,
                  paper=False, split=True):
    """Event-timed forward calls.  split: the MLP through ttt_mlp_fwd_ws / ttt_mlp_ln_fwd_ws
    (two workgroups per sequence, a workspace allocated here beforehand) where the shape has
    that kernel; False: the one-workgroup entry points."""
    ws = split_workspace(w, torch, ttt) if split else None
    bytes_, flops = algorithmic_cost(w, epochs)
    if rates:
        bytes_ += w.B * w.H * w.T * 4  # the rate factors, read once
    if rotate is None:
        rotate = max(2, min(8, int(6 * 256e6 / max(bytes_, 1)) + 1))
    sets = [make_device_inputs(w, w.seed + i, torch, rates, paper) for i in range(rotate)]
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        launch(w, sets[i % rotate], ttt, loss, epochs, ws)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        launch(w, sets[i % rotate], ttt, loss, epochs, ws)
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    return {
        "ms_per_step": ms,
        "tokens_per_s": w.B * w.T / (ms * 1e-3),
        "head_tokens_per_s": w.B * w.H * w.T / (ms * 1e-3),
        "hbm_gbs": bytes_ / (ms * 1e-3) / 1e9,
        "tflops": flops / (ms * 1e-3) / 1e12,
        "bytes": bytes_,
        "flops": flops,
        "rotated_sets": rotate,
        "kernel": ("mlp_split_kernel" if ws is not None else
                   "mlp_mfma_kernel" if w.kind == "mlp" and w.causal else None),
    }


def time_backward(w, steps, warmup, torch, ttt, rates=False):
    """Event-timed ttt_linear_bwd / ttt_mlp_bwd calls (ttt_linear_bwd with chunk 1 for the
    delta rule, ttt_linear_nc_bwd / ttt_mlp_nc_bwd for the non-causal workloads) on the workload (inputs resident in
    HBM; seeded dZ ~ N(0, 1), no upstream state gradient; rates: TTT-Linear with per-token
    rate factors, their gradient included)."""
    dev = make_device_inputs(w, w.seed, torch, rates=rates)
    g = torch.Generator(device="cuda").manual_seed(w.seed)
    dz = torch.randn(dev["q"].shape, generator=g, device="cuda").to(dev["q"].dtype)
    if not w.causal:  # the non-causal layers
        if w.kind == "linear":
            call = lambda: ttt.ttt_linear_nc_bwd(dev["q"], dev["k"], dev["v"], dev["w0"], w.eta, w.chunk,
                                                 dz, eta_tok=dev.get("eta_tok"))
        else:
            call = lambda: ttt.ttt_mlp_nc_bwd(dev["q"], dev["k"], dev["v"], dev["w1"], dev["w2"], w.eta,
                                              w.chunk, dz, eta_tok=dev.get("eta_tok"))
    elif w.kind in ("linear", "delta"):  # the delta rule is TTT-Linear with chunk 1
        call = lambda: ttt.ttt_linear_bwd(dev["q"], dev["k"], dev["v"], dev["w0"], w.eta, w.chunk, dz,
                                          eta_tok=dev.get("eta_tok"))
    else:
        call = lambda: ttt.ttt_mlp_bwd(dev["q"], dev["k"], dev["v"], dev["w1"], dev["w2"], w.eta,
                                       w.chunk, dz)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        call()
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps
    return {"ms_per_step": ms, "tokens_per_s": w.B * w.T / (ms * 1e-3)}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(w, budget_s=1.5, repeats=3):
    """Time the CPU oracle (the NumPy recurrence as it stands) on a bounded sample of the
    workload: full-length sequences of up to B*H (batch, head) chains, repeated in passes so
    one run takes about budget_s.  Median of `repeats` runs each in float32 with every host
    core, float32 with one thread and float64 with every core (about 15 s of CPU work in
    all); tokens/s scaled to the metric's unit (a token counts once across its H heads)."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    from oracle import ttt_oracle as O
    from test_sequence_layers_amd.workloads import make_inputs

    def run(n_chains, dtype, passes=1):
        x = make_inputs(w, B=1, H=n_chains)
        t0 = time.perf_counter()
        for _ in range(passes):
            if w.kind == "linear":
                O.ttt_linear(x["q"], x["k"], x["v"], x["w0"], w.eta, w.chunk, w.causal, dtype=dtype)
            elif w.kind == "delta":
                O.delta_rule(x["q"], x["k"], x["v"], x["w0"], w.eta, dtype=dtype)
            else:
                O.ttt_mlp(x["q"], x["k"], x["v"], x["w1"], x["w2"], w.eta, w.chunk, w.causal,
                          dtype=dtype)
        return time.perf_counter() - t0

    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1

    def timed(threads, dtype):
        """(sequences, passes, median seconds, tokens/s): passes over up to B*H sequences,
        enough for one run to take about budget_s."""
        ctx = threadpool_limits(limits=threads) if threadpool_limits else None
        if ctx:
            ctx.__enter__()
        try:
            t1 = run(1, dtype)
            n = int(max(1, min(w.B * w.H, budget_s / max(t1, 1e-6))))
            tn = run(n, dtype)
            passes = int(max(1, round(budget_s / max(tn, 1e-6))))
            ts = sorted(run(n, dtype, passes) for _ in range(repeats))
        finally:
            if ctx:
                ctx.__exit__(None, None, None)
        tm = ts[len(ts) // 2]
        return n, passes, tm, n * passes * w.T / w.H / tm

    n_all, p_all, t_all, v_all = timed(cores, np.float32)
    n_one, p_one, t_one, v_one = timed(1, np.float32)
    n_64, p_64, t_64, v_64 = timed(cores, np.float64)
    return {
        "value": v_all,
        "unit": "tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{n_all} of the {w.B * w.H} (batch, head) sequences at full length T={w.T}, "
                  f"{p_all} pass(es) per run, float32 NumPy, median of {repeats} runs "
                  f"({t_all:.2f} s each) with {cores} threads allowed",
        "one_thread": {"value": v_one, "unit": "tokens/s", "cores": 1,
                       "sample": f"{n_one} sequences x {p_one} pass(es), median of {repeats} "
                                 f"runs ({t_one:.2f} s each)"},
        "float64": {"value": v_64, "unit": "tokens/s", "cores": cores,
                    "sample": f"{n_64} sequences x {p_64} pass(es), median of {repeats} runs "
                              f"({t_64:.2f} s each)"},
        "cpu_model": _cpu_model(),
        "note": "the oracle steps through the tokens in Python, each step a few NumPy calls "
                "on small matrices batched over the sampled sequences, so the thread count "
                "barely changes it",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="linear_d64_T2048")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-others", action="store_true", help="time only the headline workload")
    ap.add_argument("--rotate", type=int, default=None,
                    help="input/output sets rotated per step (default: enough to exceed the 256 MB "
                         "Infinity Cache; 1 = every step re-reads the same cache-warm buffers)")
    ap.add_argument("--token-rates", action="store_true",
                    help="time the workload with per-token rate factors eta_tok [B, H, T]")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="before timing, run one plain device copy of this many MB (counter scale)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU only (every GPU would run its own "
                                   "share of the independent sequences); --gpus must be 1"}))
        sys.exit(2)
    for key in ("RANK", "WORLD_SIZE"):
        if int(os.environ.get(key, "0" if key == "RANK" else "1")) not in (0, 1):
            print("multi-rank runs are not supported", file=sys.stderr)
            sys.exit(2)

    import torch

    import test_sequence_layers_amd as ttt
    from test_sequence_layers_amd.workloads import WORKLOADS, workload

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    ttt.load_library()

    if args.copy_probe_mb:
        n = args.copy_probe_mb * (1 << 20) // 4
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    w = named_workload(args.workload)
    res = time_workload(w, args.steps, args.warmup, torch, ttt, rotate=args.rotate,
                        rates=args.token_rates)

    def roofline_of(wl, r, rates=False):
        if wl.kind == "mlp":
            # dense bf16 contractions: priced against the matrix-core peak
            kern = r.get("kernel") or ("mlp_mfma_kernel" if wl.causal else "mlp_nc_kernel")
            return {
                "bound": "mfma",
                "achieved": round(r["tflops"], 2),
                "peak": BF16_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s",
                "frac": round(r["tflops"] / BF16_MFMA_PEAK_TFLOPS, 4),
                "traffic": None if rates else measured_traffic(wl.name, kern),
                "kernel": f"{kern} (per launch: the method's flops, tril products at half)",
                "flops_per_launch": r["flops"],
            }
        kern = ("linear_mfma_kernel (delta rule)" if wl.kind == "delta"
                else "linear_mfma_kernel" if wl.causal else "linear_nc_kernel")
        return {
            "bound": "hbm",
            "achieved": round(r["hbm_gbs"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(r["hbm_gbs"] / HBM_PEAK_GBS, 4),
            "traffic": None if rates else measured_traffic(wl.name),
            "kernel": f"{kern} (per launch: Q,K,V read + Z written + W0 read)",
            "bytes_per_launch": r["bytes"],
        }

    roofline = roofline_of(w, res, args.token_rates)
    # the MFMA half of the metric: the matrix-core-bound d = 64, T = 2048 workload (the causal
    # TTT-MLP, hidden 256), timed here as a first-class figure next to the headline
    mw = workload("mlp_h256_T2048")
    mres = res if w.name == mw.name else time_workload(mw, max(10, args.steps // 2), 5, torch, ttt)
    line = {
        "metric": "TTT-layer fwd tokens/sec at d=64,T=2048 + MFMA util % (1 MI355X)",
        "value": round(res["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.io == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) Q/K/V, unit keys, W0 ~ N(0, 0.02^2))",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "d": w.d,
                   "chunk": w.chunk, "causal": w.causal, "eta": w.eta, "state": "f32",
                   "per_token_rates": bool(args.token_rates),
                   "rotated_input_sets": res["rotated_sets"]},
        "mfma_util_pct": round(100 * mres["tflops"] / BF16_MFMA_PEAK_TFLOPS, 3),
        "mfma_util_workload": mw.name,
        "mfma_util_rocprof_pct": measured_mfma_util(mw.name, mres.get("kernel")),
        "mfma_util_kernel": mres.get("kernel"),
        "roofline": roofline,
        "roofline_mfma": dict(roofline_of(mw, mres), workload=mw.name,
                              tokens_per_s=round(mres["tokens_per_s"], 1),
                              ms_per_step=round(mres["ms_per_step"], 5)),
        "headline_mfma_util_pct": round(100 * res["tflops"] / BF16_MFMA_PEAK_TFLOPS, 3),
        "headline_mfma_util_rocprof_pct": None if args.token_rates else measured_mfma_util(w.name),
    }
    if not args.no_others:
        others = {}
        for o in WORKLOADS:
            if o.name == w.name:
                continue
            r = mres if o.name == mw.name else time_workload(o, max(10, args.steps // 2), 5, torch, ttt)
            others[o.name] = {
                "tokens_per_s": round(r["tokens_per_s"], 1),
                "ms_per_step": round(r["ms_per_step"], 5),
                "hbm_gbs": round(r["hbm_gbs"], 1),
                "tflops": round(r["tflops"], 3),
                "mfma_util_pct": round(100 * r["tflops"] / BF16_MFMA_PEAK_TFLOPS, 3),
            }
            mu = measured_mfma_util(o.name, r.get("kernel"))
            if mu is not None:
                others[o.name]["mfma_util_rocprof_pct"] = mu
            if r.get("kernel"):
                others[o.name]["kernel"] = r["kernel"]
        # variants: the headline workload with per-token rate factors (uniform in [0, 1)),
        # the dot-product loss on the headline and the vision workloads, mini-batches with
        # epochs on the vision workload
        variants = []
        if not args.token_rates:
            variants.append((w, "+token_rates", dict(rates=True)))
        variants.append((w, "+dot_loss", dict(loss="dot")))
        variants += [(o, "+dot_loss", dict(loss="dot")) for o in WORKLOADS
                     if o.name == "mlp_vision_N196"]
        # the non-causal TTT-Linear layer at the vision shape (one full-batch step), with the
        # reconstruction and the dot-product loss
        lnc = named_workload("linear_nc_N196")
        if w.name != lnc.name:
            variants.append((lnc, "", {}))
        variants.append((lnc, "+dot_loss", dict(loss="dot")))
        # the vision workload in four consecutive mini-batches of 49 pairs, two epochs
        # (eta 0.01: at eta 1 several steps diverge)
        variants += [(o.replace(chunk=49, eta=0.01), "+chunk49_epochs2", dict(epochs=2))
                     for o in WORKLOADS if o.name == "mlp_vision_N196"]
        # the paper's inner models (x + LN(f_res(x)); GELU in the MLP) on the headline linear
        # and the causal MLP workloads
        variants += [(o, "+paper_ln", dict(paper=True)) for o in WORKLOADS
                     if o.name in ("linear_d64_T2048", "mlp_h256_T2048")]
        # the causal MLP workloads on the one-workgroup kernel (ttt_mlp_fwd / ttt_mlp_ln_fwd,
        # no workspace)
        variants += [(o, "+one_workgroup", dict(split=False)) for o in WORKLOADS
                     if o.name == "mlp_h256_T2048"]
        variants += [(o, "+paper_ln+one_workgroup", dict(paper=True, split=False))
                     for o in WORKLOADS if o.name == "mlp_h256_T2048"]
        # backward passes of the headline linear workload, the delta rule, the causal MLP
        # workload and the vision workload (dz ~ N(0, 1), no upstream state gradient)
        bwd = [w] if w.kind == "linear" else []
        bwd += [o for o in WORKLOADS
                if o.name in ("delta_d64_T8192", "mlp_h256_T2048", "mlp_vision_N196")]
        for o in bwd:
            quick = o.kind == "linear" and o.chunk > 1
            r = time_backward(o, max(10, args.steps // 2) if quick else 3, 3 if quick else 1,
                              torch, ttt)
            others[o.name + "+backward"] = {
                "tokens_per_s": round(r["tokens_per_s"], 1),
                "ms_per_step": round(r["ms_per_step"], 5),
            }
            if o.kind == "linear":
                r = time_backward(o, max(10, args.steps // 2), 3, torch, ttt, rates=True)
                others[o.name + "+backward+token_rates"] = {
                    "tokens_per_s": round(r["tokens_per_s"], 1),
                    "ms_per_step": round(r["ms_per_step"], 5),
                }
        for o, tag, kw in variants:
            r = time_workload(o, max(10, args.steps // 2), 5, torch, ttt, **kw)
            others[o.name + tag] = {
                "tokens_per_s": round(r["tokens_per_s"], 1),
                "ms_per_step": round(r["ms_per_step"], 5),
                "hbm_gbs": round(r["hbm_gbs"], 1),
                "tflops": round(r["tflops"], 3),
                "mfma_util_pct": round(100 * r["tflops"] / BF16_MFMA_PEAK_TFLOPS, 3),
            }
        line["other_workloads"] = others
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
