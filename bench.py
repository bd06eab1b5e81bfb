"""Benchmark: one MoE layer forward + backward on one MI355X, through the libmoe C ABI.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--config 3] [--no-cpu-baseline]

A step is the whole hot path on one batch: gate logits, router, permute, grouped SwiGLU
experts (+ shared expert), combine, and the backward of all of it (combine backward,
expert data and weight gradients, router backward, gate backward, unpermute-reduce).
Inputs are seeded synthetic tensors of the named layer, resident in HBM before timing.
Each C-ABI call of a step is bracketed by HIP events on the launch stream, so every
phase's duration is measured live over the timed steps.  The expert backward runs as its
data gradients followed by four grouped weight-gradient calls of one kernel launch each; the
routed fc1 weight gradient, the longest single kernel of the step, is the one the roofline
object reports.  Prints one JSON line.

    python bench.py --copy-calibration   # only 3 x 1 GiB device copies, for counter scaling
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# Published MI355X peaks.
PEAK_BF16_TFLOPS = 2516.6
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBPS = 8000.0

PHASES = ["gate", "router", "permute", "experts_fwd", "combine", "combine_bwd", "experts_bwd_data", "wgrad_fc2",
          "wgrad_fc1", "wgrad_shared", "router_bwd", "gate_bwd", "unpermute_reduce"]
GEMM_PHASES = ["experts_fwd", "experts_bwd_data", "wgrad_fc2", "wgrad_fc1", "wgrad_shared"]
# The kernel the roofline object reports: the routed fc1 weight gradient, one launch of the
# reduction-ragged weight-gradient kernel, the longest single kernel of the step.
ROOFLINE_PHASE = "wgrad_fc1"
ROOFLINE_SOURCE = os.path.join(ROOT, "mixture_experts_layer_aux_amd", "csrc", "moe_wgrad.hip")


def algorithmic(shape, wgrad_bytes=4):
    """Algorithmic work per step: the bytes each HBM-bound kernel must move and the FLOP
    each GEMM must compute, at minimum.  wgrad_bytes: bytes per expert weight-gradient
    element (2 for bf16, 4 for fp32).  bf16 layers keep no grouped copy of x: the permute
    moves indices only and the fc1 GEMMs read the token rows through token_of."""
    T, d, E, k, F, Fs = shape.T, shape.d, shape.E, shape.k, shape.F, shape.Fs
    A = T * k
    eb = 2 if shape.act == "bf16" else 4
    gather = shape.act == "bf16"
    gemm_fwd = 6.0 * d * (F * A + Fs * T)          # fc1 (2 x d x 2F) + fc2 (2 x F x d) per row
    return dict(
        grouped_gemm_flop=3.0 * gemm_fwd,          # forward + data gradient + weight gradient
        wgrad_fc1_flop=2.0 * A * 2 * F * d,        # dW13 = dH^T X over the routed rows
        # dW13 written once, dH and the routed rows of x read once, the offsets (and the
        # token index of each routed row)
        wgrad_fc1_bytes=E * 2 * F * d * wgrad_bytes + A * 2 * F * eb + A * d * eb + (E + 1) * 4 + (A * 4 if gather else 0),
        gate_flop=6.0 * T * E * d,                 # logits, dWg, dx_r
        # bytes each HBM-bound phase must move at least once, every activation row in the
        # activation dtype (the layer's statement: Y_perm, dX_perm, y, dy, dx as act rows)
        router_bytes=T * E * 4 + T * k * 8 + E * 8,
        # idx read, row_of and token_of written (+ x read and x_perm written with the copy)
        permute_bytes=A * 4 * 3 + (0 if gather else T * d * eb + A * d * eb),
        combine_bytes=A * d * eb + (T * d * eb if Fs else 0) + T * d * eb + T * k * 8,
        combine_bwd_bytes=T * d * eb + 2 * A * d * eb + T * k * 12,
        unpermute_reduce_bytes=A * d * eb + T * d * eb + T * k * 4,
        # the same with this library's storage: Y_perm, Y_s, dX_perm, dx_s, dx_r, y, dy, dx in
        # fp32, dY_perm and dY_s in the activation dtype
        combine_bytes_storage=A * d * 4 + (T * d * 4 if Fs else 0) + T * k * 8 + T * d * 4,
        combine_bwd_bytes_storage=T * d * 4 + A * d * 4 + A * d * eb + (T * d * eb if Fs else 0) + T * k * 12,
        unpermute_reduce_bytes_storage=A * d * 4 + (T * d * 4 if Fs else 0) + T * d * 4 + T * d * 4 + T * k * 4,
    )


def measured_traffic(shape):
    """HBM bytes per launch of the roofline kernel from the committed rocprofv3 counter
    summary, or None when there is none for this layer or the kernel's source has changed
    since the counters were taken (the summary records the source's sha256)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"wgrad_fc1_{shape.name}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ": " in line:
                key, val = line[2:].split(": ", 1)
                fields[key.strip("` ")] = val.strip().strip("`")
    with open(ROOFLINE_SOURCE, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    if fields.get("kernel_source_sha256") != sha or "traffic_bytes_per_launch" not in fields:
        return None
    return int(fields["traffic_bytes_per_launch"])


def roofline(alg, ms, peak_tflops, shape, wgrad_name="fp32"):
    """Roofline of one launch of the routed fc1 weight-gradient kernel: the bound is the
    resource whose peak gives the longer time for its algorithmic work."""
    flop, nbytes = alg["wgrad_fc1_flop"], alg["wgrad_fc1_bytes"]
    t_mfma = flop / (peak_tflops * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBPS * 1e9)
    s = ms * 1e-3
    x_rows = "the token rows of x through token_of" if shape.act == "bf16" else "x_perm"
    common = dict(kernel=f"routed fc1 weight gradient dW13 = dH^T X, X = {x_rows} (one launch of the "
                         f"reduction-ragged weight-gradient kernel, bf16 MFMA, {wgrad_name} output)",
                  launch_ms=round(ms, 4), flop_per_launch=flop, bytes_per_launch=int(nbytes),
                  mfma_frac=round(flop / s / 1e12 / peak_tflops, 4), hbm_frac=round(nbytes / s / 1e9 / PEAK_HBM_GBPS, 4))
    if t_hbm >= t_mfma:
        gbps = nbytes / s / 1e9
        return dict(bound="hbm", achieved=round(gbps, 1), peak=PEAK_HBM_GBPS, unit="GB/s",
                    frac=round(gbps / PEAK_HBM_GBPS, 4), traffic=measured_traffic(shape), **common)
    tf = flop / s / 1e12
    return dict(bound="mfma", achieved=round(tf, 2), peak=peak_tflops, unit="TFLOP/s", frac=round(tf / peak_tflops, 4),
                traffic=measured_traffic(shape), **common)


def gate_engine(shape):
    """Where the router GEMMs run: on the bf16 matrix cores through exact three-way bf16
    splits of the fp32 operand (bf16 activations, E % 16 == 0: 4x the algorithmic FLOP are
    executed over forward and backward), else fp32 FMA tiles."""
    if shape.act == "bf16" and shape.E % 16 == 0:
        return dict(engine="bf16 MFMA, exact 3-way split of the fp32 operand", flop_executed_per_flop=4.0,
                    peak=PEAK_BF16_TFLOPS)
    return dict(engine="fp32 FMA", flop_executed_per_flop=1.0, peak=PEAK_FP32_TFLOPS)


def cpu_model() -> str:
    """The host CPU's model name (lscpu, else /proc/cpuinfo)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(shape, inp, tokens: int):
    """The fp64 oracle's layer forward + backward on the first `tokens` tokens of the same
    inputs, timed on the host cores.  The fp64 copies of the weights of the experts those
    tokens reach (and of the router and shared expert) are made before the clock starts."""
    from threadpoolctl import threadpool_info

    from mixture_experts_layer_aux_amd import workloads as W
    from oracle import moe_oracle as O

    act = shape.act
    x = W.to_f32(inp["x"][:tokens], act).astype(np.float64)
    dy = W.to_f32(inp["dy"][:tokens], act).astype(np.float64)
    spec = O.LayerSpec(E=shape.E, k=shape.k, score=shape.score, scaling=shape.scaling, aux_coeff=shape.aux_coeff)
    Wg = inp["Wg"].astype(np.float64)
    idx = O.route(O.gate_logits(x, Wg, inp["bg"]), spec, inp["expert_bias"])["idx"]
    experts = sorted(set(idx.ravel().tolist()))
    W13 = {e: W.to_f32(inp["W13"][e], act).astype(np.float64) for e in experts}
    W2 = {e: W.to_f32(inp["W2"][e], act).astype(np.float64) for e in experts}
    W13s = W.to_f32(inp["W13s"], act).astype(np.float64) if shape.Fs else None
    W2s = W.to_f32(inp["W2s"], act).astype(np.float64) if shape.Fs else None
    # the same sample, run until at least 10 s of CPU work is timed (at most 8 runs): a
    # larger sample would reach more experts, each an fp64 weight copy of hundreds of MB
    runs, t0 = 0, time.perf_counter()
    while True:
        f = O.layer_forward(x, Wg, W13, W2, spec, bg=inp["bg"], expert_bias=inp["expert_bias"], W13s=W13s, W2s=W2s)
        O.layer_backward(f, x, Wg, W13, W2, dy, spec, W13s=W13s, W2s=W2s, sparse_expert_grads=True)
        runs += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or runs >= 8:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return dict(value=round(tokens * runs / dt, 4), unit="tokens/s", cores=int(threads), kind="oracle",
                cpu_model=cpu_model(), os_cpu_count=os.cpu_count(),
                sample=(f"fp64 oracle forward+backward of the first {tokens} of {shape.T} tokens of the "
                        f"{shape.name} layer ({len(experts)} experts reached), run {runs} times in {dt:.1f} s on "
                        f"{threads} BLAS threads; fp64 weight copies made before timing"))


PHASES_FP8 = ["gate", "router", "quantize_x", "permute", "experts_fwd", "combine", "combine_bwd", "router_bwd",
              "gate_bwd"]
PEAK_FP8_TFLOPS = 5033.2


def bench_fp8(args, shape, cfg, inp, up, dev) -> int:
    """The layer with e4m3 experts: the forward plus the backward through the router path
    (the experts are frozen).  The e4m3 weights come from the fp32 masters through the
    library's quantiser before timing."""
    import torch

    from mixture_experts_layer_aux_amd import _lib as L
    from mixture_experts_layer_aux_amd import workloads as W

    T, d, E, k, F, A = shape.T, shape.d, shape.E, shape.k, shape.F, shape.A
    f32, u8 = torch.float32, torch.uint8
    e = lambda *s_, dt=f32: torch.empty(*s_, dtype=dt, device=dev)  # noqa: E731
    W13m, W2m = up(inp["W13"]), up(inp["W2"])
    W13q, W13s = e(E, 2 * F, d, dt=u8), e(E * 2 * F // 128, d // 128)
    W2q, W2s = e(E, d, F, dt=u8), e(E * d // 128, F // 128)
    L.quantize_fp8(W13m.view(E * 2 * F, d), 128, W13q.view(E * 2 * F, d), W13s)
    L.quantize_fp8(W2m.view(E * d, F), 128, W2q.view(E * d, F), W2s)
    torch.cuda.synchronize()
    del W13m, W2m
    Wg, bg = up(inp["Wg"]), up(inp["bg"])
    x = up(inp["x"])
    dy = up(W.to_f32(inp["dy"], shape.act))
    S = L.alloc_saved(cfg, dev)
    ws = L.alloc_workspace(cfg, dev)
    xq, xs = e(T, d, dt=u8), e(T, d // 128)
    y, dx, dw, dlogits = e(T, d), e(T, d), e(T, k), e(T, E)
    dWg, dbg = e(E, d), (e(E) if bg is not None else None)
    stats = e(L.MOE_NSTATS)

    def step(ev):
        i = 0

        def mark():
            nonlocal i
            if ev is not None:
                ev[i].record()
            i += 1

        mark()
        L.gate_logits(cfg, x, Wg, bg, S["logits"], ws)
        mark()
        L.router_topk(cfg, S["logits"], None, S["idx"], S["w"], S["counts"], None, stats, ws)
        mark()
        L.quantize_fp8(x, 1, xq, xs)
        mark()
        L.permute_fp8(cfg, None, None, S["idx"], S["offsets"], S["row_of"], S["token_of"], None, None, ws)
        mark()
        L.grouped_gemm_swiglu_fp8(cfg, xq, xs, S["offsets"], W13q, W13s.view(-1), W2q, W2s.view(-1), None,
                                  S["Act"], S["Act_scale"], S["Y_perm"], ws, token_of=S["token_of"])
        mark()
        L.unpermute_combine(cfg, S["Y_perm"], S["row_of"], S["w"], None, y)
        mark()
        L.unpermute_combine_bwd(cfg, dy, S["Y_perm"], S["row_of"], S["w"], None, dw, None)
        mark()
        L.router_bwd(cfg, S["logits"], S["idx"], S["w"], dw, S["counts"], 1.0, dlogits)
        mark()
        L.gate_logits_bwd(cfg, x, Wg, dlogits, dWg, dbg, dx, ws)
        mark()

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(PHASES_FP8) + 1)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for st in range(args.steps):
        step(events[st])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    phase_ms = {p: float(np.mean([events[st][i].elapsed_time(events[st][i + 1]) for st in range(args.steps)]))
                for i, p in enumerate(PHASES_FP8)}
    ms_step = elapsed * 1e3 / args.steps
    st_ = stats.cpu().numpy()
    flop = 6.0 * d * F * A                                   # fc1 (4 d F) + fc2 (2 d F) per routed row
    ms = phase_ms["experts_fwd"]
    tf = flop / (ms * 1e-3) / 1e12
    out = dict(
        metric="MoE layer fwd+bwd tokens/s on 1 MI355X", value=round(T / (ms_step * 1e-3), 1), unit="tokens/s",
        n_gpus=1, steps=args.steps, warmup=args.warmup, ms_per_step=round(ms_step, 3), higher_is_better=True,
        scaling="weak", vs_baseline=None, dtype="fp8-e4m3 experts, bf16 activations",
        data="synthetic (seeded generator, random-init weights)",
        config=dict(workload=shape.name, T=T, d=d, E=E, k=k, F=F, Fs=0, score=shape.score, bias=shape.bias,
                    passes="forward + router-path backward (frozen fp8 experts)",
                    fc1_rows="token rows' e4m3 codes through token_of (no grouped copy)", parallelism="single GPU"),
        roofline=dict(kernel="grouped fp8 SwiGLU experts forward (fc1 GEMM, Act quantised in its epilogue with "
                             "128-row tiles or by the quantiser after it, fc2 GEMM)",
                      bound="mfma", achieved=round(tf, 2), peak=PEAK_FP8_TFLOPS, unit="TFLOP/s",
                      frac=round(tf / PEAK_FP8_TFLOPS, 4), traffic=None, flop_per_step=flop, ms_per_step=round(ms, 4)),
        phases_ms={p: round(v, 4) for p, v in phase_ms.items()},
        load=dict(maxvio=round(float(st_[1]), 4), empty_experts=int(st_[2]), max_count=int(st_[3]),
                  mean_count=T * k / E))
    print(json.dumps(out), flush=True)
    return 0


def bench_wgrad_f32(args, shape, L, S, x, dY_perm, dH, dev, phase_ms, ws):
    """The two routed weight-gradient launches again with fp32 output (the other option of
    the weight-gradient dtype), timed with HIP events on the launch stream, beside the
    step's bf16 ones."""
    import torch
    T, d, E, k, F = shape.T, shape.d, shape.E, shape.k, shape.F
    A = T * k
    c32 = L.config_from_shape(shape, wgrad="f32")
    dW13 = torch.empty(E, 2 * F, d, dtype=torch.float32, device=dev)
    dW2 = torch.empty(E, d, F, dtype=torch.float32, device=dev)
    runs = max(args.steps // 2, 3)
    res = {}
    X, x_rows = (x, S["token_of"]) if "x_perm" not in S else (S["x_perm"], None)
    for name, fn in (("wgrad_fc1", lambda: L.grouped_wgrad(c32, S["offsets"], E, A, dH, 2 * F, X, d, dW13,
                                                           x_rows=x_rows, ws=ws)),
                     ("wgrad_fc2", lambda: L.grouped_wgrad(c32, S["offsets"], E, A, dY_perm, d, S["Act"], F, dW2, ws=ws))):
        fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(runs + 1)]
        ev[0].record()
        for i in range(runs):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        res[name + "_ms"] = round(float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(runs)])), 4)
    del dW13, dW2
    res["step_ms_estimate"] = round(sum(phase_ms.values()) - phase_ms["wgrad_fc1"] - phase_ms["wgrad_fc2"]
                                    + res["wgrad_fc1_ms"] + res["wgrad_fc2_ms"], 3)
    res["note"] = ("fp32 output of the routed weight gradients (bench.py --wgrad f32 times the whole step that way); "
                   "the shared expert's two launches are small and not repeated")
    return res


# Sequence length of each layer's batch for the sequence-wise loss (tokens in [S, B] order):
# 4 x 2048 for the small layer (as it is named), 4096-token sequences for the others.
SEQ_LEN = {1: 32, 2: 2048, 3: 4096, 4: 4096, 5: 4096}


def bench_balancing(args, shape, L, S, expert_bias, dw, dlogits, dev):
    """The balancing step around the router, timed with HIP events on the launch stream:
    the router with the sequence-wise loss (1e-4, DeepSeek-V3's value) and, for softmax
    routers, the z-loss (1e-3, ST-MoE's value) on; its backward with those losses; and the
    sign update of the expert bias (rate 1e-3) for the sigmoid and sqrt(softplus) routers."""
    import torch
    T, E, k = shape.T, shape.E, shape.k
    cid = args.config
    z = 1e-3 if shape.score == "softmax" else 0.0
    cfg = L.config_from_shape(shape, z_coeff=z, seq_aux_coeff=1e-4, seq_len=SEQ_LEN[cid])
    B = L.num_sequences(cfg)
    sc = torch.empty(B, E, dtype=torch.int32, device=dev)
    st = torch.empty(L.MOE_NSTATS, dtype=torch.float32, device=dev)
    ws = torch.empty(L.workspace_size(cfg)[0], dtype=torch.uint8, device=dev)   # the router needs the forward part
    bias = expert_bias.clone() if expert_bias is not None else None
    runs = max(args.steps, 5)

    def timed(fn):
        for _ in range(2):
            fn()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(runs + 1)]
        ev[0].record()
        for i in range(runs):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        return float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(runs)]))

    def fwd():
        L.router_topk(cfg, S["logits"], expert_bias, S["idx"], S["w"], S["counts"], None, st, ws, seq_counts=sc)

    out = dict(recipe=f"sequence-wise aux loss 1e-4 over {B} sequences of {SEQ_LEN[cid]} tokens"
               + (", z-loss 1e-3" if z else ", sign update of the expert bias at rate 1e-3"),
               router_ms=round(timed(fwd), 4))
    out["router_bwd_ms"] = round(timed(lambda: L.router_bwd(cfg, S["logits"], S["idx"], S["w"], dw, S["counts"], 1.0,
                                                           dlogits, seq_counts=sc)), 4)
    if bias is not None:
        out["bias_update_ms"] = round(timed(lambda: L.expert_bias_update(cfg, S["counts"], 1e-3, False, bias)), 4)
    # quantile balancing on the same logits: the router's scores (sigmoid, or the full
    # softmax), bias solved from zero, then the EMA update (0.9)
    scores = (torch.sigmoid(S["logits"]) if shape.score != "softmax" else torch.softmax(S["logits"], dim=1)).contiguous()
    qbeta = torch.zeros(E, dtype=torch.float32, device=dev)
    qidx = torch.empty(T, k, dtype=torch.int32, device=dev)
    qalpha = torch.empty(T, dtype=torch.float32, device=dev)
    qlocal = torch.empty(E, dtype=torch.float32, device=dev)
    if (T * k) % E == 0 and k < E:
        out["quantile_router_ms"] = round(timed(lambda: L.router_quantile(cfg, scores, qbeta, qidx, qalpha, qlocal,
                                                                          ws)), 4)
        out["quantile_update_ms"] = round(timed(lambda: L.quantile_bias_update(cfg, qlocal, 0.9, qbeta)), 4)
        # scores read once for the top-(k+1) and once per radix pass (4), alpha and idx
        out["quantile_bytes"] = 5 * T * E * 4 + T * k * 4 + 5 * T * 4
    # bytes the sequence pass must move on top of the router's: the logits again, idx, and
    # the per-token normalisers written and read
    seq_bytes = T * E * 4 + T * k * 4 + 2 * T * 8
    vals = st.cpu().numpy()
    out.update(seq_pass_bytes=seq_bytes, z_loss=float(vals[4]), seq_aux_loss=float(vals[5]))
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--wgrad", choices=["default", "f32"], default="default",
                    help="dtype of the expert weight gradients: the activation dtype (default) or fp32")
    ap.add_argument("--no-entry-points", action="store_true",
                    help="skip timing the layer through moe_layer_fwd + moe_layer_bwd (reported beside value)")
    ap.add_argument("--cpu-tokens", type=int, default=0, help="tokens in the oracle sample (0 = by layer)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 3 device copies of 1 GiB each (the known-size kernel that scales the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the layer; --gpus {args.gpus} is not supported "
              "(expert-parallel sharding across GPUs is not built)", file=sys.stderr)
        return 2

    import torch

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps(dict(copy_bytes_read=src.numel() * 4, copy_bytes_written=dst.numel() * 4, copies=3)))
        return 0

    from mixture_experts_layer_aux_amd import _lib as L
    from mixture_experts_layer_aux_amd import workloads as W

    if not os.path.exists(L.LIB_PATH):
        from mixture_experts_layer_aux_amd import build as B
        B.build()
    L.load()
    shape = W.LAYERS[args.config]
    cfg = L.config_from_shape(shape, **({"wgrad": "f32"} if args.wgrad == "f32" else {}))
    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    inp = W.make_inputs(shape, seed=args.config)
    t_gen = time.perf_counter() - t_gen
    print(f"[bench] {shape.name}: inputs generated in {t_gen:.1f} s", file=sys.stderr, flush=True)

    def up(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    T, d, E, k, F, Fs, A = shape.T, shape.d, shape.E, shape.k, shape.F, shape.Fs, shape.A
    if shape.wq == "fp8":
        return bench_fp8(args, shape, cfg, inp, up, dev)
    Wt = dict(Wg=up(inp["Wg"]), bg=up(inp["bg"]), expert_bias=up(inp["expert_bias"]), W13=up(inp["W13"]),
              W2=up(inp["W2"]), W13s=up(inp["W13s"]), W2s=up(inp["W2s"]))
    x = up(inp["x"])
    dy = up(W.to_f32(inp["dy"], shape.act))
    S = L.alloc_saved(cfg, dev)        # bf16: no grouped copy of x, the fc1 GEMMs read it through token_of
    gather = "x_perm" not in S
    tok = S["token_of"] if gather else None
    X1 = x if gather else S["x_perm"]   # the fc1 weight gradient's X
    G = L.alloc_grads(cfg, dev, with_dbg=inp["bg"] is not None)
    ws = L.alloc_workspace(cfg, dev)
    f32, ad = torch.float32, L.act_dtype(cfg)
    y = torch.empty(T, d, dtype=f32, device=dev)
    dx = torch.empty(T, d, dtype=f32, device=dev)
    stats = torch.empty(L.MOE_NSTATS, dtype=f32, device=dev)
    # backward scratch owned by the caller (the piecewise calls name every tensor)
    # dY_perm must outlive the data gradients here: the fc2 weight gradient runs after them
    dY_perm = torch.empty(A, d, dtype=ad, device=dev)
    dX_perm = torch.empty(A, d, dtype=f32, device=dev)
    dH = torch.empty(A, 2 * F, dtype=ad, device=dev)
    dw = torch.empty(T, k, dtype=f32, device=dev)
    dlogits = torch.empty(T, E, dtype=f32, device=dev)
    dx_r = torch.empty(T, d, dtype=f32, device=dev)
    dH_s = torch.empty(T, 2 * Fs, dtype=ad, device=dev) if Fs else None
    dx_s = torch.empty(T, d, dtype=f32, device=dev) if Fs else None
    dY_s = torch.empty(T, d, dtype=ad, device=dev) if Fs else None
    torch.cuda.synchronize()

    def step(ev):
        i = 0

        def mark():
            nonlocal i
            if ev is not None:
                ev[i].record()
            i += 1

        mark()
        L.gate_logits(cfg, x, Wt["Wg"], Wt["bg"], S["logits"], ws)
        mark()
        L.router_topk(cfg, S["logits"], Wt["expert_bias"], S["idx"], S["w"], S["counts"], None, stats, ws)
        mark()
        L.permute(cfg, None if gather else x, S["idx"], S["offsets"], S["row_of"], S["token_of"], S.get("x_perm"), ws)
        mark()
        L.grouped_gemm_swiglu(cfg, S.get("x_perm"), S["offsets"], Wt["W13"], Wt["W2"], x if Fs or gather else None,
                              Wt["W13s"], Wt["W2s"], S["H"], S["Act"], S["Y_perm"], S.get("H_s"), S.get("Act_s"),
                              S.get("Y_s"), ws, token_of=tok)
        mark()
        L.unpermute_combine(cfg, S["Y_perm"], S["row_of"], S["w"], S.get("Y_s"), y)
        mark()
        L.unpermute_combine_bwd(cfg, dy, S["Y_perm"], S["row_of"], S["w"], dY_perm, dw, dY_s)
        mark()
        L.grouped_gemm_swiglu_bwd(cfg, S.get("x_perm"), S["offsets"], Wt["W13"], Wt["W2"], S["H"], S["Act"], dY_perm,
                                  dH, dX_perm, None, None, x if Fs else None, Wt["W13s"], Wt["W2s"],
                                  S.get("H_s"), S.get("Act_s"), dY_s, dH_s, dx_s, None, None, ws)
        mark()
        L.grouped_wgrad(cfg, S["offsets"], E, A, dY_perm, d, S["Act"], F, G["dW2"], ws=ws)
        mark()
        L.grouped_wgrad(cfg, S["offsets"], E, A, dH, 2 * F, X1, d, G["dW13"], x_rows=tok, ws=ws)
        mark()
        if Fs:
            L.grouped_wgrad(cfg, None, 1, T, dH_s, 2 * Fs, x, d, G["dW13s"], ws=ws)
            L.grouped_wgrad(cfg, None, 1, T, dY_s, d, S["Act_s"], Fs, G["dW2s"], ws=ws)
        mark()
        L.router_bwd(cfg, S["logits"], S["idx"], S["w"], dw, S["counts"], 1.0, dlogits)
        mark()
        L.gate_logits_bwd(cfg, x, Wt["Wg"], dlogits, G["dWg"], G.get("dbg"), dx_r, ws)
        mark()
        L.permute_bwd(cfg, dX_perm, S["row_of"], dx_s, dx_r, dx)
        mark()

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(PHASES) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    phase_ms = {p: float(np.mean([events[s][i].elapsed_time(events[s][i + 1]) for s in range(args.steps)]))
                for i, p in enumerate(PHASES)}
    ms_step = elapsed * 1e3 / args.steps
    st = stats.cpu().numpy()

    # the same layer through the two product entry points, moe_layer_fwd and moe_layer_bwd,
    # on one stream and with the expert weight gradients on a second stream of the caller
    layer_ms = {}
    if not args.no_entry_points:
        side = torch.cuda.Stream()

        def layer_step(ws2):
            L.layer_fwd(cfg, Wt, x, S, y, stats, ws)
            L.layer_bwd(cfg, Wt, S, x, dy, 1.0, dx, G, ws, wgrad_stream=ws2)

        for name, ws2 in (("one_stream", None), ("two_streams", side)):
            for _ in range(args.warmup):
                layer_step(ws2)
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            for _ in range(args.steps):
                layer_step(ws2)
            torch.cuda.synchronize()
            layer_ms[name] = (time.perf_counter() - t1) * 1e3 / args.steps

    wbf16 = cfg.wgrad_dtype == L.MOE_BF16
    alg = algorithmic(shape, 2 if wbf16 else 4)
    gemm_ms = sum(phase_ms[p] for p in GEMM_PHASES)
    gemm_tflops = alg["grouped_gemm_flop"] / (gemm_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if shape.act == "bf16" else PEAK_FP32_TFLOPS
    roof = roofline(alg, phase_ms[ROOFLINE_PHASE], peak, shape, "bf16" if wbf16 else "fp32")

    def hbm(p, key):
        """frac against the bytes of activation-dtype rows; where this library keeps fp32
        rows, the bytes it must move with them, their rate and their ratio beside it."""
        gbps = alg[key] / (phase_ms[p] * 1e-3) / 1e9
        out = dict(ms=round(phase_ms[p], 4), bytes=int(alg[key]), achieved_gbps=round(gbps, 1),
                   frac=round(gbps / PEAK_HBM_GBPS, 4))
        if key + "_storage" in alg:
            sb = alg[key + "_storage"]
            sg = sb / (phase_ms[p] * 1e-3) / 1e9
            out.update(bytes_fp32_storage=int(sb), storage_over_act_bytes=round(sb / alg[key], 3),
                       achieved_gbps_fp32_storage=round(sg, 1), frac_fp32_storage=round(sg / PEAK_HBM_GBPS, 4))
        return out

    layer_flop = alg["grouped_gemm_flop"] + alg["gate_flop"]
    out = dict(
        metric="MoE layer fwd+bwd tokens/s on 1 MI355X",
        value=round(T / (ms_step * 1e-3), 1),
        unit="tokens/s",
        n_gpus=1,
        steps=args.steps,
        warmup=args.warmup,
        ms_per_step=round(ms_step, 3),
        higher_is_better=True,
        scaling="weak",
        vs_baseline=None,
        dtype="bf16" if shape.act == "bf16" else "f32",
        data="synthetic (seeded generator, random-init weights)",
        config=dict(workload=shape.name, T=T, d=d, E=E, k=k, F=F, Fs=Fs, score=shape.score,
                    bias=shape.bias, aux_coeff=shape.aux_coeff, wgrad_dtype="bf16" if wbf16 else "f32",
                    fc1_rows="token rows of x through token_of (no grouped copy)" if gather else "grouped copy x_perm",
                    parallelism="single GPU"),
        roofline=roof,
        grouped_gemm=dict(kernels="every expert projection of fwd + bwd (routed and shared)",
                          flop_per_step=alg["grouped_gemm_flop"], ms_per_step=round(gemm_ms, 3),
                          tflops=round(gemm_tflops, 2), peak=peak, frac=round(gemm_tflops / peak, 4)),
        layer_tflops=round(layer_flop / (ms_step * 1e-3) / 1e12, 2),
        layer_entry_points=None if not layer_ms else {
            n: dict(calls="moe_layer_fwd + moe_layer_bwd" + (" (wgrad_stream)" if n == "two_streams" else ""),
                    ms_per_step=round(v, 3), tokens_per_s=round(T / (v * 1e-3), 1)) for n, v in layer_ms.items()},
        phases_ms={p: round(v, 4) for p, v in phase_ms.items()},
        hbm_phases=dict(router=hbm("router", "router_bytes"), permute=hbm("permute", "permute_bytes"),
                        combine=hbm("combine", "combine_bytes"), combine_bwd=hbm("combine_bwd", "combine_bwd_bytes"),
                        unpermute_reduce=hbm("unpermute_reduce", "unpermute_reduce_bytes")),
        gate_gemm=dict(ms=round(phase_ms["gate"] + phase_ms["gate_bwd"], 4), flop=alg["gate_flop"],
                       tflops=round(alg["gate_flop"] / ((phase_ms["gate"] + phase_ms["gate_bwd"]) * 1e-3) / 1e12, 2),
                       **gate_engine(shape)),
        load=dict(maxvio=round(float(st[1]), 4), empty_experts=int(st[2]), max_count=int(st[3]),
                  mean_count=T * k / E),
    )
    out["balancing"] = bench_balancing(args, shape, L, S, Wt["expert_bias"], dw, dlogits, dev)
    if wbf16:
        out["wgrad_f32"] = bench_wgrad_f32(args, shape, L, S, x, dY_perm, dH, dev, phase_ms, ws)
    if not args.no_cpu_baseline:
        tokens = args.cpu_tokens or {1: 128, 2: 8192, 3: 48, 4: 1024, 5: 256}[args.config]
        out["cpu_baseline"] = cpu_baseline(shape, inp, min(tokens, T))
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
