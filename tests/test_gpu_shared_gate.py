"""Parity of the shared expert's sigmoid gate (The Ultimate MoE Training Handbook, §3.4
Shared experts: the shared output times sigmoid(x Wsg)) against the fp64 oracle: the gate
kernel, the gated combine and its backward (dY_s = gs dy and the gate's logit gradient),
the gate's weight gradient, the rank-1 input gradient in the unpermute-reduce, and whole
layers with the gate (bf16 DeepSeek-V3- and Qwen3-Next-shaped reductions, fp32 tiny).
"""
from dataclasses import replace

import numpy as np
import pytest

from helpers import O, W, dev, f64, rel_err, storage_ok, to_dev, to_np, torch_mod
from test_gpu_layer import _check_layer

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("act,T,d,k", [("bf16", 300, 512, 4), ("f32", 77, 64, 2)])
def test_shared_gate_pieces(act, T, d, k):
    torch = torch_mod()
    from mixture_experts_layer_aux_amd import _lib as L
    E = 8
    rng = np.random.default_rng(T + d)
    cfg = L.make_config(T, d, E, k, 128, Fs=128, act=act, shared_gate=True)
    x_np = W.random_rows(T, d, seed=3, act=act)
    xo = f64(x_np, act)
    Wsg = (rng.standard_normal(d) / np.sqrt(d)).astype(np.float32)
    # the gate
    gs = torch.empty(T, dtype=torch.float32, device=dev())
    print(f"shared gate pieces act={act} T={T} d={d}", flush=True)
    L.shared_gate(cfg, to_dev(x_np), to_dev(Wsg), gs)
    torch.cuda.synchronize()
    gs_ref = O.sigmoid(xo @ Wsg.astype(np.float64))
    assert np.abs(to_np(gs) - gs_ref).max() < 1e-6
    # the gated combine and its backward, on a random permutation of the A rows
    A = T * k
    row_of = rng.permutation(A).reshape(T, k).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    Yp = rng.standard_normal((A, d)).astype(np.float32)
    Ys = rng.standard_normal((T, d)).astype(np.float32)
    dy = rng.standard_normal((T, d)).astype(np.float32)
    g32 = to_np(gs).astype(np.float32)
    y = torch.empty(T, d, dtype=torch.float32, device=dev())
    L.unpermute_combine(cfg, to_dev(Yp), to_dev(row_of), to_dev(w), to_dev(Ys), y, gs=to_dev(g32))
    dYp = torch.empty(A, d, dtype=L.act_dtype(cfg), device=dev())
    dw = torch.empty(T, k, dtype=torch.float32, device=dev())
    dYs = torch.empty(T, d, dtype=L.act_dtype(cfg), device=dev())
    dl = torch.empty(T, dtype=torch.float32, device=dev())
    L.unpermute_combine_bwd(cfg, to_dev(dy), to_dev(Yp), to_dev(row_of), to_dev(w), dYp, dw, dYs, gs=to_dev(g32),
                            Y_s=to_dev(Ys), dl_s=dl)
    torch.cuda.synchronize()
    g64 = g32.astype(np.float64)
    y_ref = np.einsum("tk,tkd->td", w.astype(np.float64), Yp.astype(np.float64)[row_of]) + g64[:, None] * Ys
    assert rel_err(to_np(y), y_ref) < 1e-5
    assert storage_ok(to_np(dYs), g64[:, None] * dy, act) <= 1.0
    dl_ref = g64 * (1 - g64) * np.sum(dy.astype(np.float64) * Ys, axis=1)
    assert rel_err(to_np(dl), dl_ref) < 1e-5
    # the gate's weight gradient and the rank-1 input gradient
    dWsg = torch.empty(d, dtype=torch.float32, device=dev())
    ws = L.alloc_workspace(cfg, dev())
    dl32 = to_np(dl).astype(np.float32)
    L.shared_gate_bwd(cfg, to_dev(x_np), to_dev(dl32), dWsg, ws)
    dXp = rng.standard_normal((A, d)).astype(np.float32)
    dx = torch.empty(T, d, dtype=torch.float32, device=dev())
    L.permute_bwd(cfg, to_dev(dXp), to_dev(row_of), None, None, dx, dl_s=to_dev(dl32), Wsg=to_dev(Wsg))
    torch.cuda.synchronize()
    assert rel_err(to_np(dWsg), dl32.astype(np.float64) @ xo) < 1e-5
    dx_ref = dXp.astype(np.float64)[row_of].sum(axis=1) + dl32.astype(np.float64)[:, None] * Wsg.astype(np.float64)
    assert rel_err(to_np(dx), dx_ref) < 1e-5


@pytest.mark.parametrize("name", ["deepseek_reduced", "qwen3_next_reduced", "tiny_fp32"])
def test_layer_with_shared_gate(name):
    shape = {"deepseek_reduced": replace(W.SMALL[3], shared_gate=True),
             "qwen3_next_reduced": replace(W.SMALL[4], shared_gate=True),
             "tiny_fp32": replace(W.LAYERS[1], Fs=128, shared_gate=True)}[name]
    print(f"shared gate layer {name}", flush=True)
    _check_layer(shape, seed=9)
