"""Parity of the router variants and the balancing step against the fp64 oracle, through
the C ABI: pre-softmax top-k, sqrt(softplus) scores, the aux loss on normalised sigmoid
scores, the router z-loss, the sequence-wise aux loss and the loss-free bias update.

Integer results (indices, counts, per-sequence counts) and the fp32 bias update are
bit-exact; the weights and losses are compared at fp32 accuracy; the router gradient of
the losses alone (dw = 0) at max |err| / rms <= 1e-4, the fp32 bar; the whole layer at the
layer's own bar.
"""
import zlib
from dataclasses import replace

import numpy as np
import pytest

from helpers import (MARGIN, O, W, check_router_grads, dev, f64, oracle_inputs, rel_err, routing_moved, spec_of, to_dev,
                     to_np, tol, torch_mod)

pytestmark = pytest.mark.gpu


def _lib():
    from mixture_experts_layer_aux_amd import _lib as L
    L.load()
    return L


# router-only cases: (name, shape, logits law, bias law)
_ROUTER_CASES = {
    "pre_softmax_top1": (W.LayerShape("r", T=1000, d=64, E=64, k=1, F=128, act="f32", pre_softmax=True,
                                      aux_coeff=0.01, z_coeff=1e-3, seq_aux_coeff=0.1, seq_len=250), "ties", None),
    "pre_softmax_k6_seq1": (W.LayerShape("r", T=333, d=64, E=300, k=6, F=128, act="f32", pre_softmax=True,
                                         scaling=2.5, z_coeff=0.01, seq_aux_coeff=0.2, seq_len=1), "normal", None),
    "sqrtsoftplus_bias": (W.LayerShape("r", T=1024, d=64, E=256, k=8, F=128, act="f32", score="sqrtsoftplus",
                                       aux_coeff=1e-3, z_coeff=1e-3, seq_aux_coeff=0.05, seq_len=128),
                          "ties", "ties"),
    "sqrtsoftplus_top1": (W.LayerShape("r", T=77, d=64, E=16, k=1, F=128, act="f32", score="sqrtsoftplus",
                                       aux_coeff=0.3), "normal", None),
    "sigmoid_deepseek_balancing": (W.LayerShape("r", T=1024, d=64, E=256, k=8, F=128, act="f32", score="sigmoid",
                                                aux_coeff=1e-3, z_coeff=1e-3, seq_aux_coeff=1e-4, seq_len=256),
                                   "normal", "normal"),
    "softmax_many_sequences": (W.LayerShape("r", T=2048, d=64, E=512, k=10, F=128, act="f32", z_coeff=1e-3,
                                            seq_aux_coeff=0.01, seq_len=64), "normal", None),
    # group-limited routing: DeepSeek-V3's 8 groups, 4 kept, with the selection bias; and
    # quantised logits whose group scores tie, so the lower group index decides
    "sigmoid_grouped_8x4": (W.LayerShape("r", T=1024, d=64, E=256, k=8, F=128, act="f32", score="sigmoid",
                                         num_groups=8, group_topk=4, seq_aux_coeff=1e-4, seq_len=256),
                            "normal", "normal"),
    "softmax_grouped_ties": (W.LayerShape("r", T=500, d=64, E=64, k=6, F=128, act="f32", num_groups=16,
                                          group_topk=3, aux_coeff=0.01), "ties", None),
}


def _case_inputs(name, shape):
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    _, law, blaw = _ROUTER_CASES[name]
    if law == "ties":   # quantised logits: many exact ties, so the lowest-index rule decides
        logits = (rng.integers(-6, 7, size=(shape.T, shape.E)) * 0.5).astype(np.float32)
    else:
        logits = (rng.standard_normal((shape.T, shape.E)) * 1.5).astype(np.float32)
    bias = None
    if blaw == "ties":
        bias = (rng.integers(-2, 3, size=shape.E) * 0.125).astype(np.float32)
    elif blaw == "normal":
        bias = (rng.standard_normal(shape.E) * 0.1).astype(np.float32)
    return logits, bias


def _route_gpu(shape, logits32, bias):
    torch = torch_mod()
    L = _lib()
    cfg = L.config_from_shape(shape)
    T, E, k = shape.T, shape.E, shape.k
    idx = torch.empty(T, k, dtype=torch.int32, device=dev())
    w = torch.empty(T, k, dtype=torch.float32, device=dev())
    counts = torch.empty(E, dtype=torch.int32, device=dev())
    ps = torch.empty(E, dtype=torch.float32, device=dev())
    stats = torch.full((L.MOE_NSTATS,), float("nan"), dtype=torch.float32, device=dev())
    B = L.num_sequences(cfg)
    sc = torch.empty(B, E, dtype=torch.int32, device=dev()) if B else None
    ws = L.alloc_workspace(cfg, dev())
    print(f"router case T={T} E={E} k={k} score={shape.score} seq_len={shape.seq_len}", flush=True)
    L.router_topk(cfg, to_dev(logits32), to_dev(bias), idx, w, counts, ps, stats, ws, seq_counts=sc)
    torch.cuda.synchronize()
    return cfg, dict(idx=to_np(idx), w=to_np(w), counts=to_np(counts), prob_sum=to_np(ps), stats=to_np(stats),
                     seq_counts=None if sc is None else to_np(sc))


@pytest.mark.parametrize("name", sorted(_ROUTER_CASES))
def test_router_variants_and_losses(name):
    shape = _ROUTER_CASES[name][0]
    logits, bias = _case_inputs(name, shape)
    _, g = _route_gpu(shape, logits, bias)
    spec = spec_of(shape)
    r = O.route(logits.astype(np.float64), spec, None if bias is None else bias.astype(np.float64))
    assert np.array_equal(g["idx"], r["idx"]), "top-k indices differ"
    assert np.array_equal(g["counts"], r["counts"]), "counts differ"
    np.testing.assert_allclose(g["w"], r["w"], rtol=2e-6, atol=1e-7)
    np.testing.assert_allclose(g["prob_sum"], r["prob_sum"], rtol=2e-5, atol=1e-5)
    st = g["stats"]
    assert st[0] == pytest.approx(r["aux"], rel=2e-5, abs=1e-12)
    assert st[1] == pytest.approx(r["maxvio"], rel=1e-5, abs=1e-6)
    assert st[4] == pytest.approx(r["z"], rel=2e-5, abs=1e-12)
    if shape.seq_aux_coeff:
        assert np.array_equal(g["seq_counts"], r["seq_counts"]), "per-sequence counts differ"
        assert st[5] == pytest.approx(r["seq_aux"], rel=2e-5)
    else:
        assert st[5] == 0.0


@pytest.mark.parametrize("name", sorted(_ROUTER_CASES))
def test_router_backward_of_variants_and_losses(name):
    torch = torch_mod()
    L = _lib()
    shape = _ROUTER_CASES[name][0]
    logits, bias = _case_inputs(name, shape)
    spec = spec_of(shape)
    r = O.route(logits.astype(np.float64), spec, None if bias is None else bias.astype(np.float64))
    cfg = L.config_from_shape(shape)
    T, E, k = shape.T, shape.E, shape.k
    w32 = r["w"].astype(np.float32)
    rng = np.random.default_rng(5)
    sc = None if r["seq_counts"] is None else to_dev(r["seq_counts"].astype(np.int32))
    for dw_law, daux in (("zero", 1.0), ("normal", 0.7), ("normal", 0.0)):
        dw = np.zeros((T, k), np.float32) if dw_law == "zero" else rng.standard_normal((T, k)).astype(np.float32)
        dl = torch.empty(T, E, dtype=torch.float32, device=dev())
        L.router_bwd(cfg, to_dev(logits), to_dev(r["idx"].astype(np.int32)), to_dev(w32), to_dev(dw),
                     to_dev(r["counts"].astype(np.int32)), daux, dl, seq_counts=sc)
        torch.cuda.synchronize()
        ref = O.router_backward(logits.astype(np.float64), r["idx"], w32.astype(np.float64), dw.astype(np.float64),
                                spec, counts=r["counts"], daux=daux, seq_counts=r["seq_counts"])
        got = to_np(dl)
        if not np.any(ref):
            assert not np.any(got)
            continue
        assert rel_err(got, ref) < 1e-4, (dw_law, daux, rel_err(got, ref))
        # the selected-set part is exactly zero off the selected experts when no loss acts
        if daux == 0.0 and not (shape.score == "softmax" and shape.pre_softmax):
            off = np.ones((T, E), bool)
            np.put_along_axis(off, r["idx"], False, axis=1)
            assert not np.any(got[off])


@pytest.mark.parametrize("E,centered,rate", [(256, False, 1e-3), (256, True, 1e-3), (7, False, 0.37),
                                             (7, True, 0.37), (2048, True, 3e-4), (1, False, 1e-3)])
def test_expert_bias_update_bit_exact(E, centered, rate):
    torch = torch_mod()
    L = _lib()
    rng = np.random.default_rng(E + int(centered))
    k = min(8, E)
    T = 4099
    counts = np.bincount(rng.choice(E, size=T * k, p=rng.dirichlet(np.ones(E))), minlength=E).astype(np.int64)
    if E >= 3:   # two empty experts, their share moved to a third
        counts[:2] = 0
        counts[2] += T * k - counts.sum()
    assert counts.sum() == T * k
    bias = (rng.standard_normal(E) * 0.3).astype(np.float32)
    cfg = L.make_config(T, 64, E, k, 128, act="f32", score="sigmoid")
    b = to_dev(bias.copy())
    L.expert_bias_update(cfg, to_dev(counts.astype(np.int32)), rate, centered, b)
    torch.cuda.synchronize()
    ref = O.expert_bias_update(bias, counts, rate, centered)
    assert np.array_equal(to_np(b).astype(np.float32).view(np.uint32), ref.view(np.uint32))
    # exact mean: unchanged (sign update) -- an integer mean with E | T k
    c2 = np.full(E, 3, np.int32)
    b2 = to_dev(bias.copy())
    L.expert_bias_update(cfg, to_dev(c2), rate, False, b2)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(b2), bias)


# whole layers with the variants and every balancing loss on; coefficients large enough
# that their gradients show at the layer's tolerance
_LAYER_CASES = {
    "sqrtsoftplus_all_losses": replace(W.SMALL[3], score="sqrtsoftplus", aux_coeff=0.05, z_coeff=0.02,
                                       seq_aux_coeff=0.3, seq_len=256),
    "pre_softmax_top1": replace(W.SMALL[2], k=1, pre_softmax=True, z_coeff=0.01, seq_aux_coeff=0.2, seq_len=128,
                                aux_coeff=0.05),
    "sigmoid_seq_aux_fp32": replace(W.LAYERS[1], score="sigmoid", aux_coeff=0.1, z_coeff=0.05, seq_aux_coeff=0.5,
                                    seq_len=32),
    "grouped_deepseek_reduced": replace(W.SMALL[3], num_groups=8, group_topk=4, seq_aux_coeff=0.2, seq_len=256),
}


@pytest.mark.parametrize("name", sorted(_LAYER_CASES))
def test_layer_with_variants_and_losses(name):
    torch = torch_mod()
    L = _lib()
    shape = _LAYER_CASES[name]
    inp = W.make_inputs(shape, seed=7)
    eb = inp["expert_bias"] if shape.score != "softmax" else None
    cfg = L.config_from_shape(shape)
    d = dev()
    Wt = dict(Wg=to_dev(inp["Wg"]), bg=to_dev(inp["bg"]), expert_bias=to_dev(eb),
              W13=to_dev(inp["W13"]), W2=to_dev(inp["W2"]), W13s=to_dev(inp["W13s"]), W2s=to_dev(inp["W2s"]))
    x = to_dev(inp["x"])
    dy = to_dev(W.to_f32(inp["dy"], shape.act).copy())
    S = L.alloc_saved(cfg, d)
    G = L.alloc_grads(cfg, d, with_dbg=inp["bg"] is not None)
    ws = L.alloc_workspace(cfg, d)
    y = torch.empty(shape.T, shape.d, dtype=torch.float32, device=d)
    dx = torch.empty(shape.T, shape.d, dtype=torch.float32, device=d)
    stats = torch.empty(L.MOE_NSTATS, dtype=torch.float32, device=d)
    print(f"layer case {name}", flush=True)
    L.layer_fwd(cfg, Wt, x, S, y, stats, ws)
    L.layer_bwd(cfg, Wt, S, x, dy, 1.0, dx, G, ws)
    torch.cuda.synchronize()
    o = oracle_inputs(inp, shape)
    spec = spec_of(shape)
    f = O.layer_forward(o["x"], o["Wg"], o["W13"], o["W2"], spec, bg=o["bg"],
                        expert_bias=None if eb is None else o["expert_bias"], W13s=o["W13s"], W2s=o["W2s"])
    b = O.layer_backward(f, o["x"], o["Wg"], o["W13"], o["W2"], o["dy"], spec, W13s=o["W13s"], W2s=o["W2s"],
                         daux=1.0)
    r = f["route"]
    tl = tol(shape)
    safe = r["margin"] > MARGIN
    moved = routing_moved(to_np(S["idx"]), r)
    assert rel_err(to_np(y), f["y"], safe) < tl, "y"
    if not moved.any():
        st = to_np(stats)
        assert st[0] == pytest.approx(r["aux"], rel=1e-4)
        assert st[4] == pytest.approx(r["z"], rel=1e-4)
        assert st[5] == pytest.approx(r["seq_aux"], rel=1e-4)
        assert np.array_equal(to_np(S["seq_counts"]), r["seq_counts"])
        # dx carries the router path (with every loss gradient) through the gate GEMM
        assert rel_err(to_np(dx), b["dx"], safe) < tl, "dx"
        check_router_grads({"dWg": to_np(G["dWg"])}, f, b, o, spec, o["W2"], shape)


# quantile balancing: (T, E, k, scores law, solve)
_QUANTILE_CASES = {
    "softmax_64x8": (2048, 64, 8, "softmax", True),
    "sigmoid_256x8_bias": (1024, 256, 8, "sigmoid", True),
    "ragged_12x2": (300, 12, 2, "softmax", True),
    "wide_896x16": (1792, 896, 16, "softmax", True),
    "route_only_odd_T": (333, 40, 3, "sigmoid", False),
}


@pytest.mark.parametrize("name", sorted(_QUANTILE_CASES))
def test_quantile_router_bit_exact(name):
    torch = torch_mod()
    L = _lib()
    T, E, k, law, solve = _QUANTILE_CASES[name]
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    logits = rng.standard_normal((T, E)) * 1.5 + np.linspace(-1.0, 1.0, E)[None, :]
    scores = (O.softmax_full(logits) if law == "softmax" else O.sigmoid(logits)).astype(np.float32)
    beta = (rng.standard_normal(E) * (0.01 if law == "softmax" else 0.1)).astype(np.float32)
    if name == "sigmoid_256x8_bias":   # scores and bias on a coarse grid: many exact ties
        scores = (np.round(scores * 16) / 16).astype(np.float32)
        beta = (np.round(beta * 32) / 32).astype(np.float32)
    cfg = L.make_config(T, 64, E, k, 128, act="f32", score="sigmoid" if law == "sigmoid" else "softmax")
    idx = torch.empty(T, k, dtype=torch.int32, device=dev())
    alpha = torch.empty(T, dtype=torch.float32, device=dev())
    bl = torch.full((E,), float("nan"), dtype=torch.float32, device=dev()) if solve else None
    ws = L.alloc_workspace(cfg, dev())
    print(f"quantile case {name}: T={T} E={E} k={k}", flush=True)
    L.router_quantile(cfg, to_dev(scores), to_dev(beta), idx, alpha, bl, ws)
    torch.cuda.synchronize()
    ridx, ralpha, rbl = O.quantile_route(scores, beta, k, update=solve)
    assert np.array_equal(to_np(idx), ridx), "selected experts differ"
    assert np.array_equal(to_np(alpha).astype(np.float32).view(np.uint32), ralpha.view(np.uint32)), "alpha differs"
    if solve:
        got = to_np(bl).astype(np.float32)
        assert np.all(got == rbl), "solved bias differs"


def test_quantile_bias_update_matches_oracle():
    torch = torch_mod()
    L = _lib()
    rng = np.random.default_rng(41)
    for E, ema in ((256, 0.9), (896, 0.0), (7, 1.0)):
        beta = (rng.standard_normal(E) * 0.1).astype(np.float32)
        local = (rng.standard_normal(E) * 0.1).astype(np.float32)
        cfg = L.make_config(64 * E, 64, E, 1, 128, act="f32", score="sigmoid")
        b = to_dev(beta.copy())
        L.quantile_bias_update(cfg, to_dev(local), ema, b)
        torch.cuda.synchronize()
        ref = O.quantile_bias_update(beta, local, ema)
        np.testing.assert_allclose(to_np(b), ref, rtol=1e-6, atol=2e-8)
        assert abs(to_np(b).mean()) < 1e-7


def test_full_size_deepseek_balancing_and_quantile():
    """The DeepSeek-V3-shaped layer at its real size (T=16384, E=256, k=8): the router with
    8 groups of which 4 are kept, the selection bias and the sequence-wise loss over 4
    sequences of 4096, and quantile balancing on the same logits; both sides get the same
    fp32 logits (and fp32 scores), so routing, counts, per-sequence counts, alpha and the
    solved bias are bit-exact."""
    torch = torch_mod()
    L = _lib()
    base = W.LAYERS[3]
    shape = replace(base, num_groups=8, group_topk=4, seq_aux_coeff=1e-4, seq_len=4096)
    inp = W.make_inputs(shape, seed=3, with_dy=False, with_experts=False)
    logits = O.gate_logits(f64(inp["x"], shape.act), inp["Wg"], inp["bg"]).astype(np.float32)
    _, g = _route_gpu(shape, logits, inp["expert_bias"])
    r = O.route(logits.astype(np.float64), spec_of(shape), inp["expert_bias"].astype(np.float64))
    assert np.array_equal(g["idx"], r["idx"])
    assert np.array_equal(g["counts"], r["counts"])
    assert np.array_equal(g["seq_counts"], r["seq_counts"])
    assert g["stats"][5] == pytest.approx(r["seq_aux"], rel=2e-5)
    # quantile balancing on the sigmoid scores of the same logits
    scores = (1.0 / (1.0 + np.exp(-logits.astype(np.float64)))).astype(np.float32)
    beta = (inp["expert_bias"] * np.float32(0.1)).astype(np.float32)
    cfg = L.config_from_shape(base)
    T, E, k = base.T, base.E, base.k
    idx = torch.empty(T, k, dtype=torch.int32, device=dev())
    alpha = torch.empty(T, dtype=torch.float32, device=dev())
    bl = torch.empty(E, dtype=torch.float32, device=dev())
    ws = L.alloc_workspace(cfg, dev())
    L.router_quantile(cfg, to_dev(scores), to_dev(beta), idx, alpha, bl, ws)
    torch.cuda.synchronize()
    ridx, ralpha, rbl = O.quantile_route(scores, beta, k)
    assert np.array_equal(to_np(idx), ridx)
    assert np.array_equal(to_np(alpha).astype(np.float32).view(np.uint32), ralpha.view(np.uint32))
    assert np.all(to_np(bl).astype(np.float32) == rbl)
